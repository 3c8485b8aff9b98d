"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only draws numbers. It holds none of the method's arithmetic: no
normalization, no scaling, no quantization. Values are drawn in float32 from
``numpy.random.default_rng(seed)`` and handed to torch's CPU cast to become
bfloat16 bit patterns (``uint16`` arrays); nothing here is shared with the HIP
path or with ``oracle/`` beyond these arrays.

Draw order inside one workload is fixed: x, then gamma, then beta, then group
counts, then the Hadamard sign mask. The shapes and distributions follow the
workloads the pages measure (DeepSeek-V3 style hidden sizes, per-token
activations, weight matrices and a grouped MoE activation tensor), as fixed by
the five named configurations below.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "to_bf16_bits",
    "quantize_only",
    "prefill",
    "decode",
    "weight_2d",
    "grouped_moe",
    "experts_2d",
    "qk_heads",
    "make",
    "NAMES",
    "SR_SEED",
    "SR_OFFSET",
]

SR_SEED = 0x5EED
SR_OFFSET = 0


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bfloat16 bit patterns (uint16) via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass
class Workload:
    name: str
    x: np.ndarray                      # uint16 bf16 bits [rows, cols]
    gamma: Optional[np.ndarray] = None  # uint16 bf16 bits [cols]
    beta: Optional[np.ndarray] = None   # uint16 bf16 bits [cols]
    eps: float = 1e-6
    weight_offset: float = 0.0
    rounding: str = "rtne"             # "rtne" | "sr"
    seed: int = SR_SEED
    offset: int = SR_OFFSET
    colwise: bool = False               # 2D: also produce the transposed plane
    rowwise: bool = True
    offsets: Optional[np.ndarray] = None  # int32 [G+1] for grouped inputs
    rht_mask: int = 0
    apply_rht: bool = False
    experts: int = 1                    # stacked weights (grouped 2D weights)
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return int(self.x.shape[0])

    @property
    def cols(self) -> int:
        return int(self.x.shape[1])


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def quantize_only(seed: int = 1, rows: int = 256, cols: int = 1024) -> Workload:
    """bf16 tensor ~N(0,1), rowwise quantize, round-to-nearest-even."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(_normal(rng, (rows, cols)))
    return Workload("quantize_256x1024" if (rows, cols) == (256, 1024) else f"quantize_{rows}x{cols}", x)


def prefill(seed: int = 2, tokens: int = 4096, hidden: int = 4096) -> Workload:
    """Prefill: x ~N(0,1), gamma = 1 + 0.1 N(0,1), no bias, eps 1e-6, RTNE rowwise."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(_normal(rng, (tokens, hidden)))
    gamma = to_bf16_bits(1.0 + 0.1 * _normal(rng, (hidden,)))
    return Workload(f"prefill_{tokens}x{hidden}", x, gamma=gamma, eps=1e-6)


def decode(seed: int = 3, tokens: int = 8, hidden: int = 7168) -> Workload:
    """Decode: x ~Student-t(3) (outlier heavy), gamma = 1 + 0.1 N, beta = 0.01 N, eps 1e-6."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(rng.standard_t(3, size=(tokens, hidden)).astype(np.float32))
    gamma = to_bf16_bits(1.0 + 0.1 * _normal(rng, (hidden,)))
    beta = to_bf16_bits(0.01 * _normal(rng, (hidden,)))
    return Workload(f"decode_{tokens}x{hidden}", x, gamma=gamma, beta=beta, eps=1e-6)


def weight_2d(seed: int = 4, rows: int = 8192, cols: int = 8192) -> Workload:
    """2D weight: W ~N(0, 0.02), rowwise + columnwise planes, stochastic rounding."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(_normal(rng, (rows, cols), std=0.02))
    return Workload(f"weight_{rows}x{cols}", x, rounding="sr", colwise=True)


def grouped_moe(seed: int = 5, tokens: int = 16384, hidden: int = 7168, groups: int = 64,
                apply_rht: bool = True, rounding: str = "sr") -> Workload:
    """Grouped MoE activations: x ~N(0,1), per-expert counts ~Multinomial(tokens, uniform)."""
    rng = np.random.default_rng(seed)
    x = to_bf16_bits(_normal(rng, (tokens, hidden)))
    counts = rng.multinomial(tokens, np.full(groups, 1.0 / groups))
    offsets = np.zeros(groups + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    mask = int(rng.integers(0, 1 << 16))
    return Workload(f"grouped_{tokens}x{hidden}_g{groups}", x, rounding=rounding, rowwise=False,
                    colwise=True, offsets=offsets, rht_mask=mask, apply_rht=apply_rht)


def experts_2d(seed: int = 6, experts: int = 4, rows: int = 4096, cols: int = 7168) -> Workload:
    """Grouped 2D weights: `experts` stacked [rows, cols] weights (a DeepSeek-V3 style gate/up projection
    of 2 x 2048 rows over hidden 7168, four local experts), expert e ~N(0, 0.02 s_e) with s_e drawn from
    U(0.5, 2) so that the experts' amax differ; stochastic rounding."""
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.5, 2.0, experts).astype(np.float32)
    x = np.concatenate([_normal(rng, (rows, cols), std=0.02) * s[e] for e in range(experts)])
    return Workload(f"experts_{experts}x{rows}x{cols}", to_bf16_bits(x), rounding="sr", colwise=True,
                    experts=experts)


def qk_heads(seed: int = 7, tokens: int = 4096, q_heads: int = 32, k_heads: int = 8, head_dim: int = 128) -> Workload:
    """QK norm: q [tokens, q_heads * head_dim] and k [tokens, k_heads * head_dim] (a Qwen3 style attention
    layer: 32 query and 8 key heads of 128), x ~N(0, 1) times a per-(token, head) factor exp(U(-2, 2)); weights
    1 + 0.1 N(0, 1), eps 1e-6. x holds q, gamma q's weight; meta holds k, k's weight and head_dim."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (tokens, q_heads, head_dim)) * np.exp(rng.uniform(-2, 2, (tokens, q_heads, 1))).astype(np.float32)
    k = _normal(rng, (tokens, k_heads, head_dim)) * np.exp(rng.uniform(-2, 2, (tokens, k_heads, 1))).astype(np.float32)
    wq = to_bf16_bits(1.0 + 0.1 * _normal(rng, (head_dim,)))
    wk = to_bf16_bits(1.0 + 0.1 * _normal(rng, (head_dim,)))
    return Workload(f"qknorm_{tokens}x{q_heads}+{k_heads}x{head_dim}", to_bf16_bits(q.reshape(tokens, -1)),
                    gamma=wq, eps=1e-6,
                    meta={"k": to_bf16_bits(k.reshape(tokens, -1)), "k_weight": wk, "head_dim": head_dim})


NAMES = {
    "quantize": quantize_only,
    "prefill": prefill,
    "decode": decode,
    "weight": weight_2d,
    "grouped": grouped_moe,
    "experts": experts_2d,
    "qknorm": qk_heads,
}


def make(name: str, **kw) -> Workload:
    return NAMES[name](**kw)

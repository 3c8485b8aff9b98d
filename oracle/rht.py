"""16-point random Hadamard transform applied ahead of columnwise quantization.

Test infrastructure only.

PR, Optimization item 2 and Fast math: the columnwise path multiplies each
16-element block by a Hadamard matrix with an fp32 accumulator and, in exact
mode, rounds that accumulator through bfloat16 before quantization; the
rowwise path has no transform. The pages do not fix the matrix ordering, the
normalization, where the random signs sit, or the summation order (their
accumulator is a tensor-core product). Reading R-rht fixes all four:

  t   = D x                       D = diag(d_0..d_15), d_i = -1 iff mask bit i
  FWHT: for h in 1, 2, 4, 8: for each i with (i & h) == 0:
        (t_i, t_{i+h}) <- (RN(t_i + t_{i+h}), RN(t_i - t_{i+h}))
  y   = bf16_RNE(RN(0.25 * t))

This is (1/4) H D x with H the 16x16 Sylvester Hadamard matrix; (1/4) H D is
orthogonal. The same D is used for every block of every group.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, f32_to_bf16

F32 = np.float32


def sign_vector(mask: int) -> np.ndarray:
    """Diagonal of D as float32 (+1 / -1) from a 16-bit mask."""
    return np.array([-1.0 if (int(mask) >> i) & 1 else 1.0 for i in range(16)], dtype=F32)


def rht16_f32(blocks, mask: int) -> np.ndarray:
    """Transform float32 blocks[..., 16]; returns RN(0.25 * FWHT(D x)) in float32 (before bf16)."""
    t = (np.asarray(blocks, dtype=F32) * sign_vector(mask)).astype(F32)
    t = t.copy()
    h = 1
    while h < 16:
        for i in range(16):
            if i & h:
                continue
            a = t[..., i].copy()
            b = t[..., i + h].copy()
            t[..., i] = (a + b).astype(F32)
            t[..., i + h] = (a - b).astype(F32)
        h *= 2
    return (t * F32(0.25)).astype(F32)


def rht16(blocks_bf16_bits, mask: int) -> np.ndarray:
    """bf16 bits [..., 16] -> bf16 bits [..., 16] of the transformed blocks."""
    return f32_to_bf16(rht16_f32(bf16_to_f32(blocks_bf16_bits), mask))

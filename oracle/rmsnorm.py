"""Per-token RMSNorm feeding the rowwise NVFP4 quantizer.

Test infrastructure only.

Blog, QK Norm: the squared norm is a horizontal sum over the row, the inverse
RMS is rsqrt(sum / n + EPS), and the output is ((w + WEIGHT_BIAS) * (x * rms))
cast back to the element type; WEIGHT_BIAS and EPS are compile-time
constants. The formula printed in that section's prose omits the square root;
the kernel code printed in the same section includes it and is followed here.

Readings: R-eps (eps is the float32 value the ABI carries), R-bias (the scalar
weight offset c of the Blog plus an optional per-channel additive beta), R-y
(the quantizer consumes the bfloat16-rounded output, so the tensor amax is
max |y_bf16|). The statistics are evaluated in float64 and y is rounded once
to bfloat16, so this is the exact value for any fp32 evaluation order.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, f64_to_bf16
from .quantize import quantize_rowwise


def _f64(a):
    """bf16 bits (uint16) or float16 / float32 values, as float64."""
    a = np.asarray(a)
    return bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def round_to(y64, dtype):
    """y rounded to nearest even in the output type: bf16 bits, or float16 / float32 values (reading R-dtype)."""
    if dtype == "bf16":
        return f64_to_bf16(y64)
    return np.asarray(y64, dtype=np.float64).astype(np.float16 if dtype == "fp16" else np.float32)


def rmsnorm_bf16(x, gamma, beta=None, weight_offset=0.0, eps=1e-6, return_f64=False, out_dtype="bf16"):
    """y = RN_T((gamma + c) * (x * r) [+ beta]),  r = 1 / sqrt(mean_k x^2 + eps), T = out_dtype.

    x, gamma, beta: bf16 bits, or float16 / float32 values (the input's type is the output's type;
    reading R-dtype). The default rounds to bfloat16, as the name says.
    """
    x64 = _f64(x)
    K = x64.shape[-1]
    g64 = _f64(gamma) + float(np.float32(weight_offset))
    eps64 = float(np.float32(eps))
    ms = np.sum(x64 * x64, axis=-1, keepdims=True) / K
    r = 1.0 / np.sqrt(ms + eps64)
    y64 = g64 * (x64 * r)
    if beta is not None:
        y64 = y64 + _f64(beta)
    y = round_to(y64, out_dtype)
    return (y, y64, r[..., 0]) if return_f64 else y


def rmsnorm_quantize(x, gamma, beta=None, weight_offset=0.0, eps=1e-6, amax=None,
                     rounding="rtne", seed=0, offset=0, out_dtype="bf16"):
    """Fused reference: RMSNorm to the input's type (bfloat16 by default), then rowwise NVFP4 of that tensor."""
    y = rmsnorm_bf16(x, gamma, beta, weight_offset, eps, out_dtype=out_dtype)
    q = quantize_rowwise(y, amax=amax, rounding=rounding, seed=seed, offset=offset, tag=0)
    q["y"] = y
    return q


def _kind(a):
    """Element type of an oracle array: bf16 bits (uint16), float16 or float32 values."""
    a = np.asarray(a)
    kinds = {np.dtype(np.uint16): "bf16", np.dtype(np.float16): "fp16", np.dtype(np.float32): "fp32"}
    assert a.dtype in kinds, "bf16 bits (uint16), float16 or float32 expected"
    return kinds[a.dtype]


def qk_norm(q, k, q_weight, k_weight, head_dim, weight_offset=0.0, eps=1e-6):
    """Per-head RMSNorm of the attention heads of q [T, Hq*D] and k [T, Hk*D] (reading R-qk).

    Blog, QK Norm: the norm is applied per head (64, 128 or 256 elements), each
    tensor with its own weight vector of head_dim entries, in place, through the
    same formula as above: y = (w + c) * (x * r), r = rsqrt(sum x^2 / D + EPS),
    cast back to the element type. This is rmsnorm_bf16 over rows of head_dim
    elements, rounded once to the input's type (Blog, Configuration space: the
    I/O type is a knob; reading R-dtype): q, k and the weights are bf16 bits
    (uint16), float16 or float32 values, all of one type. k may be None.
    """
    def one(x, w):
        x = np.asarray(x)
        kind = _kind(x)
        assert _kind(w) == kind, "the weight has the type of its tensor"
        T = x.shape[0]
        assert x.shape[1] % head_dim == 0
        return rmsnorm_bf16(x.reshape(-1, head_dim), w, None, weight_offset, eps, out_dtype=kind).reshape(T, -1)

    return one(q, q_weight), (None if k is None else one(k, k_weight))

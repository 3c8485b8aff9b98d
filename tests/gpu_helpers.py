"""Helpers shared by the GPU parity tests: host<->device moves and comparisons
against the oracle. Nothing here computes any step of the method."""
import numpy as np

import oracle
from oracle import formats as F


def to_dev(bits: np.ndarray):
    """uint16 bf16 bit array -> CUDA bfloat16 tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_np_bf16(t) -> np.ndarray:
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def np_u8(t, cols=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a if cols is None else a[:, :cols]


def f32(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32)


def assert_same_bits(name, got: np.ndarray, want: np.ndarray):
    if got.shape != want.shape:
        raise AssertionError(f"{name}: shape {got.shape} != {want.shape}")
    bad = np.argwhere(got != want)
    if len(bad):
        idx = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} of {got.size} differ; first at {idx}: got {got[idx]:#x} "
                             f"want {want[idx]:#x}")


def assert_f32_bits(name, got, want):
    g = np.float32(got).view(np.uint32)
    w = np.float32(want).view(np.uint32)
    assert g == w, f"{name}: {np.float32(got)!r} ({int(g):#x}) != {np.float32(want)!r} ({int(w):#x})"


def code_step_mismatch(got_packed: np.ndarray, want_packed: np.ndarray):
    """(number of differing codes, all differences are <= 1 magnitude step with the same sign)."""
    a = F.unpack_nibbles(got_packed).astype(np.int64)
    b = F.unpack_nibbles(want_packed).astype(np.int64)
    diff = a != b
    n = int(diff.sum())
    if n == 0:
        return 0, True
    ma, mb = a[diff] & 7, b[diff] & 7
    sa, sb = a[diff] >> 3, b[diff] >> 3
    same_sign = (sa == sb) | (ma == 0) | (mb == 0)
    ok = bool(np.all((np.abs(ma - mb) <= 1) & same_sign))
    return n, ok


# ---------------------------------------------------------------- rounded outputs of the norms
# Relative error bounds of the kernels' fp32 arithmetic for y = RN(RN(x * (w + c)) * r) [+ beta]: the sum of
# squares is a sum of positive fp32 terms whose longest dependency chain (per-lane accumulation plus the
# lane tree) has at most 134 additions for hidden <= 16384 (at most 13 for a head of <= 256), so its
# relative error is at most that many units of 2^-24; r = rsq(mean + eps) carries half of it plus the
# rounding of the mean, of + eps and v_rsq_f32's 1 ulp, and the two products one unit each. The bounds
# below (256 and 64 units) sit above those worst cases.
REL_ERR_RMSNORM = 2.0 ** -16
REL_ERR_QK = 2.0 ** -18
# Fraction of elements whose rounded output may differ from the oracle's: an element can differ only if
# its exact value lies within the relative error bound E of a rounding boundary of the output type, which
# covers at most 2E / (relative spacing of the type, at least 2^-8 for bf16 and 2^-11 for fp16) of the
# values; truncation in place of round-to-nearest-even would move about half of them.
MAX_DIFF_FRACTION = {"bf16": 2 * REL_ERR_RMSNORM / 2.0 ** -8, "fp16": 2 * REL_ERR_RMSNORM / 2.0 ** -11}


def out_values(a, out_dtype) -> np.ndarray:
    """Values of an output array (bf16 bits as uint16, or float16 / float32 values) as float64."""
    a = np.asarray(a)
    return F.bf16_to_f32(a).astype(np.float64) if out_dtype == "bf16" else a.astype(np.float64)


def _ordered(v, out_dtype) -> np.ndarray:
    """Monotone integer image of the output type's bit patterns (adjacent values differ by 1)."""
    if out_dtype == "bf16":
        b = np.asarray(v, np.uint16).astype(np.int64)
        sign, mag = b >> 15, b & 0x7FFF
    elif out_dtype == "fp16":
        b = np.asarray(v, np.float16).view(np.uint16).astype(np.int64)
        sign, mag = b >> 15, b & 0x7FFF
    else:
        b = np.asarray(v, np.float32).view(np.uint32).astype(np.int64)
        sign, mag = b >> 31, b & 0x7FFFFFFF
    return np.where(sign == 1, -mag, mag)


def assert_rounded_output(name, got, ref, y64, out_dtype, rel, beta64=None):
    """The norms' output against the exact value y64 (float64):

    * fp32 output: |got - y64| <= rel m (the arithmetic's own error; no further rounding);
    * bf16 / fp16 output: got is the round-to-nearest-even of some value within rel m of y64 (the set
      of such roundings is every value of the type between RN(y64 - rel m) and RN(y64 + rel m)), so it
      is within one step of the oracle's RN(y64) wherever that set holds at most two values (everywhere
      without a bias; with one, not where beta cancels the rest to far below its magnitude), and it
      differs from RN(y64) on at most MAX_DIFF_FRACTION of the elements.
    ref: the oracle's rounded output (its own RN(y64)); y64: the oracle's float64 value before rounding.
    m = |y64| without a bias; with an additive bias beta (y = t + beta, the bias added by one fused
    multiply-add) m = |t| + |beta|, since the error of t does not shrink when beta cancels it.
    Returns the number of elements that differ from the oracle's rounded value.
    """
    from oracle.rmsnorm import round_to

    y64 = np.asarray(y64, np.float64)
    m = np.abs(y64) if beta64 is None else np.abs(y64 - beta64) + np.abs(beta64)
    gv = out_values(got, out_dtype)
    if out_dtype == "fp32":
        err = np.abs(gv - y64)
        bad = err > rel * m
        assert not bad.any(), f"{name}: {int(bad.sum())} elements beyond {rel} relative; max {err.max()}"
        return int(np.sum(np.asarray(got, np.float32) != y64.astype(np.float32)))
    lo = out_values(round_to(y64 - rel * m, out_dtype), out_dtype)
    hi = out_values(round_to(y64 + rel * m, out_dtype), out_dtype)
    a, b = np.minimum(lo, hi), np.maximum(lo, hi)
    bad = (gv < a) | (gv > b)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{name}: {int(bad.sum())} elements are no rounding of a value within {rel} of the "
                             f"exact one; first at {i}: got {gv[i]!r}, exact {y64[i]!r}")
    steps = np.abs(_ordered(got, out_dtype) - _ordered(ref, out_dtype))
    # where the bound spans at most two values of the type (no cancellation against a bias), within one step
    span = np.abs(_ordered(round_to(y64 + rel * m, out_dtype), out_dtype)
                  - _ordered(round_to(y64 - rel * m, out_dtype), out_dtype))
    far = (span <= 1) & (steps > 1)
    assert not far.any(), f"{name}: an element is {steps[far].max()} steps from the oracle's"
    n = int(np.count_nonzero(steps))
    assert n <= MAX_DIFF_FRACTION[out_dtype] * steps.size, f"{name}: {n} of {steps.size} differ from the oracle"
    return n


def assert_code_diffs_follow_y(name, got_codes, ref_codes, y_got, y_ref, amax_got, amax_ref):
    """Every code that differs from the float64 oracle's lies in a 16-element block where the GPU's rounded
    y differs from the oracle's (or the tensor amax differs, which moves every scale): the code differences
    come from the normalization's rounding, not from the quantizer."""
    a = F.unpack_nibbles(got_codes) != F.unpack_nibbles(ref_codes)
    if not a.any():
        return
    if np.float32(amax_got) != np.float32(amax_ref):
        assert np.any(np.asarray(y_got) != np.asarray(y_ref)), f"{name}: amax differs with identical y"
        return
    rows = a.shape[0]
    cblk = a.reshape(rows, -1, 16).any(axis=-1)
    yblk = (np.asarray(y_got) != np.asarray(y_ref)).reshape(rows, -1, 16).any(axis=-1)
    bad = cblk & ~yblk
    assert not bad.any(), f"{name}: {int(bad.sum())} blocks have different codes but identical y"

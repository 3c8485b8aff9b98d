"""CPU checks of the GPU tests' comparison rules: a plain fp32 evaluation of the norm, rounded to nearest
even, passes them; the same values truncated (a wrong rounding mode) do not."""
import numpy as np
import pytest

import oracle
from oracle import formats as F
from tests.gpu_helpers import REL_ERR_RMSNORM, assert_code_diffs_follow_y, assert_rounded_output


def _fp32_norm(x, g, b):
    """y in fp32 the way a kernel evaluates it: a sequential fp32 sum of squares, r = 1/sqrt(mean + eps),
    RN(RN(x g) r) [+ b]."""
    x32, g32 = x.astype(np.float32), g.astype(np.float32)
    ss = np.cumsum(x32 * x32, axis=1, dtype=np.float32)[:, -1:]
    r = (np.float32(1) / np.sqrt(ss * np.float32(1.0 / x.shape[1]) + np.float32(1e-6))).astype(np.float32)
    y = ((x32 * g32).astype(np.float32) * r).astype(np.float32)
    return y if b is None else (y + b.astype(np.float32)).astype(np.float32)


def _truncate_bf16(y32):
    return (np.asarray(y32, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@pytest.mark.parametrize("bias", [False, True])
def test_rounding_rule_accepts_rne_and_rejects_truncation(bias):
    rng = np.random.default_rng(5 + bias)
    T, H = 64, 2048
    x = (rng.standard_normal((T, H)) * np.exp(rng.uniform(-3, 3, (T, 1)))).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    b = (0.01 * rng.standard_normal(H)).astype(np.float32) if bias else None
    for od in ("bf16", "fp16"):
        xi = F.f32_to_bf16(x) if od == "bf16" else x.astype(np.float16)
        gi = F.f32_to_bf16(g) if od == "bf16" else g.astype(np.float16)
        bi = None if b is None else (F.f32_to_bf16(b) if od == "bf16" else b.astype(np.float16))
        xv = F.bf16_to_f32(xi) if od == "bf16" else xi.astype(np.float32)
        gv = F.bf16_to_f32(gi) if od == "bf16" else gi.astype(np.float32)
        bv = None if bi is None else (F.bf16_to_f32(bi) if od == "bf16" else bi.astype(np.float32))
        y_ref, y64, _ = oracle.rmsnorm_bf16(xi, gi, bi, 0.0, 1e-6, return_f64=True, out_dtype=od)
        y32 = _fp32_norm(xv, gv, bv)
        b64 = None if bv is None else bv.astype(np.float64)[None, :]
        good = F.f32_to_bf16(y32) if od == "bf16" else y32.astype(np.float16)
        assert_rounded_output("rne", good, y_ref, y64, od, REL_ERR_RMSNORM, b64)
        if od == "bf16":
            bad = _truncate_bf16(y32)
        else:
            # fp16 toward zero: the nearest even value, stepped down by one where it lies above |y|
            h = y32.astype(np.float16)
            over = np.abs(h.astype(np.float32)) > np.abs(y32)
            bad = np.where(over, np.nextafter(h, np.float16(0)), h)
        with pytest.raises(AssertionError):
            assert_rounded_output("truncated", bad, y_ref, y64, od, REL_ERR_RMSNORM, b64)
    fp32_out = oracle.rmsnorm_bf16(x, g, b, 0.0, 1e-6, return_f64=True, out_dtype="fp32")
    assert_rounded_output("fp32", _fp32_norm(x, g, b), fp32_out[0], fp32_out[1], "fp32", REL_ERR_RMSNORM,
                          None if b is None else b.astype(np.float64)[None, :])


def test_code_difference_attribution():
    rng = np.random.default_rng(8)
    y = F.f32_to_bf16(rng.standard_normal((4, 64)).astype(np.float32))
    q = oracle.quantize_rowwise(y)
    assert_code_diffs_follow_y("same", q["codes"], q["codes"], y, y, q["amax"], q["amax"])
    codes = q["codes"].copy()
    codes[1, 9] ^= 0x01                    # a code changed in block (1, 1) while y is the same there
    with pytest.raises(AssertionError):
        assert_code_diffs_follow_y("planted", codes, q["codes"], y, y, q["amax"], q["amax"])
    y2 = y.copy()
    y2[1, 20] ^= 0x0001                    # y differs in that block: the difference is attributed to it
    assert_code_diffs_follow_y("explained", codes, q["codes"], y2, y, q["amax"], q["amax"])

"""GPU pins of the hardware conversions the kernels rely on, through the C ABI and against the oracle.

The quantizer uses gfx950's E2M1 conversion (round to nearest even, saturating, sign kept), its E4M3
conversion (round to nearest even on [0, 448], with a clamp for saturation), a corrected multiply for
RN(bmax / 6), and the bf16 / fp16 output roundings of the norms. These inputs put values exactly on, and
one unit in the last place either side of, every decision point of those conversions, so that a wrong
rounding mode, a lost sign, a flushed subnormal or an inexact division changes a code, a scale or a y.

Quantize calls take fp32 input (values as given, no bf16 step) and amax = 2688 * 2^k, which makes
S_enc = 2^-k and S_dec = 2^k exact: with k = 0 a block whose maximum is 6 has scale 1 and encode
multiplier 1, so its other elements reach the E2M1 conversion unchanged.
"""
import numpy as np
import pytest

import oracle
from oracle import formats as F
from tests.gpu_helpers import assert_f32_bits, assert_same_bits, f32, np_u8

pytestmark = pytest.mark.gpu

E2M1_MAG = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
E2M1_MID = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def _around(v):
    """v and its two fp32 neighbours."""
    v = np.float32(v)
    return [np.nextafter(v, np.float32(-np.inf)), v, np.nextafter(v, np.float32(np.inf))]


def _blocks_to_rows(blocks, per_row=16):
    """[n, 16] fp32 blocks -> [rows, per_row * 16] fp32, zero blocks appended to fill the last row."""
    b = np.asarray(blocks, np.float32)
    pad = (-len(b)) % per_row
    if pad:
        b = np.concatenate([b, np.zeros((pad, 16), np.float32)])
    return np.ascontiguousarray(b.reshape(-1, per_row * 16))


def _quantize_check(gpu_lib, x, amax):
    import torch

    a = torch.tensor([amax], dtype=torch.float32, device="cuda")
    got = gpu_lib.nvfp4q_quantize(torch.from_numpy(x).cuda(), amax=a)
    q = oracle.quantize_rowwise(x, amax=np.float32(amax))
    C = x.shape[1]
    assert_same_bits(f"codes (amax {amax})", np_u8(got["codes"], C // 2), q["codes"])
    assert_same_bits(f"scales (amax {amax})", np_u8(got["scales"], C // 16), q["scales"])
    assert_f32_bits("scale", f32(got["scale"])[0], q["s_dec"])
    return q


def test_e2m1_decision_points(gpu_lib):
    """Every E2M1 magnitude and midpoint, one ulp either side, both signs, signed zeros and fp32
    subnormals, encoded with multiplier 1 (block maximum 6, amax 2688); above 6 the conversion saturates."""
    vals = []
    for m in E2M1_MAG + E2M1_MID:
        for v in _around(m):
            if 0.0 <= v <= 6.0:
                vals += [v, -v]
    vals += [0.0, -0.0, 1e-45, -1e-45, 1e-40, -1e-40, 2.0 ** -126, -(2.0 ** -126), 2.0 ** -24, -(2.0 ** -24)]
    vals = np.array(vals, np.float32)
    n = -(-len(vals) // 15)
    blocks = np.zeros((n, 16), np.float32)
    blocks[:, 0] = 6.0                     # block maximum 6: scale code of 1.0, encode multiplier 1
    flat = np.zeros(n * 15, np.float32)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(n, 15)
    # saturation: maxima up to 6.37 still give scale 1 (RN(max / 6) lies below 1.0625, the E4M3 midpoint
    # above 1), so their elements reach the conversion above 6
    sat = np.zeros((4, 16), np.float32)
    for i, top in enumerate([np.float32(6.0), np.nextafter(np.float32(6.0), np.float32(7.0)),
                             np.float32(6.3), np.float32(6.37)]):
        sat[i, 0] = top
        sat[i, 1:] = np.linspace(-top, top, 15, dtype=np.float32)
    x = _blocks_to_rows(np.concatenate([blocks, sat]))
    q = _quantize_check(gpu_lib, x, 2688.0)
    assert np.all(q["scales"].reshape(-1)[:n + 4] == 0x38)   # every test block's scale is E4M3 1.0


def _scale_sweep(k):
    """Blocks whose maxima put RN(bmax / 6) * 2^-k at, and one ulp either side of, every E4M3 value and
    midpoint (bmax = 6 t 2^k, and its neighbours two ulps either side), plus maxima past the saturation."""
    vals = np.array([F.e4m3_decode(np.array([c]))[0] for c in range(127)], np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    targets = np.concatenate([vals[1:], mids])
    blocks = []
    for t in targets:
        b0 = np.float32(6.0 * t * 2.0 ** k)      # exact: t has at most 5 significant bits
        up1 = np.nextafter(b0, np.float32(np.inf))
        dn1 = np.nextafter(b0, np.float32(0))
        for b in (np.nextafter(dn1, np.float32(0)), dn1, b0, up1, np.nextafter(up1, np.float32(np.inf))):
            blk = np.zeros(16, np.float32)
            blk[0] = b
            blk[1:] = (np.float32(b) * np.linspace(-1.0, 1.0, 15)).astype(np.float32)
            blocks.append(blk)
    for b in (2688.0 * 2.0 ** k, 2700.0 * 2.0 ** k, 4000.0 * 2.0 ** k):   # scale 448 and saturation
        blk = np.zeros(16, np.float32)
        blk[0] = b
        blk[1:] = np.float32(b) * np.float32(0.25)
        blocks.append(blk)
    return _blocks_to_rows(np.array(blocks, np.float32))


@pytest.mark.parametrize("k", [0, -9, 7])
def test_e4m3_scale_decision_points(gpu_lib, k):
    """Scale codes at and around every E4M3 value and midpoint, subnormal codes included, and the 448
    saturation; with amax = 2688 * 2^k the division by 6 is the only rounding before the conversion."""
    _quantize_check(gpu_lib, _scale_sweep(k), 2688.0 * 2.0 ** k)


def test_div6_strided_exponent_sweep(gpu_lib):
    """The same decision points for amax = 2688 * 2^k over the exponent range in which S_enc = 2^-k is a
    normal float (k from -110 to 110 in steps of 4): RN(bmax / 6) is exercised at every binade of normal
    block maxima, where an inexact quotient moves a tie to the other side."""
    for k in range(-110, 111, 4):
        _quantize_check(gpu_lib, _scale_sweep(k), 2688.0 * 2.0 ** k)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_norm_output_rounding(gpu_lib, dtype):
    """The norm's output rounding on exactly known values: rows of constant magnitude 2 give a sum of
    squares of 4 H, mean 4 and r = 1/sqrt(4) = 1/2 (eps 0), so with weight offset 1 the output is
    RN_T(gamma + 1) with the sign of x, gamma + 1 being exact in fp32 (and the hidden size a power of two,
    so that the mean is exactly 4). gamma runs over every value of the type in [2^-16, 1) (bf16, 2048
    values) or [2^-8, 1) (fp16, 8192 values): among them are the exact midpoints of T in [1, 2) (ties,
    which go to the even neighbour) and their neighbours on either side."""
    import torch

    if dtype == "bf16":
        g = np.concatenate([(1.0 + np.arange(128) / 128.0) * 2.0 ** e for e in range(-16, 0)])
        gin = F.f32_to_bf16(g.astype(np.float32))
        assert np.array_equal(F.bf16_to_f32(gin).astype(np.float64), g)
    else:
        g = np.concatenate([(1.0 + np.arange(1024) / 1024.0) * 2.0 ** e for e in range(-8, 0)])
        gin = g.astype(np.float16)
        assert np.array_equal(gin.astype(np.float64), g)
    H = len(g)
    assert H & (H - 1) == 0
    x = np.full((2, H), 2.0, np.float32)
    x[1] *= -1.0
    xin = F.f32_to_bf16(x) if dtype == "bf16" else x.astype(np.float16)
    if dtype == "bf16":
        dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        dev = lambda a: torch.from_numpy(a).cuda()
    got = gpu_lib.rmsnorm_nvfp4q(dev(xin), dev(gin), weight_offset=1.0, eps=0.0, y_out=True)
    y_ref = oracle.rmsnorm_bf16(xin, gin, None, 1.0, 0.0, out_dtype=dtype)
    if dtype == "bf16":
        yg = got["y"].view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        yg = got["y"].cpu().numpy().view(np.uint16)
    assert_same_bits(f"y ({dtype})", yg, np.asarray(y_ref).view(np.uint16))
    # the sweep does hold ties of the output type (gamma + 1 exactly half-way between two values)
    ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -10
    assert np.any(np.mod(g, ulp) == ulp / 2)

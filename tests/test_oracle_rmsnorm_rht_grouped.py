"""Pins for the oracle's RMSNorm, Hadamard transform and grouped layout."""
import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from oracle import formats as F
from oracle import quantize as Q
from oracle.grouped import grouped_quantize, padded_offsets
from oracle.rht import rht16, rht16_f32, sign_vector
from oracle.rmsnorm import rmsnorm_bf16, rmsnorm_quantize


def _bits(a):
    return F.f32_to_bf16(np.asarray(a, dtype=np.float32))


# ---- RMSNorm ----

def test_rmsnorm_matches_torch_rms_norm_float64():
    rng = np.random.default_rng(20)
    x = _bits(rng.standard_normal((64, 4096)))
    g = _bits(1 + 0.1 * rng.standard_normal(4096))
    b = _bits(0.01 * rng.standard_normal(4096))
    eps = 1e-6
    y, y64, _ = rmsnorm_bf16(x, g, b, 0.0, eps, return_f64=True)
    xt = torch.from_numpy(F.bf16_to_f32(x).astype(np.float64))
    gt = torch.from_numpy(F.bf16_to_f32(g).astype(np.float64))
    ref = torch.nn.functional.rms_norm(xt, (4096,), gt, eps=float(np.float32(eps))).numpy()
    ref = ref + F.bf16_to_f32(b).astype(np.float64)
    assert np.allclose(y64, ref, rtol=1e-13, atol=1e-15)
    assert np.array_equal(y, F.f64_to_bf16(ref))


def test_rmsnorm_weight_offset_is_added_to_gamma():
    rng = np.random.default_rng(21)
    x = _bits(rng.standard_normal((4, 256)))
    g = _bits(0.1 * rng.standard_normal(256))
    _, a, _ = rmsnorm_bf16(x, g, None, 1.0, 1e-6, return_f64=True)
    g1 = F.bf16_to_f32(g).astype(np.float64) + 1.0
    _, b, _ = rmsnorm_bf16(x, _bits(np.ones(256)), None, 0.0, 1e-6, return_f64=True)
    assert np.allclose(a, b * g1, rtol=1e-14)


def test_rmsnorm_constant_row_closed_form():
    for c in (1.0, -3.0, 0.0078125, 100.0):
        x = _bits(np.full((1, 512), c))
        g = _bits(np.full(512, 1.5))
        eps = np.float32(1e-6)
        _, y64, _ = rmsnorm_bf16(x, g, None, 0.0, float(eps), return_f64=True)
        want = 1.5 * c / np.sqrt(c * c + float(eps))
        assert np.allclose(y64, want, rtol=1e-15)


def test_fused_amax_is_max_of_bf16_output():
    rng = np.random.default_rng(22)
    x = _bits(rng.standard_t(3, (8, 7168)))
    g = _bits(1 + 0.1 * rng.standard_normal(7168))
    b = _bits(0.01 * rng.standard_normal(7168))
    q = rmsnorm_quantize(x, g, b)
    assert q["amax"] == np.max(np.abs(F.bf16_to_f32(q["y"])))
    r = Q.quantize_rowwise(q["y"])
    assert np.array_equal(r["codes"], q["codes"]) and np.array_equal(r["scales"], q["scales"])


# ---- Hadamard transform ----

def test_rht_equals_sylvester_matrix_on_exact_inputs():
    # Small integers keep every partial sum exact in fp32, so the staged
    # butterflies must equal (1/4) H D x computed with scipy's Hadamard matrix.
    H = scipy.linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(23)
    for mask in (0, 0xFFFF, 0x1234, 0x8001, int(rng.integers(0, 1 << 16))):
        x = rng.integers(-64, 65, size=(200, 16)).astype(np.float32)
        d = sign_vector(mask).astype(np.float64)
        want = (x.astype(np.float64) * d) @ H.T / 4.0
        got = rht16_f32(x, mask).astype(np.float64)
        assert np.array_equal(got, want)


def test_rht_sign_bits_index_the_input_positions():
    # with x = e_i, the output is (1/4) * d_i * column i of H
    H = scipy.linalg.hadamard(16).astype(np.float64)
    for i in range(16):
        e = np.zeros((1, 16), np.float32)
        e[0, i] = 4.0
        assert np.array_equal(rht16_f32(e, 1 << i)[0], -H[:, i])
        assert np.array_equal(rht16_f32(e, 0)[0], H[:, i])


def test_rht_is_orthogonal_and_inverts():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((1000, 16)).astype(np.float32)
    mask = 0xA5C3
    y = rht16_f32(x, mask).astype(np.float64)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-6)
    H = scipy.linalg.hadamard(16).astype(np.float64)
    back = (y @ H.T / 4.0) * sign_vector(mask).astype(np.float64)
    assert np.allclose(back, x, rtol=0, atol=4e-6 * np.abs(x).max())


def test_rht_bf16_round_through():
    rng = np.random.default_rng(25)
    x = _bits(rng.standard_normal((100, 16)))
    y = rht16(x, 0x0F0F)
    assert np.array_equal(y, F.f32_to_bf16(rht16_f32(F.bf16_to_f32(x), 0x0F0F)))


# ---- grouped layout ----

def test_padded_offsets():
    off = np.array([0, 0, 5, 21, 21, 53], np.int32)
    assert padded_offsets(off).tolist() == [0, 0, 16, 32, 32, 64]


def test_grouped_single_group_without_rht_equals_colwise():
    rng = np.random.default_rng(26)
    x = _bits(rng.standard_normal((64, 32)))
    g = grouped_quantize(x, np.array([0, 64], np.int32), apply_rht=False, rounding="sr", seed=7, offset=3)
    c = Q.quantize_colwise(x, rounding="sr", seed=7, offset=3)
    assert np.array_equal(g["codes"], c["codes"]) and np.array_equal(g["scales"], c["scales"])
    assert g["amax"][0] == c["amax"]


def test_grouped_each_group_equals_its_zero_padded_slice():
    rng = np.random.default_rng(27)
    x = _bits(rng.standard_normal((70, 32)))
    off = np.array([0, 5, 5, 40, 70], np.int32)
    mask = 0x3C5A
    g = grouped_quantize(x, off, apply_rht=True, rht_mask=mask, rounding="rtne")
    poff = g["poff"]
    for k in range(4):
        n, pg = off[k + 1] - off[k], poff[k + 1] - poff[k]
        if pg == 0:
            assert g["amax"][k] == 0 and g["s_dec"][k] == 1
            continue
        z = np.zeros((pg, 32), np.uint16)
        z[:n] = x[off[k]:off[k + 1]]
        zt = rht16(np.ascontiguousarray(z.T).reshape(32, pg // 16, 16), mask).reshape(32, pg)
        r = Q.quantize_rowwise(zt)   # rowwise of the transposed slice
        assert np.array_equal(g["codes"][:, poff[k] // 2:(poff[k] + pg) // 2], r["codes"])
        assert np.array_equal(g["scales"][:, poff[k] // 16:(poff[k] + pg) // 16], r["scales"])
        assert g["amax"][k] == r["amax"]


# ---------------------------------------------------------------- R-fast (no bf16 round-through)
def test_fast_math_equals_exact_when_the_transform_is_bf16_exact():
    # Integer inputs in [-2, 2]: every transformed value is 0.25 * (a sum of 16 terms of magnitude <= 2),
    # a multiple of 0.25 below 8 in magnitude, hence exactly a bfloat16; dropping the round-through then
    # changes nothing.
    rng = np.random.default_rng(44)
    x = F.f32_to_bf16(rng.integers(-2, 3, size=(77, 64)).astype(np.float32))
    offsets = np.array([0, 5, 40, 77], np.int32)
    for rounding in ("rtne", "sr"):
        ex = grouped_quantize(x, offsets, apply_rht=True, rht_mask=0x5A3C, rounding=rounding, seed=3)
        fa = grouped_quantize(x, offsets, apply_rht=True, rht_mask=0x5A3C, rounding=rounding, seed=3,
                              fast_math=True)
        for k in ("codes", "scales", "amax", "s_dec"):
            assert np.array_equal(ex[k], fa[k]), k


def test_fast_math_codes_stay_within_one_step_of_exact():
    # On Gaussian data the fp32 and the bf16-rounded transform differ by at most half a bf16 ulp, so the
    # codes differ rarely and then by one magnitude step with the same sign; without the transform the
    # option changes nothing.
    rng = np.random.default_rng(45)
    x = F.f32_to_bf16(rng.standard_normal((200, 96)).astype(np.float32))
    offsets = np.array([0, 70, 130, 200], np.int32)
    ex = grouped_quantize(x, offsets, apply_rht=True, rht_mask=0x1234, rounding="rtne")
    fa = grouped_quantize(x, offsets, apply_rht=True, rht_mask=0x1234, rounding="rtne", fast_math=True)
    a = F.unpack_nibbles(ex["codes"]).astype(np.int16)
    b = F.unpack_nibbles(fa["codes"]).astype(np.int16)
    diff = a != b
    assert 0 < diff.mean() < 0.02
    assert np.all((a[diff] & 8) == (b[diff] & 8))                      # same sign
    assert np.all(np.abs((a[diff] & 7) - (b[diff] & 7)) == 1)          # one magnitude step
    plain = grouped_quantize(x, offsets, apply_rht=False, rounding="rtne")
    plain_f = grouped_quantize(x, offsets, apply_rht=False, rounding="rtne", fast_math=True)
    assert np.array_equal(plain["codes"], plain_f["codes"])


def _grouped_dequant(g):
    """Dequantized columnwise plane of a grouped result: [K, Mpad], each group under its own S_dec."""
    poff = g["poff"].astype(np.int64)
    out = []
    for k in range(len(poff) - 1):
        p0, p1 = int(poff[k]), int(poff[k + 1])
        if p1 > p0:
            out.append(Q.dequantize_rowwise(g["codes"][:, p0 // 2:p1 // 2], g["scales"][:, p0 // 16:p1 // 16],
                                            g["s_dec"][k]))
    return np.concatenate(out, axis=1)


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_fast_math_meets_the_sqnr_acceptance_floor(rounding):
    # The pages accept the fast path when its dequantized output keeps an SQNR of at least 25 dB against
    # the exact path's ([PR] Fast math: measured 30.4-31.9 dB on grouped inputs, about 1.2 % of code bytes
    # differing). Here, on a grouped workload shaped like the pages' (Gaussian tokens, multinomial group
    # sizes, the transform on), with the exact path as the signal and the difference as the noise.
    rng = np.random.default_rng(47)
    counts = rng.multinomial(2048, np.full(8, 1 / 8))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = F.f32_to_bf16(rng.standard_normal((2048, 384)).astype(np.float32))
    ex = grouped_quantize(x, offsets, apply_rht=True, rht_mask=0x9C35, rounding=rounding, seed=9, offset=2)
    fa = grouped_quantize(x, offsets, apply_rht=True, rht_mask=0x9C35, rounding=rounding, seed=9, offset=2,
                          fast_math=True)
    de, df = _grouped_dequant(ex), _grouped_dequant(fa)
    sqnr = 10 * np.log10(np.sum(de ** 2) / np.sum((df - de) ** 2))
    assert sqnr >= 25.0, sqnr
    assert np.mean(ex["codes"] != fa["codes"]) < 0.03   # 1.9 % here


# ---------------------------------------------------------------- R-rowcol (rowwise plane of the grouped input)
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_grouped_rowwise_single_group_is_the_rowwise_quantizer(rounding):
    rng = np.random.default_rng(46)
    x = F.f32_to_bf16((rng.standard_normal((53, 80)) * 2).astype(np.float32))
    ref = Q.quantize_rowwise(x, rounding=rounding, seed=11, offset=5)
    got = grouped_quantize(x, np.array([0, 53], np.int32), apply_rht=True, rht_mask=0x77, rounding=rounding,
                           seed=11, offset=5, rowwise=True)
    assert np.array_equal(got["row_codes"], ref["codes"]) and np.array_equal(got["row_scales"], ref["scales"])
    assert got["row_amax"][0] == ref["amax"] and got["row_s_dec"][0] == ref["s_dec"]


def test_grouped_rowwise_uses_each_groups_own_amax_and_ignores_the_transform():
    rng = np.random.default_rng(47)
    parts = [rng.standard_normal((9, 48)) * s for s in (1.0, 1e3, 1e-3)]
    x = F.f32_to_bf16(np.concatenate(parts).astype(np.float32))
    offsets = np.array([0, 9, 9, 18, 27], np.int32)                      # an empty group in the middle
    a = grouped_quantize(x, offsets, apply_rht=True, rht_mask=0x1, rounding="sr", seed=4, rowwise=True)
    b = grouped_quantize(x, offsets, apply_rht=False, rounding="sr", seed=4, rowwise=True)
    for k in ("row_codes", "row_scales", "row_amax", "row_s_dec"):
        assert np.array_equal(a[k], b[k]), k
    xf = F.bf16_to_f32(x)
    assert a["row_amax"][1] == 0 and a["row_s_dec"][1] == 1
    for g, (lo, hi) in enumerate(zip(offsets[:-1], offsets[1:])):
        if hi > lo:
            assert a["row_amax"][g] == np.max(np.abs(xf[lo:hi]))
            # a block holding its group's amax gets the saturating scale code 0x7E (448)
            r, c = np.unravel_index(np.argmax(np.abs(xf[lo:hi])), xf[lo:hi].shape)
            assert a["row_scales"][lo + r, c // 16] == 0x7E


# ---- QK norm (reading R-qk) ----

def test_qk_norm_hand_head():
    # One head of 64 with x = (3, 4, 0, ...): mean x^2 = 25/64, r = 8/5, so (3, 4) -> (4.8, 6.4), which
    # round to the bfloat16 values 4.8125 and 6.40625 (without the square root r would be 64/25 and the
    # outputs 7.68 and 10.24). The second head, x = 2 everywhere, gives 1 everywhere; with eps = 0 exactly.
    x = np.zeros((1, 128), np.float32)
    x[0, 0], x[0, 1] = 3.0, 4.0
    x[0, 64:] = 2.0
    w = _bits(np.ones(64))
    y, _ = oracle.qk_norm(_bits(x), None, w, None, 64, eps=0.0)
    yf = F.bf16_to_f32(y)[0]
    assert yf[0] == 4.8125 and yf[1] == 6.40625 and np.all(yf[2:64] == 0.0)
    assert np.all(yf[64:] == 1.0)


def test_qk_norm_hand_head_fp16_fp32():
    # The same heads in fp16 and fp32 (reading R-dtype: one rounding to the input's type). (3, 4) -> (4.8,
    # 6.4) exactly; 4.8 = 1.2 * 4 with 1.2 = 1.0011001100|1100...b, which rounds up to 1.0011001101b in
    # fp16's 10 fraction bits: 4.80078125 (truncation would give 4.796875); 6.4 = 1.1001100110|0110...b * 4
    # rounds down to 6.3984375. fp32 gives the nearest floats of 4.8 and 6.4. With k's weight 0.5 and
    # weight offset c = 1 the second head (x = 2, r = 1/2) becomes (0.5 + 1) * 1 = 1.5 in both types.
    for dt, e0, e1 in ((np.float16, 4.80078125, 6.3984375), (np.float32, float(np.float32(4.8)),
                                                              float(np.float32(6.4)))):
        x = np.zeros((1, 128), dt)
        x[0, 0], x[0, 1] = 3.0, 4.0
        x[0, 64:] = 2.0
        yq, yk = oracle.qk_norm(x, x, np.ones(64, dt), np.full(64, 0.5, dt), 64, eps=0.0)
        assert yq.dtype == dt and yk.dtype == dt
        assert float(yq[0, 0]) == e0 and float(yq[0, 1]) == e1 and np.all(yq[0, 2:64] == 0)
        assert np.all(yq[0, 64:] == 1.0)
        yq1, yk1 = oracle.qk_norm(x, x, np.ones(64, dt), np.full(64, 0.5, dt), 64, weight_offset=1.0, eps=0.0)
        assert np.all(yk1[0, 64:] == 1.5) and np.all(yq1[0, 64:] == 2.0)
    with pytest.raises(AssertionError):  # mixed types are not one of the library's configurations
        oracle.qk_norm(np.zeros((1, 64), np.float16), None, np.ones(64, np.float32), None, 64)


def test_qk_norm_is_per_head_and_per_tensor_weight():
    # Heads of very different sizes come out with unit RMS (weight 1, eps negligible), each head is
    # unchanged by scaling it by a power of two, and k uses its own weight.
    rng = np.random.default_rng(36)
    T, Hq, Hk, D = 6, 4, 2, 128
    scale = np.exp2(rng.integers(-12, 12, (T, Hq, 1))).astype(np.float32)
    q = _bits((rng.standard_normal((T, Hq, D)) * scale).reshape(T, Hq * D))
    k = _bits(rng.standard_normal((T, Hk * D)))
    ones = _bits(np.ones(D))
    kw = _bits(1.0 + 0.25 * rng.standard_normal(D))
    yq, yk = oracle.qk_norm(q, k, ones, kw, D, eps=1e-30)
    rms = np.sqrt(np.mean(F.bf16_to_f32(yq).astype(np.float64).reshape(T, Hq, D) ** 2, axis=-1))
    assert np.all(np.abs(rms - 1.0) < 2.0 ** -7)
    q2 = F.bf16_to_f32(q).reshape(T, Hq, D).copy()
    q2[:, 1] *= np.float32(2.0 ** 5)
    yq2, _ = oracle.qk_norm(_bits(q2.reshape(T, Hq * D)), None, ones, None, D, eps=1e-30)
    assert np.array_equal(yq2, yq)
    yk_plain, _ = oracle.qk_norm(k, None, ones, None, D, eps=1e-30)
    kw64 = F.bf16_to_f32(kw).astype(np.float64)
    unit = F.bf16_to_f32(yk_plain).astype(np.float64).reshape(T, Hk, D)
    expect = F.f64_to_bf16((kw64 * unit).reshape(T, -1))
    # k's weight applied per element of each head: within two bf16 roundings of w * (unit-weight output)
    diff = np.abs(F.bf16_to_f32(yk).astype(np.float64) - F.bf16_to_f32(expect).astype(np.float64))
    assert np.all(diff <= 2.0 ** -6 * np.abs(F.bf16_to_f32(expect)) + 1e-30)


def test_rmsnorm_fp16_fp32_output_rounding():
    # 16 columns x = (3, 4, 0, ...): mean x^2 = 25/16, r = 0.8, y = (2.4, 3.2, 0, ...) (eps 0). Rounded to
    # fp16 (10 fraction bits): 2.4 = 1.2 * 2 -> 1.0011001101b * 2 = 2.400390625, 3.2 = 1.6 * 2 ->
    # 1.1001100110b * 2 = 3.19921875; to fp32 the nearest floats of 2.4 and 3.2 (reading R-dtype).
    for dt, expect in ((np.float16, (2.400390625, 3.19921875)), (np.float32, (np.float32(2.4), np.float32(3.2)))):
        x = np.zeros((1, 16), dt)
        x[0, 0], x[0, 1] = 3.0, 4.0
        y = rmsnorm_bf16(x, np.ones(16, dt), None, 0.0, 0.0, out_dtype="fp16" if dt == np.float16 else "fp32")
        assert y.dtype == dt and float(y[0, 0]) == float(expect[0]) and float(y[0, 1]) == float(expect[1])
        assert np.all(y[0, 2:] == 0)
    # bf16-exact fp32 input with fp32 output: the float64 value rounded once to fp32, which keeps
    # digits the bf16 output rounds away
    rng = np.random.default_rng(41)
    xb = _bits(rng.standard_normal((4, 256)))
    gb = _bits(1 + 0.1 * rng.standard_normal(256))
    y32, y64, _ = rmsnorm_bf16(F.bf16_to_f32(xb), F.bf16_to_f32(gb), None, 0.0, 1e-6, return_f64=True,
                               out_dtype="fp32")
    assert np.array_equal(y32, y64.astype(np.float32))
    assert not np.array_equal(y32, F.bf16_to_f32(rmsnorm_bf16(xb, gb, None, 0.0, 1e-6)))


def test_grouped_round_through_follows_the_input_type():
    # One group of 16 tokens, column 0 = (1, 3 * 2^-11, 0, ...) along the tokens, no sign flips: every
    # transform output is 0.25 (1 +- 3 * 2^-11) = 0.25 +- 3 * 2^-13. The largest, 0.25 + 1.5 * 2^-12, is a
    # tie between two fp16 values and goes to the even one, 0.25 + 2^-11 = 0.25048828125; in bf16 (step
    # 2^-9 above 0.25) it rounds to 0.25; fp32 input takes no round-through: 0.2503662109375 (reading
    # R-dtype). The group amax shows which rounding ran.
    x = np.zeros((16, 16), np.float32)
    x[0, 0], x[1, 0] = 1.0, 3.0 * 2.0 ** -11
    offs = np.array([0, 16], np.int32)
    for xin, expect in ((x, 0.2503662109375), (x.astype(np.float16), 0.25048828125), (_bits(x), 0.25)):
        q = grouped_quantize(xin, offs, apply_rht=True, rht_mask=0, rounding="rtne")
        assert float(q["amax"][0]) == expect, (xin.dtype, float(q["amax"][0]))
    # fp32 input equals the bf16 path in fast-math mode on bf16-exact values (neither rounds the output)
    rng = np.random.default_rng(43)
    xb = _bits(rng.standard_normal((40, 32)))
    offs = np.array([0, 17, 40], np.int32)
    a = grouped_quantize(F.bf16_to_f32(xb), offs, apply_rht=True, rht_mask=0x35A9, rounding="sr", seed=3)
    b = grouped_quantize(xb, offs, apply_rht=True, rht_mask=0x35A9, rounding="sr", seed=3, fast_math=True)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


def test_grouped_ends_only_sampling_matches_the_full_call():
    # the sampling option of the grouped oracle computes the same bytes for the blocks it keeps, and the
    # same group amax (which still covers every block)
    rng = np.random.default_rng(3)
    counts = rng.multinomial(700, np.full(8, 1 / 8))
    counts[2], counts[5] = 0, 5
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = _bits(rng.standard_normal((int(off[-1]), 64)))
    for r in ("rtne", "sr"):
        full = grouped_quantize(x, off, True, 0x1234, rounding=r, seed=5, offset=1)
        ends = grouped_quantize(x, off, True, 0x1234, rounding=r, seed=5, offset=1, ends_only=True)
        assert np.array_equal(full["amax"], ends["amax"])
        poff = full["poff"]
        for g in range(8):
            a0, a1 = int(poff[g]), int(poff[g + 1])
            for t0 in ({a0, a1 - 16} if a1 > a0 else set()):
                assert np.array_equal(full["codes"][:, t0 // 2:t0 // 2 + 8], ends["codes"][:, t0 // 2:t0 // 2 + 8])
                assert np.array_equal(full["scales"][:, t0 // 16], ends["scales"][:, t0 // 16])

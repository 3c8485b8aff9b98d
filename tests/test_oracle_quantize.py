"""Pins for the oracle's quantizer: hand-derived blocks, closed forms, round trips,
error bounds, stochastic-rounding statistics and layout identities."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import formats as F
from oracle import quantize as Q
from oracle.philox import block_random_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")


def _bf16(vals):
    a = np.asarray(vals, dtype=np.float32)
    bits = F.f32_to_bf16(a)
    assert np.array_equal(F.bf16_to_f32(bits), a), "golden inputs must be exact bf16 values"
    return bits


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_hand_derived_blocks(case):
    x = _bf16(case["x"]).reshape(1, 16)
    q = Q.quantize_rowwise(x, amax=case["amax_in"])
    assert q["codes"].tolist()[0] == case["bytes"]
    assert F.unpack_nibbles(q["codes"]).tolist()[0] == case["codes4"]
    assert int(q["scales"][0, 0]) == case["scale"]
    assert int(np.float32(q["s_dec"]).view(np.uint32)) == case["s_dec_bits"]
    assert int(np.float32(q["s_enc"]).view(np.uint32)) == case["s_enc_bits"]


def test_power_of_two_global_scale_closed_form():
    for k in range(-20, 20):
        amax = np.float32(2688.0 * 2.0 ** k)
        s_enc, s_dec = Q.global_scales(amax)
        assert s_dec == np.float32(2.0 ** k) and s_enc == np.float32(2.0 ** -k)


def test_block_holding_the_amax_gets_scale_448():
    # RN(RN(amax/6) * RN(2688/amax)) is within a few ulps of 448 and rounds to it.
    rng = np.random.default_rng(5)
    amax = F.bf16_to_f32(F.f32_to_bf16(np.exp2(rng.uniform(-30, 30, 20000)).astype(np.float32)))
    s_enc, _ = Q.global_scales(amax)
    assert np.all(Q.block_scale_codes(amax, s_enc) == 0x7E)


def test_exact_round_trip_of_representable_blocks():
    # Blocks built as e2m1 * s * S_dec with a +-6 entry re-quantize to the same codes and scale.
    rng = np.random.default_rng(6)
    n = 4000
    codes = rng.integers(0, 16, size=(n, 16)).astype(np.uint8)
    codes[np.arange(n), rng.integers(0, 16, n)] = rng.choice([7, 15], n)   # one +-6 per block
    scodes = rng.integers(1, 0x7F, size=n).astype(np.uint8)
    for k in (-8, 0, 5):
        s_dec = np.float32(2.0 ** k)
        amax = np.float32(2688.0) * s_dec
        vals = F.e2m1_decode(codes) * F.e4m3_decode(scodes)[:, None] * s_dec
        x = F.f32_to_bf16(vals.astype(np.float32))
        assert np.array_equal(F.bf16_to_f32(x), vals.astype(np.float32))
        q = Q.quantize_rowwise(x.reshape(n, 16), amax=amax)
        got = F.unpack_nibbles(q["codes"])
        # -0 inputs are 0x8 codes that decode to -0.0: compare decoded values and signs
        assert np.array_equal(F.e2m1_decode(got), F.e2m1_decode(codes))
        assert np.array_equal(np.signbit(F.e2m1_decode(got)), np.signbit(vals))
        assert np.array_equal(q["scales"][:, 0], scodes)


def _dequant(q):
    return Q.dequantize_rowwise(q["codes"], q["scales"], q["s_dec"])


def test_rtne_error_bound_and_sqnr():
    rng = np.random.default_rng(7)
    x = F.f32_to_bf16(rng.standard_normal((512, 1024)).astype(np.float32))
    q = Q.quantize_rowwise(x)
    xf = F.bf16_to_f32(x).astype(np.float64)
    xh = _dequant(q)
    # per element: error <= half the local E2M1 gap times the block step (plus the
    # scale's own rounding); bound it by 1/4 of the block's max plus relative slack
    blk = np.abs(xf).reshape(512, 64, 16).max(-1)
    err = np.abs(xf - xh).reshape(512, 64, 16).max(-1)
    assert np.all(err <= blk * (1.0 / 6.0) * 1.07 + 1e-30)
    sqnr = 10 * np.log10(np.sum(xf ** 2) / np.sum((xf - xh) ** 2))
    assert sqnr >= 20.0  # PR, Correctness: round-to-nearest bar


def test_rowwise_equals_brute_force_nearest_in_block():
    # For each element, the chosen code minimizes |x*rcp - e2m1| (ties -> even code).
    rng = np.random.default_rng(8)
    x = F.f32_to_bf16((rng.standard_normal((64, 256)) * np.exp2(rng.integers(-10, 10, (64, 1)))).astype(np.float32))
    q = Q.quantize_rowwise(x)
    sc = q["scales"].repeat(16, axis=1)
    rcp = Q.encode_reciprocal(sc, q["s_dec"])
    v = (F.bf16_to_f32(x) * rcp).astype(np.float32).astype(np.float64)
    got = F.e2m1_decode(F.unpack_nibbles(q["codes"])).astype(np.float64)
    grid = np.concatenate([-F.E2M1_VALUES[::-1], F.E2M1_VALUES]).astype(np.float64)
    d = np.abs(np.minimum(np.abs(v), 6.0)[..., None] * np.sign(v)[..., None] - grid)
    assert np.all(np.abs(np.minimum(np.abs(v), 6.0) * np.sign(v) - got) <= d.min(-1) + 0.0)


def test_colwise_is_rowwise_of_transpose():
    rng = np.random.default_rng(9)
    x = F.f32_to_bf16(rng.standard_normal((64, 48)).astype(np.float32))
    d = Q.quantize_2d(x)
    r = Q.quantize_rowwise(np.ascontiguousarray(x.T), amax=d["amax"])
    assert np.array_equal(d["col"]["codes"], r["codes"]) and np.array_equal(d["col"]["scales"], r["scales"])
    assert d["row"]["s_dec"] == d["col"]["s_dec"]


# ---- stochastic rounding (reading R-sr) ----

def test_sr_mean_is_exact_over_all_random_bytes():
    # For each v, averaging the SR result over all 256 byte values gives
    # lo + gap * floor(256 frac) / 256 exactly (so the bias is below gap/256).
    rng = np.random.default_rng(10)
    v = np.concatenate([rng.uniform(0, 6.5, 3000), rng.uniform(0, 0.01, 200)]).astype(np.float32)
    r = np.arange(256)
    codes = Q.sr_round(np.repeat(v, 256), np.tile(r, len(v))).reshape(len(v), 256)
    mean = F.e2m1_decode(codes).astype(np.float64).mean(axis=1)
    a = np.minimum(v.astype(np.float64), 6.0)
    lo = np.array([F.E2M1_VALUES[F.E2M1_VALUES <= t].max() for t in a], dtype=np.float64)
    hi = np.array([F.E2M1_VALUES[F.E2M1_VALUES >= t].min() for t in a], dtype=np.float64)
    gap = np.where(hi > lo, hi - lo, 1.0)
    want = lo + gap * np.floor(256 * (a - lo) / gap) / 256
    assert np.allclose(mean, want, rtol=0, atol=1e-12)
    assert np.all(np.abs(mean - a) < gap / 256 + 1e-12)


def test_sr_exact_halfway_is_half_up():
    for lo, hi in [(0, .5), (.5, 1), (1, 1.5), (1.5, 2), (2, 3), (3, 4), (4, 6)]:
        mid = np.float32((lo + hi) / 2)
        c = Q.sr_round(np.full(256, mid), np.arange(256))
        up = F.e2m1_decode(c) == hi
        assert up.sum() == 128


def test_sr_halfway_statistics_on_philox_stream():
    # 2^20 exact-halfway values through the real block stream: |p - 1/2| <= 5 sigma.
    n_blk = 1 << 16
    rb = block_random_bytes(np.arange(n_blk, dtype=np.uint64), 0, 0x5EED, 0)
    v = np.full((n_blk, 16), 1.25, dtype=np.float32)
    c = Q.sr_round(v, rb)
    p = np.mean(F.e2m1_decode(c) == 1.5)
    assert abs(p - 0.5) <= 5 * 0.5 / np.sqrt(n_blk * 16)
    # no position in the block is biased either (a correlated stream would show here)
    per_pos = np.mean(F.e2m1_decode(c) == 1.5, axis=0)
    assert np.all(np.abs(per_pos - 0.5) <= 5 * 0.5 / np.sqrt(n_blk))


def test_sr_within_one_step_of_rtne_and_reproducible():
    rng = np.random.default_rng(11)
    x = F.f32_to_bf16(rng.standard_normal((128, 512)).astype(np.float32))
    a = Q.quantize_rowwise(x, rounding="rtne")
    s = Q.quantize_rowwise(x, rounding="sr", seed=0x5EED, offset=0)
    s2 = Q.quantize_rowwise(x, rounding="sr", seed=0x5EED, offset=0)
    s3 = Q.quantize_rowwise(x, rounding="sr", seed=0x5EED, offset=1)
    ca, cs = F.unpack_nibbles(a["codes"]), F.unpack_nibbles(s["codes"])
    assert np.all(np.abs((ca & 7).astype(int) - (cs & 7).astype(int)) <= 1)
    nz = ((ca & 7) != 0) & ((cs & 7) != 0)
    assert np.array_equal((ca & 8)[nz], (cs & 8)[nz])
    assert np.array_equal(a["scales"], s["scales"])         # scales stay round-to-nearest
    assert np.array_equal(s["codes"], s2["codes"])
    assert not np.array_equal(s["codes"], s3["codes"])
    xf = F.bf16_to_f32(x).astype(np.float64)
    sq = 10 * np.log10(np.sum(xf ** 2) / np.sum((xf - _dequant(s)) ** 2))
    assert sq >= 15.0   # PR, Correctness: SR reconstruction bar


def test_reciprocal_zero_and_clamp():
    assert Q.encode_reciprocal(np.array([0], np.uint8), np.float32(1.0))[0] == 0.0
    # tiny S_dec: 1/(2^-9 * S_dec) overflows; the multiplier is clamped to FLT_MAX
    r = Q.encode_reciprocal(np.array([1], np.uint8), np.float32(1e-38))[0]
    assert r == np.finfo(np.float32).max


def test_sampled_rows_keep_their_block_indices():
    rng = np.random.default_rng(12)
    x = F.f32_to_bf16(rng.standard_normal((64, 96)).astype(np.float32))
    full = Q.quantize_rowwise(x, rounding="sr", seed=5, offset=2)
    rows = np.array([3, 17, 40, 63])
    part = Q.quantize_rowwise(x[rows], amax=full["amax"], rounding="sr", seed=5, offset=2, row_ids=rows)
    assert np.array_equal(part["codes"], full["codes"][rows])
    cols = np.array([0, 5, 95])
    fc = Q.quantize_colwise(x, rounding="sr", seed=5, offset=2)
    pc = Q.quantize_colwise(x[:, cols], amax=fc["amax"], rounding="sr", seed=5, offset=2, col_ids=cols)
    assert np.array_equal(pc["codes"], fc["codes"][cols])


# ---------------------------------------------------------------- 16 x 16 tile scales (reading R-2dblk)
def test_2d_block_hand_tile():
    # amax 2688 gives S_enc = S_dec = 1. Tile (0, 0) holds 12 at (0, 0), 3 at (5, 3) and -0.5 at (9, 15):
    # tile max 12, RN(12 / 6) = 2 = E4M3 0x40, multiplier 0.5, so 12 -> 6 (code 7), 3 -> 1.5 (code 3) and
    # -0.5 -> -0.25, a tie between 0 and 0.5 that goes to the even code 0 with the sign kept (0x8). With
    # 1D blocks row 5 would take its own maximum 3 (scale 0.5 = 0x30, 3 -> 6, code 7). Tile (1, 1) holds
    # only 1 at (20, 17): RN(1 / 6) = 0.16666667 lies above the midpoint 0.1640625 of the E4M3 neighbours
    # 0.15625 and 0.171875, so its scale is 0.171875 = 0x23; RN(1 / 0.171875) = 5.818182 rounds to 6.
    x = np.zeros((32, 32), np.float32)
    x[0, 0], x[5, 3], x[9, 15], x[20, 17] = 12.0, 3.0, -0.5, 1.0
    q = Q.quantize_2d_block(_bf16(x), amax=np.float32(2688.0))
    assert q["tile_scales"].tolist() == [[0x40, 0], [0, 0x23]]
    rc, cc = F.unpack_nibbles(q["row"]["codes"]), F.unpack_nibbles(q["col"]["codes"])
    expect = np.zeros((32, 32), np.uint8)
    expect[0, 0], expect[5, 3], expect[9, 15], expect[20, 17] = 7, 3, 0x8, 7
    assert np.array_equal(rc, expect)
    assert np.array_equal(cc, expect.T)
    assert np.all(q["row"]["scales"][:16, 0] == 0x40) and np.all(q["row"]["scales"][16:, 1] == 0x23)
    assert np.all(q["col"]["scales"][:16, 0] == 0x40) and np.all(q["col"]["scales"][16:, 1] == 0x23)
    assert np.all(q["row"]["scales"][:16, 1] == 0) and np.all(q["col"]["scales"][16:, 0] == 0)
    one_d = Q.quantize_rowwise(_bf16(x), amax=np.float32(2688.0))
    assert int(one_d["scales"][5, 0]) == 0x30 and F.unpack_nibbles(one_d["codes"])[5, 3] == 7


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_2d_block_reduces_to_1d_blocks(rounding):
    # Rows repeated within each 16-row band: every tile maximum is each row block's maximum, so the
    # rowwise plane is the 1D rowwise quantization; columns repeated within each 16-column band give
    # the 1D columnwise plane. SR streams are those of the 1D planes (same tags and block indices).
    rng = np.random.default_rng(31)
    band = rng.standard_normal((3, 1, 80)).astype(np.float32) * np.float32(3.0)
    xr = F.f32_to_bf16(np.repeat(band, 16, axis=1).reshape(48, 80))
    q = Q.quantize_2d_block(xr, rounding=rounding, seed=77, offset=4)
    r1 = Q.quantize_rowwise(xr, rounding=rounding, seed=77, offset=4)
    assert np.array_equal(q["row"]["codes"], r1["codes"]) and np.array_equal(q["row"]["scales"], r1["scales"])
    cband = rng.standard_normal((48, 5, 1)).astype(np.float32)
    xc = F.f32_to_bf16(np.repeat(cband, 16, axis=2).reshape(48, 80))
    q = Q.quantize_2d_block(xc, rounding=rounding, seed=77, offset=4)
    c1 = Q.quantize_colwise(xc, rounding=rounding, seed=77, offset=4)
    assert np.array_equal(q["col"]["codes"], c1["codes"]) and np.array_equal(q["col"]["scales"], c1["scales"])


def test_2d_block_tile_scale_is_the_largest_1d_scale_and_rtne_planes_transpose():
    # The scale code is monotone in the block maximum, so a tile's code is the largest of the 1D codes of
    # its 16 row blocks and of its 16 column blocks; with RTNE the columnwise plane is the transpose of
    # the rowwise plane (same element, same scale). Distinct magnitudes per tile row and column make a
    # transposed or shifted tile index visible.
    rng = np.random.default_rng(32)
    x = rng.standard_normal((64, 96)).astype(np.float32) * np.exp(rng.uniform(-6, 6, (64, 1))).astype(np.float32)
    x *= np.exp(rng.uniform(-4, 4, (1, 96))).astype(np.float32)
    xb = F.f32_to_bf16(x)
    q = Q.quantize_2d_block(xb)
    r1, c1 = Q.quantize_rowwise(xb), Q.quantize_colwise(xb)
    assert np.array_equal(q["tile_scales"], r1["scales"].reshape(4, 16, 6).max(axis=1))
    assert np.array_equal(q["tile_scales"], c1["scales"].reshape(6, 16, 4).max(axis=1).T)
    assert np.array_equal(F.unpack_nibbles(q["col"]["codes"]), F.unpack_nibbles(q["row"]["codes"]).T)
    assert np.array_equal(q["col"]["scales"], np.repeat(q["tile_scales"].T, 16, axis=0))
    # and the dequantized planes agree exactly
    dr = Q.dequantize_rowwise(q["row"]["codes"], q["row"]["scales"], q["s_dec"])
    dc = Q.dequantize_rowwise(q["col"]["codes"], q["col"]["scales"], q["s_dec"])
    assert np.array_equal(dr, dc.T)


def test_2d_block_window_matches_the_full_tensor():
    # A 16-aligned window quantized on its own (with the full tensor's amax and origin) gives the window
    # of the full planes: the sampled checks of large tensors rely on it.
    rng = np.random.default_rng(33)
    x = F.f32_to_bf16(rng.standard_normal((96, 128)).astype(np.float32))
    full = Q.quantize_2d_block(x, rounding="sr", seed=9, offset=1)
    w = Q.quantize_2d_block(x[32:64, 48:112], amax=full["amax"], rounding="sr", seed=9, offset=1,
                            origin=(32, 48), full=(96, 128))
    rc, cc = F.unpack_nibbles(full["row"]["codes"]), F.unpack_nibbles(full["col"]["codes"])
    assert np.array_equal(F.unpack_nibbles(w["row"]["codes"]), rc[32:64, 48:112])
    assert np.array_equal(w["row"]["scales"], full["row"]["scales"][32:64, 3:7])
    assert np.array_equal(F.unpack_nibbles(w["col"]["codes"]), cc[48:112, 32:64])
    assert np.array_equal(w["col"]["scales"], full["col"]["scales"][48:112, 2:4])


# ---------------------------------------------------------------- grouped 2D weights (reading R-experts)
@pytest.mark.parametrize("tile16", [False, True])
def test_2d_experts_expert_zero_is_the_single_weight(tile16):
    rng = np.random.default_rng(34)
    x = F.f32_to_bf16(rng.standard_normal((3 * 48, 64)).astype(np.float32))
    q = Q.quantize_2d_experts(x, 3, rounding="sr", seed=5, offset=2, tile16=tile16)
    one = (Q.quantize_2d_block if tile16 else Q.quantize_2d)(x[:48], rounding="sr", seed=5, offset=2)
    assert np.array_equal(q["row"]["codes"][:48], one["row"]["codes"])
    assert np.array_equal(q["row"]["scales"][:48], one["row"]["scales"])
    assert np.array_equal(q["col"]["codes"][:64], one["col"]["codes"])
    assert np.array_equal(q["col"]["scales"][:64], one["col"]["scales"])
    assert q["amax"][0] == one["amax"]


def test_2d_experts_own_amax_and_own_streams():
    # Expert 1 is expert 0 times 2^-7: with its own amax every RTNE code and block scale is the same and
    # S_dec is 2^-7 times expert 0's (a shared amax would shift its block scales). With SR the two
    # experts' codes differ (tags 0/1 against 2/3) while their scales stay equal.
    rng = np.random.default_rng(35)
    x0 = rng.standard_normal((32, 48)).astype(np.float32)
    x = F.f32_to_bf16(np.concatenate([x0, x0 * np.float32(2.0 ** -7)]))
    q = Q.quantize_2d_experts(x, 2)
    for plane in ("row", "col"):
        h = q[plane]["codes"].shape[0] // 2
        assert np.array_equal(q[plane]["codes"][:h], q[plane]["codes"][h:])
        assert np.array_equal(q[plane]["scales"][:h], q[plane]["scales"][h:])
    assert q["s_dec"][1] == q["s_dec"][0] * np.float32(2.0 ** -7)
    s = Q.quantize_2d_experts(x, 2, rounding="sr", seed=8)
    assert not np.array_equal(s["row"]["codes"][:32], s["row"]["codes"][32:])
    assert np.array_equal(s["row"]["scales"][:32], s["row"]["scales"][32:])


# ---------------------------------------------------------------- fp16 / fp32 inputs
def test_fp16_fp32_inputs_are_quantized_as_given():
    # amax 2688 gives S_enc = S_dec = 1; the block max 6 gives scale 1 (E4M3 0x38) and multiplier 1.
    # 2.5 + 2^-20 (fp32) and 2.5 + 2^-9 (fp16) lie just above the E2M1 tie between 2 and 3 and encode
    # as 3 (code 5); rounded to bf16 first they would be the tie 2.5 itself, which goes to even (2, code 4).
    a = np.float32(2688.0)
    for dt, tiny in ((np.float32, 2.0 ** -20), (np.float16, 2.0 ** -9)):
        x = np.zeros((1, 16), dt)
        x[0, 0], x[0, 1] = 6.0, 2.5 + tiny
        assert float(x[0, 1]) != 2.5
        q = Q.quantize_rowwise(x, amax=a)
        c = F.unpack_nibbles(q["codes"])[0]
        assert int(q["scales"][0, 0]) == 0x38 and c[0] == 7 and c[1] == 5
        qb = Q.quantize_rowwise(F.f32_to_bf16(x.astype(np.float32)), amax=a)
        assert F.unpack_nibbles(qb["codes"])[0, 1] == 4
    # values that bf16 holds exactly quantize the same from any of the three types
    rng = np.random.default_rng(37)
    xb = F.f32_to_bf16(rng.standard_normal((8, 64)).astype(np.float32))
    ref = Q.quantize_rowwise(xb, rounding="sr", seed=3)
    for dt in (np.float32, np.float16):
        xf = F.bf16_to_f32(xb).astype(dt)
        if dt == np.float16:
            assert np.array_equal(xf.astype(np.float32), F.bf16_to_f32(xb))   # exact in fp16 too
        q = Q.quantize_rowwise(xf, rounding="sr", seed=3)
        assert np.array_equal(q["codes"], ref["codes"]) and np.array_equal(q["scales"], ref["scales"])

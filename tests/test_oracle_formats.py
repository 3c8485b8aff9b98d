"""Pins for the oracle's number formats against library routines and definitions.

Each check compares oracle/formats.py with something it does not share code
with: torch's CPU casts (bfloat16, float8_e4m3fn), exact float64 arithmetic,
or a brute-force nearest-value search written independently here.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F

ALL_BF16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _finite_bf16():
    f = F.bf16_to_f32(ALL_BF16)
    return ALL_BF16[np.isfinite(f)]


def test_bf16_widen_matches_torch_all_patterns():
    # Widening by a 16-bit shift (PR, Optimization item 6) equals torch's conversion.
    ours = F.bf16_to_f32(ALL_BF16).view(np.uint32)
    ref = torch.from_numpy(ALL_BF16.view(np.int16).copy()).view(torch.bfloat16).float().numpy().view(np.uint32)
    finite = np.isfinite(F.bf16_to_f32(ALL_BF16))
    assert np.array_equal(ours[finite], ref[finite])


def test_f32_to_bf16_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    # include exact ties: low half exactly 0x8000
    bits[:200_000] = (bits[:200_000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.38e38)]
    ours = F.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_single_rounding():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(500_000) * np.exp2(rng.integers(-140, 60, size=500_000))
    got = F.bf16_to_f32(F.f64_to_bf16(x)).astype(np.float64)
    # neighbours: truncate toward zero on the bf16 grid of |x|, then the next bf16 up
    a = np.abs(x)
    tr = (a.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    tr = np.where(tr > a, (((a.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)) - np.uint32(0x10000))
                           .view(np.float32).astype(np.float64)), tr)
    up = ((tr.astype(np.float32).view(np.uint32) + np.uint32(0x10000)).view(np.float32)).astype(np.float64)
    assert np.all((tr <= a) & (a <= up))
    d_lo, d_hi = a - tr, up - a
    lo_even = ((tr.astype(np.float32).view(np.uint32) >> 16) & 1) == 0
    want = np.where(d_lo < d_hi, tr, np.where(d_hi < d_lo, up, np.where(lo_even, tr, up)))
    assert np.array_equal(np.abs(got), want)
    assert np.array_equal(np.signbit(got), np.signbit(x))
    # on float32-exact inputs it agrees with torch's float32 -> bfloat16 cast
    xf = x.astype(np.float32)
    ref = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ok = np.abs(xf) < 3.38e38
    assert np.array_equal(F.f64_to_bf16(xf.astype(np.float64))[ok], ref[ok])


def test_e4m3_decode_matches_torch():
    codes = np.arange(0x7F, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(F.e4m3_decode(codes), ref)
    assert F.e4m3_decode(np.array([0x7E]))[0] == 448.0


def test_e4m3_encode_matches_torch_cast_of_clamped_value():
    # torch's float8_e4m3fn cast rounds to nearest even but does not saturate;
    # clamping to 448 first gives the saturating cast the oracle defines.
    s = np.concatenate([
        np.linspace(0, 500, 2_000_003, dtype=np.float32),
        np.exp2(np.linspace(-14, 9.2, 400_000)).astype(np.float32),
        (F.e4m3_decode(np.arange(1, 0x7F)).astype(np.float64)[:-1]
         + F.e4m3_decode(np.arange(2, 0x7F)).astype(np.float64)).astype(np.float32) / 2,  # midpoints
        np.array([0.0, 448.0, 464.0, 479.9, 480.0, 1e30, np.inf], dtype=np.float32),
    ])
    ours = F.e4m3_encode(s)
    ref = torch.from_numpy(np.minimum(s, 448.0).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def _e2m1_brute(v):
    """Nearest signed E2M1 value by exhaustive search, ties to the even code, saturating."""
    vals = F.E2M1_VALUES.astype(np.float64)
    a = np.minimum(np.abs(v.astype(np.float64)), 6.0)
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    mag = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (mag | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_value_set():
    # The element grid: {0, 0.5, 1, 1.5, 2, 3, 4, 6} and their negatives.
    assert sorted(set(np.abs(F.e2m1_decode(np.arange(16, dtype=np.uint8))).tolist())) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    # every representable value encodes to itself
    vals = F.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert np.array_equal(F.e2m1_encode(vals), np.arange(16, dtype=np.uint8))


def test_e2m1_encode_brute_force_all_bf16():
    x = F.bf16_to_f32(_finite_bf16())
    for scale in (1.0, 0.75, 3.0, 1 / 48.0, 2.0 ** -7):
        v = (x * np.float32(scale)).astype(np.float32)
        assert np.array_equal(F.e2m1_encode(v), _e2m1_brute(v))


def test_e2m1_encode_dense_fp32_sweep():
    # every float32 in [2^-3, 2^3) at a stride of 37 ulps, plus ties and their neighbours
    base = np.arange(np.float32(0.125).view(np.uint32), np.float32(8.0).view(np.uint32), 37, dtype=np.uint32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32).view(np.uint32)
    near = (mids[:, None] + np.arange(-3, 4, dtype=np.int64)[None, :]).astype(np.uint32).ravel()
    v = np.concatenate([base, near]).view(np.float32)
    v = np.concatenate([v, -v, np.array([0.0, -0.0, 1e-40, -1e-40, 7.0, 1e30, -1e30], np.float32)])
    assert np.array_equal(F.e2m1_encode(v), _e2m1_brute(v))


def test_e2m1_sign_of_zero_and_small_negatives():
    assert F.e2m1_encode(np.array([-0.0], np.float32))[0] == 0x8
    assert F.e2m1_encode(np.array([-0.2], np.float32))[0] == 0x8
    assert F.e2m1_encode(np.array([0.0], np.float32))[0] == 0x0


def test_nibble_order_hand_example():
    # element 0 -> low nibble, element 1 -> high nibble
    assert F.pack_nibbles(np.array([0x1, 0x2], np.uint8))[0] == 0x21
    c = np.random.default_rng(2).integers(0, 16, size=(7, 64)).astype(np.uint8)
    assert np.array_equal(F.unpack_nibbles(F.pack_nibbles(c)), c)

"""NVFP4 block quantization: global scale, block scale, encode, SR, pack.

Test infrastructure only. Each float step is one binary32 operation on
``numpy.float32`` values, in the order the steps are listed here.

Per tensor (or per group):
  amax  = max |x|                                 (exact; bf16 values)
  S_enc = RN(2688 / amax),  S_dec = RN(amax / 2688)           reading R-scale
Per block of 16 values:
  bmax  = max |x_i|
  s     = E4M3_rne_sat(RN(RN(bmax / 6) * S_enc))              reading R-bscale
  rcp   = RN(1 / RN(f32(s) * S_dec))   (0 if s == 0)          reading R-rcp
  v_i   = RN(x_i * rcp)
  code_i = E2M1_rne_sat(v_i)  or  SR(v_i, r_i)                R-e2m1 / R-sr

Sources: PR, Fast math (the encode reciprocal is the correctly rounded
reciprocal of the decoded FP8 block scale times the global decode scale, and
the exact path uses a correctly rounded division); PR, Optimization item 1
(eight bf16-origin values are multiplied by the reciprocal and converted);
Blog, Blackwell support (NVFP4 takes its amax over 16 elements). The 2688 is
6 * 448, the largest E2M1 magnitude times the largest E4M3 value, so the
per-tensor scale is amax / (6 * 448).
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, e2m1_encode, e2m1_decode, e4m3_decode, e4m3_encode, pack_nibbles, unpack_nibbles
from .formats import E2M1_VALUES
from .philox import block_random_bytes

F32 = np.float32
_FLT_MAX = np.finfo(np.float32).max
BLOCK = 16


def global_scales(amax):
    """amax (float32, any shape) -> (S_enc, S_dec) float32 arrays. Reading R-scale."""
    amax = np.asarray(amax, dtype=F32)
    with np.errstate(divide="ignore", over="ignore"):
        s_enc = F32(2688.0) / amax
        s_dec = amax / F32(2688.0)
    bad = (amax == 0) | ~np.isfinite(s_enc)
    s_enc = np.where(bad, F32(1.0), s_enc).astype(F32)
    s_dec = np.where(bad, F32(1.0), s_dec).astype(F32)
    return s_enc, s_dec


def block_scale_codes(bmax, s_enc):
    """Block amax (float32) and S_enc -> E4M3 scale codes. Reading R-bscale: divide by 6 first."""
    bmax = np.asarray(bmax, dtype=F32)
    q = bmax / F32(6.0)
    with np.errstate(over="ignore"):
        s = (q * np.asarray(s_enc, dtype=F32)).astype(F32)
    return e4m3_encode(s)


def encode_reciprocal(scodes, s_dec):
    """Scale codes and S_dec -> encode multiplier. Reading R-rcp."""
    p = (e4m3_decode(scodes) * np.asarray(s_dec, dtype=F32)).astype(F32)
    with np.errstate(divide="ignore", over="ignore"):
        r = F32(1.0) / p
    r = np.minimum(r, F32(_FLT_MAX))
    return np.where(np.asarray(scodes) == 0, F32(0.0), r).astype(F32)


def sr_round(v, rbytes):
    """Stochastic rounding of float32 v onto the signed E2M1 grid, given one random byte each.

    Reading R-sr. |v| is clamped to 6; lo <= |v| < hi are the neighbouring
    magnitudes; frac = (|v| - lo) / (hi - lo) is exact (the gap is a power of
    two and the subtraction is exact by Sterbenz's lemma); the value moves up
    to hi iff r + floor(256 * frac) >= 256, so it moves up with probability
    floor(256 * frac) / 256. Sign as in round-to-nearest (R-e2m1).
    PR, Correctness and Optimization item 3: one random draw per block, and SR
    codes stay within one magnitude step of the round-to-nearest code.
    """
    v = np.asarray(v, dtype=F32)
    r = np.asarray(rbytes, dtype=np.int64)
    a = np.minimum(np.abs(v), F32(6.0))
    lo_i = np.searchsorted(E2M1_VALUES, a, side="right") - 1       # largest value <= a
    lo_i = np.clip(lo_i, 0, 7)
    hi_i = np.minimum(lo_i + 1, 7)
    lo = E2M1_VALUES[lo_i]
    hi = E2M1_VALUES[hi_i]
    gap = np.where(hi_i == lo_i, F32(1.0), hi - lo).astype(F32)
    frac = ((a - lo) / gap).astype(F32)
    t = np.floor(frac * F32(256.0)).astype(np.int64)
    up = (r + t >= 256) & (hi_i != lo_i)
    mag = np.where(up, hi_i, lo_i).astype(np.uint8)
    sign = np.signbit(v).astype(np.uint8) << np.uint8(3)
    return (mag | sign).astype(np.uint8)


def quantize_blocks(xb, s_enc, s_dec, rounding="rtne", rbytes=None):
    """Quantize float32 blocks xb[..., 16] with per-leading-index S_enc/S_dec.

    Returns (codes[..., 16] 4-bit, scale codes[...]).
    """
    xb = np.asarray(xb, dtype=F32)
    assert xb.shape[-1] == BLOCK
    bmax = np.max(np.abs(xb), axis=-1)
    sc = block_scale_codes(bmax, s_enc)
    return encode_blocks(xb, sc, s_dec, rounding, rbytes), sc


def encode_blocks(xb, sc, s_dec, rounding="rtne", rbytes=None):
    """Codes of float32 blocks xb[..., 16] under given scale codes sc[...] (R-rcp, R-e2m1 / R-sr)."""
    xb = np.asarray(xb, dtype=F32)
    rcp = encode_reciprocal(sc, s_dec)
    with np.errstate(over="ignore"):
        v = (xb * rcp[..., None]).astype(F32)
    if rounding == "rtne":
        codes = e2m1_encode(v)
    elif rounding == "sr":
        assert rbytes is not None and rbytes.shape == xb.shape
        codes = sr_round(v, rbytes)
    else:
        raise ValueError(rounding)
    return codes


def _as_f32(x_bits_or_f32):
    a = np.asarray(x_bits_or_f32)
    return bf16_to_f32(a) if a.dtype == np.uint16 else a.astype(F32)


def _amax(xf):
    return F32(np.max(np.abs(xf))) if xf.size else F32(0.0)


def quantize_rowwise(x, amax=None, rounding="rtne", seed=0, offset=0, tag=0, row_ids=None):
    """Rowwise NVFP4 of x[M, K]: bf16 bits (uint16), or float16 / float32 values taken as they are.

    Blocks are 16 consecutive elements of a row. Reading R-blk: the SR block
    index is row * (K/16) + kb. Returns a dict with codes [M, K/2] (packed),
    scales [M, K/16] (E4M3 codes), amax, s_enc, s_dec.

    row_ids (sampling only): when x holds selected rows of a larger tensor, their
    row indices in that tensor, so SR block indices stay those of the full tensor;
    amax must then be given.
    """
    xf = _as_f32(x)
    M, K = xf.shape
    assert K % BLOCK == 0
    assert row_ids is None or amax is not None, "a sampled quantization needs the full tensor's amax"
    a = _amax(xf) if amax is None else F32(amax)
    s_enc, s_dec = global_scales(a)
    xb = xf.reshape(M, K // BLOCK, BLOCK)
    rb = None
    if rounding == "sr":
        rid = np.arange(M, dtype=np.uint64) if row_ids is None else np.asarray(row_ids, dtype=np.uint64)
        blk = rid[:, None] * np.uint64(K // BLOCK) + np.arange(K // BLOCK, dtype=np.uint64)[None, :]
        rb = block_random_bytes(blk, tag, seed, offset)
    codes, sc = quantize_blocks(xb, s_enc, s_dec, rounding, rb)
    return {
        "codes": pack_nibbles(codes.reshape(M, K)),
        "scales": sc.reshape(M, K // BLOCK),
        "amax": F32(a),
        "s_enc": F32(s_enc),
        "s_dec": F32(s_dec),
    }


def quantize_colwise(x, amax=None, rounding="rtne", seed=0, offset=0, col_ids=None, tag=1):
    """Columnwise (transposed) NVFP4 of x[M, K]; reading R-col.

    Blocks are 16 consecutive rows of one column; the output plane is the
    rowwise quantization of x transposed: codes [K, M/2], scales [K, M/16].
    Reading R-blk/R-philox: SR block index col * (M/16) + mb, tag 1.
    col_ids (sampling only): x holds selected columns of a larger tensor.
    """
    xf = _as_f32(x)
    M, K = xf.shape
    assert M % BLOCK == 0
    a = _amax(xf) if amax is None else F32(amax)
    return quantize_rowwise(np.ascontiguousarray(xf.T), amax=a, rounding=rounding, seed=seed,
                            offset=offset, tag=tag, row_ids=col_ids)


def quantize_2d(x, amax=None, rounding="rtne", seed=0, offset=0):
    """Rowwise and columnwise planes of one tensor under one shared per-tensor scale."""
    xf = _as_f32(x)
    a = _amax(xf) if amax is None else F32(amax)
    row = quantize_rowwise(xf, amax=a, rounding=rounding, seed=seed, offset=offset, tag=0)
    col = quantize_colwise(xf, amax=a, rounding=rounding, seed=seed, offset=offset)
    return {"row": row, "col": col, "amax": F32(a), "s_enc": row["s_enc"], "s_dec": row["s_dec"]}


def quantize_2d_block(x, amax=None, rounding="rtne", seed=0, offset=0, origin=(0, 0), full=None, tags=(0, 1)):
    """Rowwise and columnwise planes under one E4M3 scale per 16 x 16 tile (reading R-2dblk).

    PR, Optimization item 2 describes the 2D weight kernel's columnwise reads as
    paired so that neighbouring rows of the transposed plane share one amax and
    one reciprocal, and the Performance section measures "2D weights" beside
    the 1D paths, but the pages never define the tile. Reading R-2dblk: the block
    amax is taken over the 16 x 16 tile (rows 16i..16i+15, columns 16j..16j+15),
    its scale code is R-bscale of that tile amax, and every element of the tile
    is encoded with it (R-rcp, R-e2m1 / R-sr) in both planes, so a weight and its
    transpose decode to the same values. The planes keep the 1D layout: the
    rowwise scales [M, K/16] repeat the tile's code on its 16 rows, the
    columnwise scales [K, M/16] on its 16 columns. SR bytes are drawn per plane
    exactly as in quantize_2d (tag 0 rowwise with block row*(K/16)+j, tag 1
    columnwise with block col*(M/16)+i).

    origin, full (sampling only): x is the window of a [full] tensor whose first
    element sits at row, column `origin` (multiples of 16); SR block indices are
    then those of the full tensor, and amax must be given.
    """
    xf = _as_f32(x)
    M, K = xf.shape
    assert M % BLOCK == 0 and K % BLOCK == 0
    r0, c0 = (int(v) for v in origin)
    FM, FK = (M, K) if full is None else (int(v) for v in full)
    assert r0 % BLOCK == 0 and c0 % BLOCK == 0 and r0 + M <= FM and c0 + K <= FK
    assert full is None or amax is not None, "a sampled window needs the full tensor's amax"
    a = _amax(xf) if amax is None else F32(amax)
    s_enc, s_dec = global_scales(a)
    tiles = np.abs(xf).reshape(M // BLOCK, BLOCK, K // BLOCK, BLOCK)
    tmax = tiles.max(axis=(1, 3)) if xf.size else np.zeros((M // BLOCK, K // BLOCK), F32)   # [M/16, K/16]
    tsc = block_scale_codes(tmax, s_enc)
    # rowwise: block (r, j) takes tile (r // 16, j)
    row_sc = np.repeat(tsc, BLOCK, axis=0)                                                  # [M, K/16]
    rb = None
    if rounding == "sr":
        blk = (np.arange(r0, r0 + M, dtype=np.uint64)[:, None] * np.uint64(FK // BLOCK)
               + np.arange(c0 // BLOCK, (c0 + K) // BLOCK, dtype=np.uint64)[None, :])
        rb = block_random_bytes(blk, tags[0], seed, offset)
    rcodes = encode_blocks(xf.reshape(M, K // BLOCK, BLOCK), row_sc, s_dec, rounding, rb)
    # columnwise: block (c, i) of the transposed plane takes tile (i, c // 16)
    xt = np.ascontiguousarray(xf.T)
    col_sc = np.repeat(tsc.T, BLOCK, axis=0)                                                # [K, M/16]
    cb = None
    if rounding == "sr":
        blk = (np.arange(c0, c0 + K, dtype=np.uint64)[:, None] * np.uint64(FM // BLOCK)
               + np.arange(r0 // BLOCK, (r0 + M) // BLOCK, dtype=np.uint64)[None, :])
        cb = block_random_bytes(blk, tags[1], seed, offset)
    ccodes = encode_blocks(xt.reshape(K, M // BLOCK, BLOCK), col_sc, s_dec, rounding, cb)
    row = {"codes": pack_nibbles(rcodes.reshape(M, K)), "scales": row_sc.astype(np.uint8)}
    col = {"codes": pack_nibbles(ccodes.reshape(K, M)), "scales": col_sc.astype(np.uint8)}
    return {"row": row, "col": col, "tile_scales": tsc, "amax": F32(a), "s_enc": F32(s_enc),
            "s_dec": F32(s_dec)}


def quantize_2d_experts(x, experts, amax=None, rounding="rtne", seed=0, offset=0, tile16=False):
    """Grouped 2D weights: E experts' [M, K] weights stacked as x[E*M, K], each with its own amax.

    PR, Performance measures a grouped 2D weight kernel (E = 4) beside the
    single-weight one without defining how experts are told apart. Reading
    R-experts: expert e is quantize_2d (or quantize_2d_block with tile16) of its
    own weight under its own amax (max |x_e|, or amax[e]), with SR tags 2e
    (rowwise) and 2e + 1 (columnwise), so expert 0 is the single-weight call and
    no two experts share a random stream. Planes are stacked: rowwise codes
    [E*M, K/2], scales [E*M, K/16]; columnwise codes [E*K, M/2], scales
    [E*K, M/16] (expert e's transposed plane in rows e*K .. e*K + K - 1).
    """
    xf = _as_f32(x)
    EM, K = xf.shape
    assert experts >= 1 and EM % experts == 0
    M = EM // experts
    outs = []
    for e in range(experts):
        xe = xf[e * M:(e + 1) * M]
        a = _amax(xe) if amax is None else F32(np.asarray(amax, dtype=F32)[e])
        if tile16:
            q = quantize_2d_block(xe, amax=a, rounding=rounding, seed=seed, offset=offset, tags=(2 * e, 2 * e + 1))
            outs.append((q["row"], q["col"], a, q["s_dec"]))
        else:
            r = quantize_rowwise(xe, amax=a, rounding=rounding, seed=seed, offset=offset, tag=2 * e)
            c = quantize_colwise(xe, amax=a, rounding=rounding, seed=seed, offset=offset, tag=2 * e + 1)
            outs.append((r, c, a, r["s_dec"]))
    cat = np.concatenate
    return {"row": {"codes": cat([o[0]["codes"] for o in outs]), "scales": cat([o[0]["scales"] for o in outs])},
            "col": {"codes": cat([o[1]["codes"] for o in outs]), "scales": cat([o[1]["scales"] for o in outs])},
            "amax": np.array([o[2] for o in outs], F32), "s_dec": np.array([o[3] for o in outs], F32)}


def dequantize_rowwise(codes, scales, s_dec):
    """Test helper: x_hat = e2m1(code) * f32(scale) * S_dec, in float64 (no rounding claims)."""
    c = unpack_nibbles(codes)
    M, K = c.shape
    v = e2m1_decode(c).astype(np.float64).reshape(M, K // BLOCK, BLOCK)
    s = e4m3_decode(scales).astype(np.float64)[..., None]
    return (v * s * float(s_dec)).reshape(M, K)

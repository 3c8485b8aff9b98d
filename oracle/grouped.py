"""Grouped (per-expert) columnwise NVFP4 over a packed token tensor.

Test infrastructure only.

PR, Grouped allocation tail: the grouped kernels write rows only up to the
last logical row; storage capacity past it is left untouched and its content
unspecified. PR, Config surface and AUTO: groups are described by a packed
tensor plus device-side offsets, with at most 64 groups. PR, Correctness: a
short trailing column group must be handled. Blog, MoE: token copies go into
optionally padded per-expert buffers.

Reading R-group: group g holds rows offsets[g]..offsets[g+1]-1. It is padded
with zero rows to P_g = 16 * ceil(n_g / 16) rows; the padded groups sit back to
back, so group g owns token columns Poff[g]..Poff[g]+P_g-1 of one transposed
plane (codes [K, Poff[G]/2], scales [K, Poff[G]/16]). The transform (if on) and
the per-group amax see the zero-padded rows. SR block index (R-blk) is
col * (Poff[G]/16) + Poff[g]/16 + b, tag 1.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f32, pack_nibbles
from .philox import block_random_bytes
from .quantize import global_scales, quantize_blocks, quantize_rowwise
from .rht import rht16, rht16_f32

MAX_GROUPS = 64


def padded_offsets(offsets) -> np.ndarray:
    """offsets[G+1] -> padded offsets Poff[G+1] (exclusive prefix sum of 16-rounded counts)."""
    off = np.asarray(offsets, dtype=np.int64)
    n = np.diff(off)
    assert np.all(n >= 0) and off[0] == 0
    p = (n + 15) // 16 * 16
    out = np.zeros(len(off), dtype=np.int64)
    out[1:] = np.cumsum(p)
    return out.astype(np.int32)


def grouped_quantize(x, offsets, apply_rht=True, rht_mask=0, amax=None, rounding="sr",
                     seed=0, offset=0, groups=None, fast_math=False, rowwise=False, row_amax=None,
                     colwise=True, ends_only=False):
    """Reference for the grouped path: the columnwise plane, optionally the rowwise one.

    x: bf16 bits [total_rows, K]. offsets: int32 [G+1]. amax: optional float32 [G].
    groups: optional iterable restricting which groups are computed (for sampling);
    columns of other groups are left as 0 in the returned planes.
    fast_math: PR, Fast math -- the transform's output enters the amax and the
    quantization in float32, without the bf16 round-through (reading R-fast).
    rowwise: also the rowwise plane of the same input (reading R-rowcol): each
    group's rows quantized rowwise, without the transform, under the group's own
    amax max|x| (row_amax: optional float32 [G] given instead); SR tag 0, block
    index row * (K/16) + k/16 with the row's index in x. Adds row_codes
    [total_rows, K/2], row_scales [total_rows, K/16], row_amax, row_s_dec [G].
    colwise=False skips the columnwise plane (its arrays stay zero).
    ends_only: quantize only the first and the last 16-token block of each computed
    group in the columnwise plane (for sampling large inputs; the group amax still
    covers every block of the group; the other blocks' bytes stay zero).
    x may also hold float16 or float32 values (reading R-dtype): the transform's
    output is then rounded through the input's type (fp16), or not at all (fp32).
    Returns dict with codes [K, Mpad/2], scales [K, Mpad/16], amax [G], s_enc [G],
    s_dec [G], poff [G+1].
    """
    x = np.asarray(x)
    if x.dtype not in (np.float16, np.float32):
        x = x.astype(np.uint16)
    dt = {np.dtype(np.uint16): "bf16", np.dtype(np.float16): "fp16", np.dtype(np.float32): "fp32"}[x.dtype]
    T, K = x.shape
    off = np.asarray(offsets, dtype=np.int64)
    G = len(off) - 1
    assert 1 <= G <= MAX_GROUPS and off[-1] == T
    poff = padded_offsets(off).astype(np.int64)
    mpad = int(poff[-1])
    codes = np.zeros((K, mpad // 2), dtype=np.uint8)
    scales = np.zeros((K, mpad // 16), dtype=np.uint8)
    amax_out = np.zeros(G, dtype=np.float32)
    s_enc_out = np.ones(G, dtype=np.float32)
    s_dec_out = np.ones(G, dtype=np.float32)
    sel = range(G) if groups is None else groups
    for g in (sel if colwise else ()):
        n = int(off[g + 1] - off[g])
        pg = int(poff[g + 1] - poff[g])
        z = np.zeros((pg, K), dtype=x.dtype)
        z[:n] = x[off[g]:off[g + 1]]
        zt = np.ascontiguousarray(z.T).reshape(K, pg // 16, 16)     # column blocks along tokens
        zv = bf16_to_f32(zt) if dt == "bf16" else zt.astype(np.float32)
        if apply_rht and (fast_math or dt == "fp32"):
            zf = rht16_f32(zv, rht_mask)                       # no round-through (fast math; fp32 input)
        elif apply_rht and dt == "bf16":
            zf = bf16_to_f32(rht16(zt, rht_mask))
        elif apply_rht:                                        # fp16: round-through to fp16
            zf = rht16_f32(zv, rht_mask).astype(np.float16).astype(np.float32)
        else:
            zf = zv
        a = np.float32(np.max(np.abs(zf))) if zf.size else np.float32(0.0)
        if amax is not None:
            a = np.float32(np.asarray(amax, dtype=np.float32)[g])
        s_enc, s_dec = global_scales(a)
        amax_out[g], s_enc_out[g], s_dec_out[g] = a, s_enc, s_dec
        if pg == 0:
            continue
        nb = pg // 16
        sel_b = sorted({0, nb - 1}) if ends_only else list(range(nb))   # the blocks quantized
        rb = None
        if rounding == "sr":
            blk = (np.arange(K, dtype=np.uint64)[:, None] * np.uint64(mpad // 16)
                   + np.uint64(poff[g] // 16) + np.asarray(sel_b, dtype=np.uint64)[None, :])
            rb = block_random_bytes(blk, 1, seed, offset)
        if ends_only:
            c, sc = quantize_blocks(zf[:, sel_b], s_enc, s_dec, rounding, rb)
            for j, b in enumerate(sel_b):
                t0 = int(poff[g]) + 16 * b
                codes[:, t0 // 2:t0 // 2 + 8] = pack_nibbles(c[:, j].reshape(K, 16))
                scales[:, t0 // 16] = sc[:, j]
            continue
        c, sc = quantize_blocks(zf, s_enc, s_dec, rounding, rb)
        codes[:, poff[g] // 2:(poff[g] + pg) // 2] = pack_nibbles(c.reshape(K, pg))
        scales[:, poff[g] // 16:(poff[g] + pg) // 16] = sc
    out = {"codes": codes, "scales": scales, "amax": amax_out, "s_enc": s_enc_out,
           "s_dec": s_dec_out, "poff": poff.astype(np.int32)}
    if rowwise:
        row_codes = np.zeros((T, K // 2), dtype=np.uint8)
        row_scales = np.zeros((T, K // 16), dtype=np.uint8)
        ra_out = np.zeros(G, dtype=np.float32)
        rd_out = np.ones(G, dtype=np.float32)
        for g in sel:
            lo, hi = int(off[g]), int(off[g + 1])
            seg = x[lo:hi]
            segv = bf16_to_f32(seg) if dt == "bf16" else seg.astype(np.float32)
            a = (np.float32(np.max(np.abs(segv))) if hi > lo else np.float32(0.0)) \
                if row_amax is None else np.float32(np.asarray(row_amax, dtype=np.float32)[g])
            ra_out[g] = a
            rd_out[g] = global_scales(a)[1]
            if hi > lo:
                q = quantize_rowwise(seg, amax=a, rounding=rounding, seed=seed, offset=offset, tag=0,
                                     row_ids=np.arange(lo, hi))
                row_codes[lo:hi], row_scales[lo:hi] = q["codes"], q["scales"]
        out.update({"row_codes": row_codes, "row_scales": row_scales, "row_amax": ra_out, "row_s_dec": rd_out})
    return out

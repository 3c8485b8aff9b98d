"""Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw, SC'11).

Test infrastructure only. Written from the published definition: a 4x32-bit
counter and a 2x32-bit key; each of the ten rounds multiplies counter words 0
and 2 by two fixed odd constants, keeps the high and low halves of the 64-bit
products, and mixes them with the other two words and the key by XOR; the key
is advanced by two Weyl increments between rounds.

PR, Optimization item 3 and the SR discussion in the conversation: one Philox
4x32-10 evaluation per 16-element block, all four output words consumed, the
counter derived from the block's coordinates rather than from a running
per-thread state. Reading R-philox fixes the key/counter layout.
"""
from __future__ import annotations

import numpy as np

_M0 = np.uint64(0xD2511F53)   # multiplier applied to counter word 0
_M1 = np.uint64(0xCD9E8D57)   # multiplier applied to counter word 2
_W0 = np.uint64(0x9E3779B9)   # key increment, word 0 (golden ratio)
_W1 = np.uint64(0xBB67AE85)   # key increment, word 1 (sqrt(3) - 1)
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Evaluate Philox4x32-10 on arrays of counters.

    ctr: sequence of 4 uint32 arrays (broadcastable), key: sequence of 2 uint32
    values or arrays. Returns four uint32 arrays (output words 0..3).
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK for c in ctr)
    k0, k1 = (np.asarray(k, dtype=np.uint64) & _MASK for k in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = _M0 * c0
        p1 = _M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(np.asarray(w, dtype=np.uint32) for w in (c0, c1, c2, c3))


def block_random_bytes(blk, tag: int, seed: int, offset: int) -> np.ndarray:
    """Random bytes for a set of 16-element blocks: shape blk.shape + (16,), uint8.

    Reading R-philox: key = (seed lo32, seed hi32); counter = (blk lo32,
    blk hi32, tag, offset). Reading R-sr: element j takes byte (j & 3) of
    output word (j >> 2), bytes numbered from the least significant.
    """
    blk = np.asarray(blk, dtype=np.uint64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    w = philox4x32_10(
        (blk & _MASK, blk >> np.uint64(32), np.full_like(blk, tag), np.full_like(blk, int(offset) & 0xFFFFFFFF)),
        (seed & 0xFFFFFFFF, seed >> 32),
    )
    words = np.stack(w, axis=-1)                         # [..., 4] uint32
    j = np.arange(16)
    return ((words[..., j >> 2] >> (8 * (j & 3)).astype(np.uint32)) & np.uint32(0xFF)).astype(np.uint8)

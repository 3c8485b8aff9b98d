"""Pins for the oracle's Philox4x32-10 against two independent implementations.

No known-answer vectors ship in this container, so the oracle is checked for
agreement with rocRAND's host-callable Philox4x32-10 engine and with Triton's
``tl.philox`` run by the Triton CPU interpreter. Neither shares code with
oracle/philox.py; both are used as black boxes through their public API.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np
import pytest

from oracle.philox import philox4x32_10, block_random_bytes

_CASES = [
    # (seed, c0, c1, c2, c3)
    (0, 0, 0, 0, 0),
    (0x5EED, 0, 0, 0, 0),
    (0x5EED, 1, 0, 1, 0),
    (0x1234567890ABCDEF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF),
    (0xDEADBEEFCAFEF00D, 123456789, 42, 2, 7),
    (1, 0x80000000, 3, 1, 0x12345678),
]

_ROCRAND_SRC = r"""
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>
int main(int argc, char** argv) {
  // argv: seed c0 c1 c2 c3. rocRAND keeps a 128-bit counter; its subsequence
  // argument lands in words 2,3 and its offset / 4 in words 0,1. Word 1 is
  // advanced by skipping 2^34 numbers per unit so no 64-bit offset overflows.
  unsigned long long seed = strtoull(argv[1], 0, 0);
  unsigned long long c0 = strtoull(argv[2], 0, 0), c1 = strtoull(argv[3], 0, 0);
  unsigned long long c2 = strtoull(argv[4], 0, 0), c3 = strtoull(argv[5], 0, 0);
  rocrand_state_philox4x32_10 st;
  rocrand_init(seed, (c3 << 32) | c2, 4ull * c0, &st);
  for (int k = 0; k < 32; ++k) {
    if (!((c1 >> k) & 1)) continue;
    if (34 + k <= 62) { skipahead(1ull << (34 + k), &st); continue; }
    for (unsigned long long n = 0; n < (1ull << (34 + k - 62)); ++n) skipahead(1ull << 62, &st);
  }
  for (int i = 0; i < 4; ++i) printf("%u\n", rocrand(&st));
  return 0;
}
"""


def _rocrand_binary(tmp):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    src = os.path.join(tmp, "rr.cpp")
    exe = os.path.join(tmp, "rr")
    with open(src, "w") as f:
        f.write(_ROCRAND_SRC)
    subprocess.run([hipcc, "-O1", src, "-o", exe], check=True, capture_output=True)
    return exe


def test_philox_matches_rocrand_host_engine():
    with tempfile.TemporaryDirectory() as tmp:
        exe = _rocrand_binary(tmp)
        for seed, c0, c1, c2, c3 in _CASES:
            out = subprocess.run([exe, str(seed), str(c0), str(c1), str(c2), str(c3)],
                                 check=True, capture_output=True, text=True).stdout.split()
            ref = [int(v) for v in out]
            got = philox4x32_10((c0, c1, c2, c3), (seed & 0xFFFFFFFF, seed >> 32))
            assert [int(w) for w in got] == ref, (seed, c0, c1, c2, c3)


_TRITON_SCRIPT = r"""
import os, sys, json
os.environ["TRITON_INTERPRET"] = "1"
import numpy as np, torch, triton, triton.language as tl

@triton.jit
def k(out, c_ptr, seed, N: tl.constexpr):
    i = tl.arange(0, N)
    c0 = tl.load(c_ptr + 4 * i + 0)
    c1 = tl.load(c_ptr + 4 * i + 1)
    c2 = tl.load(c_ptr + 4 * i + 2)
    c3 = tl.load(c_ptr + 4 * i + 3)
    a, b, c, d = tl.philox(seed, c0, c1, c2, c3)
    tl.store(out + 4 * i + 0, a)
    tl.store(out + 4 * i + 1, b)
    tl.store(out + 4 * i + 2, c)
    tl.store(out + 4 * i + 3, d)

cases = json.loads(sys.argv[1])
res = []
for seed, c0, c1, c2, c3 in cases:
    cs = torch.tensor([c0, c1, c2, c3], dtype=torch.uint32)
    o = torch.zeros(4, dtype=torch.uint32)
    k[(1,)](o, cs, seed, N=1)
    res.append([int(v) for v in o.tolist()])
print(json.dumps(res))
"""


def test_philox_matches_triton_interpreter():
    pytest.importorskip("triton")
    import json

    cases = [c for c in _CASES if c[0] < (1 << 63)]
    env = dict(os.environ, TRITON_INTERPRET="1")
    p = subprocess.run([sys.executable, "-c", _TRITON_SCRIPT, json.dumps(cases)], env=env,
                       capture_output=True, text=True, timeout=600)
    if p.returncode != 0:
        pytest.skip("triton interpreter unavailable: " + p.stderr[-300:])
    ref = json.loads(p.stdout.strip().splitlines()[-1])
    for (seed, c0, c1, c2, c3), r in zip(cases, ref):
        got = philox4x32_10((c0, c1, c2, c3), (seed & 0xFFFFFFFF, seed >> 32))
        assert [int(w) for w in got] == [v & 0xFFFFFFFF for v in r], (seed, c0, c1, c2, c3)


def test_vectorized_equals_scalar_calls():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 1 << 32, size=(4, 100), dtype=np.uint64).astype(np.uint32)
    vec = philox4x32_10(tuple(c), (0x5EED, 0))
    for i in range(100):
        one = philox4x32_10(tuple(c[:, i]), (0x5EED, 0))
        assert [int(w[i]) for w in vec] == [int(w) for w in one]


def test_block_bytes_layout():
    # element j of a block takes byte (j & 3) of word (j >> 2), LSB first
    w = philox4x32_10((7, 0, 1, 9), (0x5EED, 0))
    b = block_random_bytes(np.array([7], np.uint64), 1, 0x5EED, 9)[0]
    for j in range(16):
        assert b[j] == (int(w[j >> 2]) >> (8 * (j & 3))) & 0xFF


def test_block_bytes_are_the_rocrand_output_in_memory_order():
    # Reading R-sr, stated the other way round: element j of a block takes byte j of the generator's 128-bit
    # output as it lies in memory (four little-endian 32-bit words), here produced by rocRAND's engine for
    # the block's counter (block lo, block hi, tag, offset) and key (seed lo, seed hi). A byte or word order
    # mistake in the oracle (big-endian bytes, reversed words, a shifted lane) fails this.
    cases = [(0x5EED, 7, 1, 9), (0x1234567890ABCDEF, (3 << 32) | 0xFFFFFFF0, 0, 0), (1, 123456, 1, 77)]
    with tempfile.TemporaryDirectory() as tmp:
        exe = _rocrand_binary(tmp)
        for seed, blk, tag, offset in cases:
            out = subprocess.run([exe, str(seed), str(blk & 0xFFFFFFFF), str(blk >> 32), str(tag), str(offset)],
                                 check=True, capture_output=True, text=True).stdout.split()
            mem = np.array([int(v) for v in out], dtype="<u4").tobytes()
            got = block_random_bytes(np.array([blk], np.uint64), tag, seed, offset)[0]
            assert bytes(got.tolist()) == mem, (seed, blk, tag, offset)

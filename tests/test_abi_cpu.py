"""CPU-side checks of the C ABI: the library loads, exports every function that
include/nvfp4q.h declares, and rejects bad arguments before touching the GPU.
Nothing here launches a kernel (every call below fails validation first)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4q.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4q_\w+|rmsnorm_nvfp4q\w*)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    import rmsnorm_nvfp4_block_amd as q

    if not os.path.exists(q.lib_path):
        pytest.fail("libnvfp4q.so is not built (run __graft_entry__.build())")
    return q.load()


def test_header_declares_the_entry_points():
    d = _declared()
    for name in ("nvfp4q_quantize", "rmsnorm_nvfp4q", "nvfp4q_quantize_2d", "nvfp4q_quantize_2d_grouped",
                 "nvfp4q_grouped", "nvfp4q_qk_norm", "rmsnorm_nvfp4q_noalloc"):
        assert name in d


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_names_match_the_abi():
    import rmsnorm_nvfp4_block_amd as q

    for name in ("nvfp4q_quantize", "rmsnorm_nvfp4q", "nvfp4q_quantize_2d", "nvfp4q_quantize_2d_grouped",
                 "nvfp4q_grouped", "nvfp4q_qk_norm", "rmsnorm_nvfp4q_noalloc"):
        assert callable(getattr(q, name))


def test_status_strings_and_workspace(lib):
    import rmsnorm_nvfp4_block_amd as q

    assert lib.nvfp4q_version() == 1
    assert q.nvfp4q_workspace_bytes() % 128 == 0 and q.nvfp4q_workspace_bytes() >= 4096
    for s in range(7):
        assert q.nvfp4q_status_string(s)
    assert q.nvfp4q_status_string(99) == "unknown status"


def test_library_was_built_from_these_sources():
    """The library names the sha256 of the sources it was built from; it is the tree's (rebuild if not)."""
    import rmsnorm_nvfp4_block_amd as q
    from rmsnorm_nvfp4_block_amd import build

    got = q.library_source_sha256()
    assert len(got) == 64 and int(got, 16) >= 0
    assert got == build.source_digest(), "libnvfp4q.so is older than its sources: rebuild it"


FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call fails validation


def _quant(lib, x=FAKE, dtype=0, rows=4, cols=32, ld=32, codes=FAKE, ldc=16, scales=FAKE, lds=2, rnd=0,
           rng=True, ws=FAKE, wsb=1 << 16):
    import rmsnorm_nvfp4_block_amd as q

    plane = q.Plane(codes, ldc, scales, lds)
    g = q.Global(None, None, None)
    r = q.Rng(1, 0)
    return lib.nvfp4q_quantize(x, dtype, rows, cols, ld, ctypes.byref(g), ctypes.byref(plane), rnd,
                               ctypes.byref(r) if rng else None, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), 4),                  # bf16, fp16 or fp32 only
    (dict(dtype=1), 6),                  # fp16 accepted (stops at the small workspace)
    (dict(dtype=2, ld=36), 6),           # fp32 rows of 144 bytes stay 16-byte aligned
    (dict(dtype=2, ld=34), 3),           # 136-byte fp32 rows do not
    (dict(dtype=1, ld=36), 3),           # 72-byte fp16 rows do not
    (dict(cols=24, ld=24), 2),           # cols % 16
    (dict(ld=16), 2),                    # ld < cols
    (dict(ld=1 << 41), 2),               # leading dimensions stop at 2^40
    (dict(ldc=1 << 41), 2),
    (dict(lds=1 << 41), 2),
    (dict(rows=-1), 2),
    (dict(x=0), 1),                      # NULL input
    (dict(x=FAKE + 2), 3),               # misaligned input
    (dict(ld=36, cols=32), 3),           # ld not a multiple of 8 elements
    (dict(codes=0), 1),
    (dict(ldc=8), 2),                    # plane row too short
    (dict(codes=FAKE + 8), 3),
    (dict(ldc=20), 3),
    (dict(rnd=2), 4),
    (dict(rnd=1, rng=False), 1),         # SR needs an rng
    (dict(ws=0), 6),
    (dict(ws=FAKE + 16), 6),             # workspace alignment
    (dict(wsb=100), 6),
])
def test_quantize_validation(lib, kw, status):
    assert _quant(lib, **kw) == status


def test_rmsnorm_validation(lib):
    import rmsnorm_nvfp4_block_amd as q

    plane = q.Plane(FAKE, 16, FAKE, 2)
    g = q.Global(None, None, None)
    r = q.Rng(0, 0)

    def call(gamma=FAKE, beta=None, woff=0.0, eps=1e-6, y=None, ldy=0, hidden=32, p=plane, ws=FAKE, dtype=0):
        return lib.rmsnorm_nvfp4q(FAKE, dtype, 4, hidden, hidden, gamma, beta, woff, eps, y, ldy, ctypes.byref(g),
                                  ctypes.byref(p), 0, ctypes.byref(r), ws, 1 << 16, None)

    assert call(gamma=None) == 1
    assert call(beta=FAKE + 4) == 3
    assert call(woff=0.5) == 4
    assert call(eps=-1.0) == 2
    assert call(hidden=40) == 2
    # rows beyond 32 superchunks (2-byte types) or 16 (fp32)
    assert call(hidden=32 * 1024 + 16, p=q.Plane(FAKE, 16392, FAKE, 2050)) == 4
    assert call(hidden=16 * 1024 + 16, p=q.Plane(FAKE, 8208, FAKE, 1026), dtype=2) == 4
    assert call(p=q.Plane(None, 0, None, 0)) == 1                               # nothing to produce
    assert call(p=q.Plane(None, 0, None, 0), y=FAKE, ldy=16) == 2
    assert call(p=q.Plane(None, 0, None, 0), y=FAKE + 2, ldy=32) == 3
    assert call(p=q.Plane(None, 0, None, 0), y=FAKE, ldy=1 << 41) == 2
    assert call(ws=None) == 6


def test_dtype_acceptance_per_entry_point(lib):
    # Every call here stops at validation: the workspace is too small (1 << 16 bytes, status 6) for the
    # accepted dtypes, so nothing is ever launched on the fake pointers.
    import rmsnorm_nvfp4_block_amd as q

    g = q.Global(None, None, None)
    r = q.Rng(0, 0)
    p = q.Plane(FAKE, 16, FAKE, 2)
    for dt in (1, 2):
        assert lib.rmsnorm_nvfp4q(FAKE, dt, 4, 32, 32, FAKE, None, 0.0, 1e-6, None, 0, ctypes.byref(g),
                                  ctypes.byref(p), 0, ctypes.byref(r), FAKE, 1 << 16, None) == 6   # fp16/fp32 taken
        assert lib.nvfp4q_quantize_2d(FAKE, dt, 32, 32, 32, ctypes.byref(g), ctypes.byref(p), None, 0,
                                      ctypes.byref(r), FAKE, 1 << 16, None) == 6    # fp16/fp32 taken
        pg = q.Plane(FAKE, 32, FAKE, 4)
        assert lib.nvfp4q_grouped(FAKE, dt, 32, 32, 32, FAKE, 1, None, 1, 0, ctypes.byref(g), ctypes.byref(pg),
                                  None, None, 0, ctypes.byref(r), FAKE, 1 << 16, None) == 6    # fp16/fp32 taken
    assert lib.rmsnorm_nvfp4q(FAKE, 3, 4, 32, 32, FAKE, None, 0.0, 1e-6, None, 0, ctypes.byref(g),
                              ctypes.byref(p), 0, ctypes.byref(r), FAKE, 1 << 16, None) == 4
    # fp32 y rows must stay 16-byte aligned: ld_y 34 floats = 136 bytes
    assert lib.rmsnorm_nvfp4q(FAKE, 2, 4, 32, 32, FAKE, None, 0.0, 1e-6, FAKE, 34, ctypes.byref(g),
                              ctypes.byref(p), 0, ctypes.byref(r), FAKE, 1 << 16, None) == 3
    # the QK norm takes all three; an unknown dtype is refused before anything is launched
    assert lib.nvfp4q_qk_norm(FAKE, None, 3, 3, 4, 0, 128, 512, 0, FAKE, None, 0.0, 1e-6, None) == 4
    assert lib.nvfp4q_qk_norm(FAKE, None, 2, 3, 4, 0, 128, 510, 0, FAKE, None, 0.0, 1e-6, None) == 2
    assert lib.nvfp4q_qk_norm(FAKE, None, 2, 3, 4, 0, 64, 258, 0, FAKE, None, 0.0, 1e-6, None) == 3


def test_qk_norm_validation(lib):
    def call(d=128, hq=4, hk=2, ldq=512, ldk=256, q=FAKE, k=FAKE, wq=FAKE, wk=FAKE, woff=0.0, eps=1e-6, t=3):
        return lib.nvfp4q_qk_norm(q, k, 0, t, hq, hk, d, ldq, ldk, wq, wk, woff, eps, None)

    assert call(d=96) == 4 and call(d=512) == 4
    assert call(hq=0, hk=0) == 2 and call(hq=-1) == 2
    assert call(ldq=504) == 2 and call(ldk=248) == 2
    assert call(q=None) == 1 and call(wk=None) == 1
    assert call(q=FAKE + 8) == 3 and call(ldq=516) == 3
    assert call(ldq=1 << 41) == 2 and call(ldk=1 << 41) == 2
    assert call(woff=0.5) == 4 and call(eps=-1.0) == 2
    assert call(t=0, q=None, k=None, wq=None, wk=None) == 0      # nothing to do, nothing launched
    assert call(hk=0, t=0, k=None, wk=None) == 0


def test_2d_and_grouped_validation(lib):
    import rmsnorm_nvfp4_block_amd as q

    g = q.Global(None, None, None)
    r = q.Rng(0, 0)
    none = q.Plane(None, 0, None, 0)
    row = q.Plane(FAKE, 16, FAKE, 2)
    col = q.Plane(FAKE, 16, FAKE, 2)
    # columnwise plane needs rows % 16 == 0
    assert lib.nvfp4q_quantize_2d(FAKE, 0, 24, 32, 32, ctypes.byref(g), ctypes.byref(row), ctypes.byref(col), 0,
                                  ctypes.byref(r), FAKE, 1 << 16, None) == 2
    assert lib.nvfp4q_quantize_2d(FAKE, 0, 32, 32, 32, ctypes.byref(g), ctypes.byref(none), ctypes.byref(none), 0,
                                  ctypes.byref(r), FAKE, 1 << 16, None) == 1

    def experts(e, rows=64, cols=32, rowp=row, colp=col, rounding=0):
        return lib.nvfp4q_quantize_2d_grouped(FAKE, 0, e, rows, cols, cols, ctypes.byref(g), ctypes.byref(rowp),
                                              ctypes.byref(colp), rounding, ctypes.byref(r), FAKE, 1 << 8, None)

    big_row, big_col = q.Plane(FAKE, 16, FAKE, 2), q.Plane(FAKE, 32, FAKE, 4)
    assert experts(0) == 2 and experts(65) == 2
    assert experts(4, rowp=big_row, colp=big_col) == 6                   # valid; stops at the small workspace
    assert experts(4, rows=24, rowp=big_row, colp=none) == 6             # rowwise only: rows need not be 16k
    assert experts(4, rows=24, rowp=big_row, colp=big_col) == 2          # columnwise needs rows % 16 == 0
    assert experts(4, rows=24, rowp=big_row, colp=none, rounding=0x200) == 2   # and so do tile scales

    def grouped(groups=4, rht=1, mask=0x1234, ldc=64, lds=8, offs=FAKE, rows=64, ld=32, colp=True, rowp=None):
        p = q.Plane(FAKE, ldc, FAKE, lds)
        return lib.nvfp4q_grouped(FAKE, 0, rows, 32, ld, offs, groups, None, rht, mask, ctypes.byref(g),
                                  ctypes.byref(p) if colp else None, ctypes.byref(g),
                                  ctypes.byref(rowp) if rowp is not None else None, 1, ctypes.byref(r), FAKE,
                                  1 << 16, None)

    assert grouped(groups=0) == 2
    assert grouped(groups=65) == 2
    assert grouped(rht=2) == 4
    assert grouped(mask=0x10000) == 4
    assert grouped(offs=0) == 1
    assert grouped(ldc=48) == 2       # 2 * 48 < 64 + 15 * 4
    assert grouped(lds=7) == 2        # 16 * 7 < 124
    assert grouped(ld=(1 << 24) + 8) == 2   # row stride past the 32-bit offsets of the loads
    assert grouped(colp=False) == 1                                        # no plane at all
    p_noscales = q.Plane(FAKE, 64, None, 8)
    assert lib.nvfp4q_grouped(FAKE, 0, 64, 32, 32, FAKE, 4, None, 1, 0x1234, ctypes.byref(g),
                              ctypes.byref(p_noscales), None, None, 1, ctypes.byref(r), FAKE, 1 << 16, None) == 1
    # an empty 2D input may come with NULL plane pointers (rows of zero elements)
    assert lib.nvfp4q_quantize_2d(FAKE, 0, 0, 32, 32, ctypes.byref(g), ctypes.byref(none), ctypes.byref(none), 0,
                                  ctypes.byref(r), FAKE, 1 << 16, None) == 6
    assert grouped(colp=False, rowp=q.Plane(None, 16, None, 2)) == 1       # rows but no rowwise buffers
    assert grouped(colp=False, rowp=q.Plane(FAKE, 8, FAKE, 2)) == 2        # 8 < 32 / 2 code bytes per row
    assert grouped(colp=False, rowp=q.Plane(FAKE, 16, FAKE, 1)) == 2       # 1 < 32 / 16 scale bytes per row
    assert grouped(colp=False, rowp=q.Plane(FAKE, 16, FAKE, 2)) == 6       # valid; stops at the small workspace
    assert grouped(rowp=q.Plane(FAKE, 16, FAKE, 2)) == 6
    assert grouped(rows=0, colp=False, rowp=q.Plane(None, 16, None, 2)) == 6   # an empty rowwise plane


def test_rounding_option_bits(lib):
    import rmsnorm_nvfp4_block_amd as q

    hdr = open(os.path.join(ROOT, "include", "nvfp4q.h")).read()
    assert "#define NVFP4Q_FAST_MATH 0x100" in hdr and q.FAST_MATH == 0x100
    g = q.Global(None, None, None)
    r = q.Rng(0, 0)

    def grouped(rounding):
        p = q.Plane(FAKE, 64, FAKE, 8)
        # a workspace smaller than required: accepted rounding values pass their check and stop at the
        # workspace check (6); others stop at the rounding check (4). Nothing is launched.
        return lib.nvfp4q_grouped(FAKE, 0, 64, 32, 32, FAKE, 4, None, 1, 0x1234, ctypes.byref(g),
                                  ctypes.byref(p), None, None, rounding, ctypes.byref(r), FAKE, 1 << 16, None)

    assert grouped(q.RTNE | q.FAST_MATH) == 6 and grouped(q.SR | q.FAST_MATH) == 6
    assert grouped(2) == 4 and grouped(0x400) == 4 and grouped(q.SR | 0x400) == 4
    assert "#define NVFP4Q_SCALE_16X16 0x200" in hdr and q.SCALE_16X16 == 0x200
    assert grouped(q.SCALE_16X16) == 4      # tile scales exist on the 2D path only

    def two_d(rounding, rows=64, colp=True):
        p = q.Plane(FAKE, 64, FAKE, 8)
        return lib.nvfp4q_quantize_2d(FAKE, 0, rows, 32, 32, ctypes.byref(g), ctypes.byref(p),
                                      ctypes.byref(p) if colp else None, rounding, ctypes.byref(r), FAKE, 1 << 8,
                                      None)

    assert two_d(q.SCALE_16X16) == 6 and two_d(q.SR | q.SCALE_16X16 | q.FAST_MATH) == 6
    assert two_d(q.SCALE_16X16 | 0x400) == 4   # NVFP4Q_ONE_LAUNCH belongs to the RMSNorm entry points
    assert "#define NVFP4Q_ONE_LAUNCH 0x400" in hdr and q.ONE_LAUNCH == 0x400

    def rms(rounding):
        p = q.Plane(FAKE, 16, FAKE, 2)
        return lib.rmsnorm_nvfp4q(FAKE, 0, 8, 32, 32, FAKE, None, ctypes.c_float(0.0), ctypes.c_float(1e-6),
                                  None, 0, ctypes.byref(g), ctypes.byref(p), rounding, ctypes.byref(r), FAKE, 1 << 8,
                                  None)

    assert rms(q.ONE_LAUNCH) == 6 and rms(q.SR | q.ONE_LAUNCH) == 6   # accepted: stops at the small workspace
    assert rms(q.ONE_LAUNCH | q.SCALE_16X16) == 4
    assert two_d(q.SCALE_16X16, rows=24, colp=False) == 2   # tiles need rows % 16 == 0
    assert two_d(q.RTNE, rows=24, colp=False) == 6          # 1D rowwise does not


def test_binding_keeps_one_workspace_per_stream(monkeypatch):
    """The Python binding gives calls on different streams different workspaces (calls that may overlap
    must not share one), and reuses a stream's workspace for every later call on it."""
    import torch

    import rmsnorm_nvfp4_block_amd as q

    made = []

    def fake_alloc(dev):
        made.append(dev)
        return object()

    monkeypatch.setattr(q, "_alloc_workspace", fake_alloc)
    monkeypatch.setattr(q, "_ws", {})
    dev = torch.device("cuda", 0)
    a, b = q.workspace(dev, stream=0x1000), q.workspace(dev, stream=0x2000)
    assert a is not b
    assert q.workspace(dev, stream=0x1000) is a and q.workspace(dev, stream=0x2000) is b
    assert q.workspace(torch.device("cuda", 1), stream=0x1000) is not a   # per device as well
    assert len(made) == 3


def test_rmsnorm_noalloc_validation(lib):
    """The no-allocation entry point validates like rmsnorm_nvfp4q, before it looks up its static
    workspace (so on a host without a GPU these calls never reach the device)."""
    import rmsnorm_nvfp4_block_amd as q

    plane = q.Plane(FAKE, 16, FAKE, 2)
    g = q.Global(None, None, None)
    r = q.Rng(0, 0)

    def call(x=FAKE, dtype=0, gamma=FAKE, beta=None, woff=0.0, eps=1e-6, hidden=32, p=plane, rnd=0):
        return lib.rmsnorm_nvfp4q_noalloc(x, dtype, 4, hidden, hidden, gamma, beta, woff, eps, None, 0,
                                          ctypes.byref(g), ctypes.byref(p), rnd, ctypes.byref(r), None)

    assert call(gamma=None) == 1
    assert call(x=FAKE + 2) == 3
    assert call(dtype=3) == 4
    assert call(beta=FAKE + 4) == 3
    assert call(woff=0.5) == 4
    assert call(eps=-1.0) == 2
    assert call(hidden=40) == 2
    assert call(p=q.Plane(None, 0, None, 0)) == 1
    assert call(rnd=2) == 4


def test_ceilings_probe_library_exports():
    """The probe kernels bench.py --ceilings runs are built beside the library and export their entry points."""
    import ctypes
    import os

    import rmsnorm_nvfp4_block_amd as q

    path = os.path.join(os.path.dirname(os.path.abspath(q.__file__)), "libnvfp4q_ceilings.so")
    assert os.path.exists(path), "build the library first"
    lib = ctypes.CDLL(path)
    for name in ("ceil_read", "ceil_mix", "ceil_rowmix", "ceil_fused", "ceil_fused_ws_bytes", "ceil_fused_count",
                 "ceil_fused_count_ws_bytes", "ceil_rate", "ceil_rate_kinds", "ceil_rate_name", "ceil_empty"):
        assert hasattr(lib, name), name
    lib.ceil_fused_ws_bytes.restype = ctypes.c_uint64
    assert lib.ceil_fused_ws_bytes() == 128 + 8 * 4096
    # counter form: header line, two count lines, two maximum lines, 64 flag lines, 4096 slots
    lib.ceil_fused_count_ws_bytes.restype = ctypes.c_uint64
    assert lib.ceil_fused_count_ws_bytes() == 128 + 2 * 128 + 2 * 128 + 64 * 128 + 8 * 4096
    # argument checks come before any runtime call (hipErrorInvalidValue = 1)
    vp, u32 = ctypes.c_void_p, ctypes.c_uint32
    lib.ceil_fused_count.argtypes = [vp, u32, vp, vp, vp, u32, ctypes.c_int, vp]
    assert lib.ceil_fused_count(None, 64, None, None, None, 1, 5, None) == 1
    assert lib.ceil_fused_count(None, 63, None, None, None, 1, 0, None) == 1
    lib.ceil_rate_name.restype = ctypes.c_char_p
    lib.ceil_rate_name.argtypes = [ctypes.c_int]
    n = lib.ceil_rate_kinds()
    names = [lib.ceil_rate_name(k).decode() for k in range(n)]
    assert n == 16 and names[0] == "v_add_u32" and len(set(names)) == n
    assert lib.ceil_rate_name(n) is None and lib.ceil_rate_name(-1) is None
    lib.ceil_rate.argtypes = [ctypes.c_int, u32, u32, vp, vp]
    assert lib.ceil_rate(n, 1, 1, None, None) == 1

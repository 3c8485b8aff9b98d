"""Python binding of the gfx950 RMSNorm + NVFP4 block-quantization library.

Argument marshalling only: torch tensors provide device memory and the current
HIP stream; every step of the computation runs in the HIP kernels of
``libnvfp4q.so`` through its C ABI (``include/nvfp4q.h``). The functions carry
the C entry points' names. There is no CPU fallback: if the shared library is
missing, :func:`load` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "load", "lib_path", "workspace", "NVFP4QError",
    "nvfp4q_quantize", "rmsnorm_nvfp4q", "nvfp4q_quantize_2d", "nvfp4q_quantize_2d_grouped", "nvfp4q_grouped",
    "nvfp4q_qk_norm", "rmsnorm_nvfp4q_noalloc", "nvfp4q_workspace_bytes", "nvfp4q_status_string", "SYMBOLS",
    "library_source_sha256",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libnvfp4q.so")

SYMBOLS = ("nvfp4q_quantize", "rmsnorm_nvfp4q", "nvfp4q_quantize_2d", "nvfp4q_quantize_2d_grouped", "nvfp4q_grouped",
           "nvfp4q_qk_norm", "rmsnorm_nvfp4q_noalloc",
           "nvfp4q_workspace_bytes", "nvfp4q_status_string", "nvfp4q_version", "nvfp4q_source_sha256")

RTNE, SR = 0, 1
FAST_MATH = 0x100  # NVFP4Q_FAST_MATH, OR-ed into the rounding argument
SCALE_16X16 = 0x200  # NVFP4Q_SCALE_16X16 (nvfp4q_quantize_2d only), OR-ed into the rounding argument
ONE_LAUNCH = 0x400  # NVFP4Q_ONE_LAUNCH (the RMSNorm entry points only), OR-ed into the rounding argument


class Plane(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("ld_scales", ctypes.c_int64)]


class Global(ctypes.Structure):
    _fields_ = [("amax_in", ctypes.c_void_p), ("amax_out", ctypes.c_void_p), ("scale_out", ctypes.c_void_p)]


class Rng(ctypes.Structure):
    _fields_ = [("seed", ctypes.c_uint64), ("offset", ctypes.c_uint32)]


class NVFP4QError(RuntimeError):
    pass


_lib = None


def load():
    """Load ``libnvfp4q.so`` (built by ``rmsnorm_nvfp4_block_amd.build``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise NVFP4QError(f"{lib_path} not found: build it with `python -m rmsnorm_nvfp4_block_amd.build`")
    lib = ctypes.CDLL(lib_path)
    vp, i64, f32, i32, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int32, ctypes.c_uint32
    P = ctypes.POINTER
    lib.nvfp4q_workspace_bytes.restype = ctypes.c_size_t
    lib.nvfp4q_status_string.restype = ctypes.c_char_p
    lib.nvfp4q_status_string.argtypes = [ctypes.c_int]
    lib.nvfp4q_version.restype = ctypes.c_int
    lib.nvfp4q_source_sha256.restype = ctypes.c_char_p
    lib.nvfp4q_quantize.restype = ctypes.c_int
    lib.nvfp4q_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, P(Global), P(Plane), ctypes.c_int, P(Rng),
                                    vp, ctypes.c_size_t, vp]
    lib.rmsnorm_nvfp4q.restype = ctypes.c_int
    lib.rmsnorm_nvfp4q.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, f32, f32, vp, i64, P(Global), P(Plane),
                                   ctypes.c_int, P(Rng), vp, ctypes.c_size_t, vp]
    lib.rmsnorm_nvfp4q_noalloc.restype = ctypes.c_int
    lib.rmsnorm_nvfp4q_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, f32, f32, vp, i64, P(Global),
                                           P(Plane), ctypes.c_int, P(Rng), vp]
    lib.nvfp4q_quantize_2d.restype = ctypes.c_int
    lib.nvfp4q_quantize_2d.argtypes = [vp, ctypes.c_int, i64, i64, i64, P(Global), P(Plane), P(Plane), ctypes.c_int,
                                       P(Rng), vp, ctypes.c_size_t, vp]
    lib.nvfp4q_quantize_2d_grouped.restype = ctypes.c_int
    lib.nvfp4q_quantize_2d_grouped.argtypes = [vp, ctypes.c_int, i32, i64, i64, i64, P(Global), P(Plane), P(Plane),
                                               ctypes.c_int, P(Rng), vp, ctypes.c_size_t, vp]
    lib.nvfp4q_qk_norm.restype = ctypes.c_int
    lib.nvfp4q_qk_norm.argtypes = [vp, vp, ctypes.c_int, i64, i32, i32, i32, i64, i64, vp, vp, f32, f32, vp]
    lib.nvfp4q_grouped.restype = ctypes.c_int
    lib.nvfp4q_grouped.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i32, vp, ctypes.c_int, u32, P(Global),
                                   P(Plane), P(Global), P(Plane), ctypes.c_int, P(Rng), vp, ctypes.c_size_t, vp]
    _lib = lib
    return lib


def nvfp4q_workspace_bytes() -> int:
    return int(load().nvfp4q_workspace_bytes())


def nvfp4q_status_string(status: int) -> str:
    return load().nvfp4q_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise NVFP4QError(f"nvfp4q status {status}: {nvfp4q_status_string(status)}")


_ws = {}


def _alloc_workspace(dev):
    """Device memory for one workspace from torch's allocator, zero-filled as the C ABI asks before first use."""
    import torch

    return torch.zeros(max(nvfp4q_workspace_bytes(), 4096), dtype=torch.uint8, device=dev)


def library_source_sha256() -> str:
    """The sha256 of the sources the loaded library was built from (``nvfp4q_source_sha256``); compare with
    ``rmsnorm_nvfp4_block_amd.build.source_digest()`` of the tree."""
    return load().nvfp4q_source_sha256().decode()


def workspace(device=None, stream=None):
    """The workspace for calls enqueued on `stream` (a HIP stream handle; default: torch's current stream
    on the device): one per (device, stream), allocated on first use and reused by every later call on
    that stream, which the stream orders. Calls on different streams get different workspaces, so they
    may run at the same time (the C ABI requires that of concurrent calls)."""
    import torch

    if device is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    else:
        dev = torch.device(device)
        dev = torch.device("cuda", dev.index if dev.index is not None else torch.cuda.current_device())
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    key = (dev.index, int(stream))
    if key not in _ws:
        _ws[key] = _alloc_workspace(dev)
    return _ws[key]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def _rounding(r: str) -> int:
    if r not in ("rtne", "sr"):
        raise ValueError(f"rounding must be 'rtne' or 'sr', not {r!r}")
    return SR if r == "sr" else RTNE


def _dtype_code(x):
    """nvfp4q_dtype of a 2-D row-contiguous CUDA tensor (bf16, fp16 or fp32)."""
    import torch

    codes = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}
    if x.dtype not in codes or x.dim() != 2 or x.stride(1) != 1 or not x.is_cuda:
        raise ValueError("x must be a 2-D row-contiguous bfloat16, float16 or float32 CUDA tensor")
    return codes[x.dtype]


def _plane(rows: int, cols: int, device, codes=None, scales=None):
    """Allocate (or wrap) a plane of `rows` plane rows of `cols` elements."""
    import torch

    if codes is None:
        ldc = ((cols // 2) + 15) // 16 * 16
        codes = torch.empty((rows, ldc), dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty((rows, max(cols // 16, 1)), dtype=torch.uint8, device=device)
    return codes, scales, Plane(codes.data_ptr(), codes.stride(0), scales.data_ptr(), scales.stride(0))


def _global(amax_in, amax_out, scale_out):
    return Global(_ptr(amax_in), _ptr(amax_out), _ptr(scale_out))


def nvfp4q_quantize(x, amax=None, rounding="rtne", seed=0, offset=0, codes=None, scales=None):
    """Rowwise NVFP4 of a bf16, fp16 or fp32 [rows, cols] tensor. Returns dict(codes, scales, amax, scale)."""
    import torch

    dt = _dtype_code(x)
    lib = load()
    R, C = x.shape
    c, s, plane = _plane(R, C, x.device, codes, scales)
    amax_out = torch.empty(1, dtype=torch.float32, device=x.device)
    scale_out = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = workspace(x.device, _stream(x))
    st = lib.nvfp4q_quantize(x.data_ptr(), dt, R, C, x.stride(0), ctypes.byref(_global(amax, amax_out, scale_out)),
                             ctypes.byref(plane), _rounding(rounding), ctypes.byref(Rng(seed, offset)),
                             ws.data_ptr(), ws.numel(), _stream(x))
    _check(st)
    return {"codes": c, "scales": s, "amax": amax_out, "scale": scale_out}


def rmsnorm_nvfp4q(x, gamma, beta=None, weight_offset=0.0, eps=1e-6, amax=None, rounding="rtne", seed=0, offset=0,
                   y_out=False, quantize=True, codes=None, scales=None, one_launch=False):
    """RMSNorm of x [tokens, hidden] (bf16, fp16 or fp32; gamma and beta of the same type) then rowwise NVFP4
    of the output rounded in that type. one_launch: NVFP4Q_ONE_LAUNCH (at most 64 tokens and no given amax:
    one launch that meets on the amax inside it; same results).

    Returns dict(codes, scales, amax, scale, y) (y only when y_out=True).
    """
    import torch

    dt = _dtype_code(x)
    for p in (gamma, beta):
        if p is not None and (p.dtype != x.dtype or not p.is_contiguous()):
            raise ValueError("gamma and beta must be contiguous and of x's dtype")
    lib = load()
    T, H = x.shape
    y = torch.empty_like(x) if y_out else None
    if quantize:
        c, s, plane = _plane(T, H, x.device, codes, scales)
    else:
        c, s, plane = None, None, Plane(None, 0, None, 0)
    amax_out = torch.empty(1, dtype=torch.float32, device=x.device)
    scale_out = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = workspace(x.device, _stream(x))
    st = lib.rmsnorm_nvfp4q(x.data_ptr(), dt, T, H, x.stride(0), gamma.data_ptr(), _ptr(beta),
                            float(weight_offset), float(eps), _ptr(y), y.stride(0) if y is not None else 0,
                            ctypes.byref(_global(amax, amax_out, scale_out)), ctypes.byref(plane),
                            _rounding(rounding) | (ONE_LAUNCH if one_launch else 0), ctypes.byref(Rng(seed, offset)),
                            ws.data_ptr(), ws.numel(), _stream(x))
    _check(st)
    return {"codes": c, "scales": s, "amax": amax_out, "scale": scale_out, "y": y}


def rmsnorm_nvfp4q_noalloc(x, gamma, beta=None, weight_offset=0.0, eps=1e-6, amax=None, rounding="rtne", seed=0,
                           offset=0, y_out=None, codes=None, scales=None, amax_out=None, scale_out=None,
                           one_launch=False):
    """rmsnorm_nvfp4q through the entry point that allocates nothing (the library's static workspace).

    Outputs are the caller's: pass y_out, codes / scales, amax_out / scale_out tensors to make the call
    allocate nothing on the Python side either (any left as None is allocated here, before the call).
    Returns dict(codes, scales, amax, scale, y).
    """
    import torch

    dt = _dtype_code(x)
    for p in (gamma, beta):
        if p is not None and (p.dtype != x.dtype or not p.is_contiguous()):
            raise ValueError("gamma and beta must be contiguous and of x's dtype")
    lib = load()
    T, H = x.shape
    c, s, plane = _plane(T, H, x.device, codes, scales)
    if amax_out is None:
        amax_out = torch.empty(1, dtype=torch.float32, device=x.device)
    if scale_out is None:
        scale_out = torch.empty(1, dtype=torch.float32, device=x.device)
    st = lib.rmsnorm_nvfp4q_noalloc(x.data_ptr(), dt, T, H, x.stride(0), gamma.data_ptr(), _ptr(beta),
                                    float(weight_offset), float(eps), _ptr(y_out),
                                    y_out.stride(0) if y_out is not None else 0,
                                    ctypes.byref(_global(amax, amax_out, scale_out)), ctypes.byref(plane),
                                    _rounding(rounding) | (ONE_LAUNCH if one_launch else 0),
                                    ctypes.byref(Rng(seed, offset)), _stream(x))
    _check(st)
    return {"codes": c, "scales": s, "amax": amax_out, "scale": scale_out, "y": y_out}


def nvfp4q_quantize_2d(x, amax=None, rounding="rtne", seed=0, offset=0, rowwise=True, colwise=True,
                       tile16=False):
    """Rowwise and columnwise planes of x [rows, cols] (bf16, fp16 or fp32) under one per-tensor scale.

    tile16: NVFP4Q_SCALE_16X16 (one block scale per 16 x 16 tile, shared by both planes).
    """
    import torch

    dt = _dtype_code(x)
    lib = load()
    R, C = x.shape
    rc = rs = cc = cs = None
    rp = Plane(None, 0, None, 0)
    cp = Plane(None, 0, None, 0)
    if rowwise:
        rc, rs, rp = _plane(R, C, x.device)
    if colwise:
        cc, cs, cp = _plane(C, R, x.device)
    amax_out = torch.empty(1, dtype=torch.float32, device=x.device)
    scale_out = torch.empty(1, dtype=torch.float32, device=x.device)
    ws = workspace(x.device, _stream(x))
    st = lib.nvfp4q_quantize_2d(x.data_ptr(), dt, R, C, x.stride(0), ctypes.byref(_global(amax, amax_out, scale_out)),
                                ctypes.byref(rp), ctypes.byref(cp),
                                _rounding(rounding) | (SCALE_16X16 if tile16 else 0),
                                ctypes.byref(Rng(seed, offset)), ws.data_ptr(), ws.numel(), _stream(x))
    _check(st)
    return {"row_codes": rc, "row_scales": rs, "col_codes": cc, "col_scales": cs, "amax": amax_out,
            "scale": scale_out}


def nvfp4q_quantize_2d_grouped(x, experts, amax=None, rounding="rtne", seed=0, offset=0, rowwise=True,
                               colwise=True, tile16=False):
    """nvfp4q_quantize_2d of `experts` weights stacked in x [experts * rows, cols] (bf16, fp16 or fp32), each
    under its own amax.

    amax: optional float32 CUDA tensor [experts]. Returns row_codes [experts * rows, ...], row_scales,
    col_codes [experts * cols, ...] (expert e's transposed plane in rows e * cols ..), col_scales, and
    amax / scale [experts].
    """
    import torch

    dt = _dtype_code(x)
    lib = load()
    ER, C = x.shape
    if experts < 1 or ER % experts != 0:
        raise ValueError("x must stack `experts` weights of equal row count")
    R = ER // experts
    rc = rs = cc = cs = None
    rp = Plane(None, 0, None, 0)
    cp = Plane(None, 0, None, 0)
    if rowwise:
        rc, rs, rp = _plane(ER, C, x.device)
    if colwise:
        cc, cs, cp = _plane(experts * C, R, x.device)
    amax_out = torch.empty(experts, dtype=torch.float32, device=x.device)
    scale_out = torch.empty(experts, dtype=torch.float32, device=x.device)
    ws = workspace(x.device, _stream(x))
    st = lib.nvfp4q_quantize_2d_grouped(x.data_ptr(), dt, experts, R, C, x.stride(0),
                                        ctypes.byref(_global(amax, amax_out, scale_out)), ctypes.byref(rp),
                                        ctypes.byref(cp), _rounding(rounding) | (SCALE_16X16 if tile16 else 0),
                                        ctypes.byref(Rng(seed, offset)), ws.data_ptr(), ws.numel(), _stream(x))
    _check(st)
    return {"row_codes": rc, "row_scales": rs, "col_codes": cc, "col_scales": cs, "amax": amax_out,
            "scale": scale_out}


def nvfp4q_qk_norm(q, k, q_weight, k_weight, head_dim, weight_offset=0.0, eps=1e-6):
    """Per-head RMSNorm of q [tokens, q_heads * head_dim] and k [tokens, k_heads * head_dim], in place.

    bf16, fp16 or fp32 (q, k and both weights of one dtype). Either of q and k (with its weight) may be
    None. Weights: [head_dim]. Returns (q, k).
    """
    ts = [t for t in (q, k) if t is not None]
    if not ts:
        raise ValueError("give q, k or both")
    dt = _dtype_code(ts[0])
    for t, w in ((q, q_weight), (k, k_weight)):
        if t is None:
            continue
        if _dtype_code(t) != dt:
            raise ValueError("q and k must share a dtype")
        if t.shape[1] % head_dim:
            raise ValueError("row length must be a multiple of head_dim")
        if w is None or w.dtype != t.dtype or w.numel() != head_dim or not w.is_contiguous():
            raise ValueError("weights must be contiguous vectors of head_dim elements of the input's dtype")
    if len(ts) == 2 and q.shape[0] != k.shape[0]:
        raise ValueError("q and k need the same number of tokens")
    lib = load()
    hq = q.shape[1] // head_dim if q is not None else 0
    hk = k.shape[1] // head_dim if k is not None else 0
    st = lib.nvfp4q_qk_norm(_ptr(q), _ptr(k), dt, ts[0].shape[0], hq, hk, head_dim,
                            q.stride(0) if q is not None else 0, k.stride(0) if k is not None else 0,
                            _ptr(q_weight) if q is not None else None, _ptr(k_weight) if k is not None else None,
                            float(weight_offset), float(eps), _stream(ts[0]))
    _check(st)
    return q, k


def nvfp4q_grouped(x, offsets, apply_rht=True, rht_mask=0, amax=None, rounding="sr", seed=0, offset=0,
                   codes=None, scales=None, fast_math=False, colwise=True, rowwise=False, row_amax=None,
                   row_codes=None, row_scales=None):
    """Per-group NVFP4 of x [total_rows, cols] (bf16, fp16 or fp32): the columnwise plane (optionally
    after the 16-point RHT) and/or the rowwise plane (no transform), one amax per
    group and plane.

    offsets: int32 CUDA tensor [G+1]. The columnwise plane is allocated for the largest
    padded length (total_rows + 15 G) unless given. fast_math: NVFP4Q_FAST_MATH (the
    transform's output is quantized without its bf16 round-through). row_amax: the
    rowwise plane's per-group amax (computed when None). Returns dict(codes, scales, amax,
    scale, poff) for the columnwise plane and row_codes, row_scales, row_amax, row_scale
    for the rowwise one (None where a plane is not asked for).
    """
    import torch

    dt = _dtype_code(x)
    if offsets.dtype != torch.int32 or not offsets.is_cuda or offsets.dim() != 1:
        raise ValueError("offsets must be a 1-D int32 CUDA tensor")
    if not colwise and not rowwise:
        raise ValueError("ask for at least one plane")
    lib = load()
    T, C = x.shape
    G = offsets.numel() - 1
    amax_out = scale_out = ramax_out = rscale_out = rc = rs = None
    plane = rplane = None
    if colwise:
        cap = T + 15 * G
        cap16 = (cap + 15) // 16 * 16
        if codes is None:
            codes = torch.empty((C, (cap16 // 2 + 15) // 16 * 16), dtype=torch.uint8, device=x.device)
        if scales is None:
            scales = torch.empty((C, cap16 // 16), dtype=torch.uint8, device=x.device)
        plane = Plane(codes.data_ptr(), codes.stride(0), scales.data_ptr(), scales.stride(0))
        amax_out = torch.empty(G, dtype=torch.float32, device=x.device)
        scale_out = torch.empty(G, dtype=torch.float32, device=x.device)
    else:
        codes = scales = None
    if rowwise:
        rc, rs, rplane = _plane(T, C, x.device, row_codes, row_scales)
        ramax_out = torch.empty(G, dtype=torch.float32, device=x.device)
        rscale_out = torch.empty(G, dtype=torch.float32, device=x.device)
    poff = torch.empty(G + 1, dtype=torch.int32, device=x.device)
    ws = workspace(x.device, _stream(x))
    gcol = _global(amax, amax_out, scale_out) if colwise else None
    grow = _global(row_amax, ramax_out, rscale_out) if rowwise else None
    st = lib.nvfp4q_grouped(x.data_ptr(), dt, T, C, x.stride(0), offsets.data_ptr(), G, poff.data_ptr(),
                            1 if apply_rht else 0, int(rht_mask),
                            ctypes.byref(gcol) if gcol is not None else None,
                            ctypes.byref(plane) if plane is not None else None,
                            ctypes.byref(grow) if grow is not None else None,
                            ctypes.byref(rplane) if rplane is not None else None,
                            _rounding(rounding) | (FAST_MATH if fast_math else 0),
                            ctypes.byref(Rng(seed, offset)),
                            ws.data_ptr(), ws.numel(), _stream(x))
    _check(st)
    return {"codes": codes, "scales": scales, "amax": amax_out, "scale": scale_out, "poff": poff,
            "row_codes": rc, "row_scales": rs, "row_amax": ramax_out, "row_scale": rscale_out}

"""Helpers shared by the GPU parity tests: host<->device moves and comparisons
against the oracle. Nothing here computes any step of the method."""
import numpy as np

import oracle
from oracle import formats as F


def to_dev(bits: np.ndarray):
    """uint16 bf16 bit array -> CUDA bfloat16 tensor."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_np_bf16(t) -> np.ndarray:
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def np_u8(t, cols=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a if cols is None else a[:, :cols]


def f32(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32)


def assert_same_bits(name, got: np.ndarray, want: np.ndarray):
    if got.shape != want.shape:
        raise AssertionError(f"{name}: shape {got.shape} != {want.shape}")
    bad = np.argwhere(got != want)
    if len(bad):
        idx = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} of {got.size} differ; first at {idx}: got {got[idx]:#x} "
                             f"want {want[idx]:#x}")


def assert_f32_bits(name, got, want):
    g = np.float32(got).view(np.uint32)
    w = np.float32(want).view(np.uint32)
    assert g == w, f"{name}: {np.float32(got)!r} ({int(g):#x}) != {np.float32(want)!r} ({int(w):#x})"


def code_step_mismatch(got_packed: np.ndarray, want_packed: np.ndarray):
    """(number of differing codes, all differences are <= 1 magnitude step with the same sign)."""
    a = F.unpack_nibbles(got_packed).astype(np.int64)
    b = F.unpack_nibbles(want_packed).astype(np.int64)
    diff = a != b
    n = int(diff.sum())
    if n == 0:
        return 0, True
    ma, mb = a[diff] & 7, b[diff] & 7
    sa, sb = a[diff] >> 3, b[diff] >> 3
    same_sign = (sa == sb) | (ma == 0) | (mb == 0)
    ok = bool(np.all((np.abs(ma - mb) <= 1) & same_sign))
    return n, ok

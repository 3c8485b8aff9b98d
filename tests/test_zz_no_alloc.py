"""The entry point that allocates nothing (rmsnorm_nvfp4q_noalloc, whose workspace is the library's static
device array) against rmsnorm_nvfp4q with a caller workspace, through the C ABI: identical outputs, on two
calls in a row, the second on a smaller input (the static array keeps the first call's contents)."""
import numpy as np
import pytest

import workloads
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


def _same(name, a, b):
    import torch

    if a is None and b is None:
        return
    assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b), name


def _compare(q, x, gamma, beta, **kw):
    import torch

    ref = q.rmsnorm_nvfp4q(x, gamma, beta, y_out=True, **kw)
    y = torch.empty_like(x)
    got = q.rmsnorm_nvfp4q_noalloc(x, gamma, beta, y_out=y, **kw)
    torch.cuda.synchronize()
    T, H = x.shape
    _same("codes", got["codes"][:, :H // 2], ref["codes"][:, :H // 2])
    _same("scales", got["scales"][:, :H // 16], ref["scales"][:, :H // 16])
    _same("amax", got["amax"], ref["amax"])
    _same("scale", got["scale"], ref["scale"])
    _same("y", got["y"], ref["y"])


def test_noalloc_matches_the_workspace_entry_point(gpu_lib):
    # first the prefill workload (amax pass storing per-row 1/rms in the workspace, then the streamed
    # encode), then the smaller decode workload with a bias (the cooperative-row amax pass) in SR, then a
    # given amax: each against the caller-workspace call on the same input
    w = workloads.prefill(seed=4)
    _compare(gpu_lib, to_dev(w.x), to_dev(w.gamma), None, eps=w.eps)
    d = workloads.decode(seed=5)
    _compare(gpu_lib, to_dev(d.x), to_dev(d.gamma), to_dev(d.beta), eps=d.eps, rounding="sr", seed=9, offset=3)
    import torch

    a = torch.tensor([3.5], dtype=torch.float32, device="cuda")
    _compare(gpu_lib, to_dev(d.x[:3]), to_dev(d.gamma), None, eps=d.eps, amax=a)


def test_noalloc_two_calls_second_smaller(gpu_lib):
    rng = np.random.default_rng(12)
    for T, H in ((2304, 2048), (5, 1040)):
        x = workloads.to_bf16_bits((rng.standard_normal((T, H)) * 3).astype(np.float32))
        g = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
        _compare(gpu_lib, to_dev(x), to_dev(g), None, eps=1e-6, weight_offset=1.0)


def test_noalloc_one_launch(gpu_lib):
    # NVFP4Q_ONE_LAUNCH on the static array (its state words start as zeros): the same outputs as the
    # caller-workspace call, twice, the second on fewer rows
    rng = np.random.default_rng(21)
    for T, H in ((64, 4096), (8, 7168)):
        x = workloads.to_bf16_bits((rng.standard_normal((T, H)) * 2).astype(np.float32))
        g = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
        _compare(gpu_lib, to_dev(x), to_dev(g), None, eps=1e-6, one_launch=True)

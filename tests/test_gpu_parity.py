"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Quantize-only paths (rowwise, 2D, grouped) must be bit-exact in codes, scales,
amax and S_dec. The fused RMSNorm path follows the rules of its contract: y
within 1e-2 relative (+2^-20 absolute) of the float64 oracle; the codes equal,
bit for bit, the oracle's quantization of the GPU's own bf16 y; against the
float64 oracle at most 1e-4 of the codes differ, each by at most one magnitude
step, and only in blocks whose rounded y differs. The norms' rounded outputs
(RMSNorm y in bf16 or fp16, QK norm) are, element by element, the
round-to-nearest-even of a value within the fp32 arithmetic's error bound of the
exact one, hence within one step of the oracle's output; fp32 outputs lie within
that bound. Full-size workloads are checked on sampled rows, columns or groups.
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle import formats as F
from tests.gpu_helpers import (REL_ERR_QK, REL_ERR_RMSNORM, assert_code_diffs_follow_y, assert_f32_bits,
                               assert_rounded_output, assert_same_bits, code_step_mismatch, f32, np_u8, to_dev,
                               to_np_bf16)

pytestmark = pytest.mark.gpu

SEEDS = [0, 1, 2, 224]


def test_gpu_library_was_built_from_these_sources(gpu_lib):
    """The library the GPU tests load was built from the sources of this tree (its embedded digest)."""
    from rmsnorm_nvfp4_block_amd import build

    assert gpu_lib.library_source_sha256() == build.source_digest(), "libnvfp4q.so is older than its sources"


def _bf16(rng, shape, scale=1.0):
    return workloads.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _check_rowwise(q, got, cols, name=""):
    assert_same_bits(name + " codes", np_u8(got["codes"], cols // 2), q["codes"])
    assert_same_bits(name + " scales", np_u8(got["scales"], cols // 16), q["scales"])
    assert_f32_bits(name + " amax", f32(got["amax"])[0], q["amax"])
    assert_f32_bits(name + " scale", f32(got["scale"])[0], q["s_dec"])


# ---------------------------------------------------------------- quantize
@pytest.mark.parametrize("seed", SEEDS)
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_quantize_256x1024(gpu_lib, seed, rounding):
    w = workloads.quantize_only(seed=seed)
    got = gpu_lib.nvfp4q_quantize(to_dev(w.x), rounding=rounding, seed=0x5EED, offset=seed)
    q = oracle.quantize_rowwise(w.x, rounding=rounding, seed=0x5EED, offset=seed)
    _check_rowwise(q, got, 1024)


@pytest.mark.parametrize("shape", [(1, 16), (3, 48), (37, 1040), (130, 2064), (5, 7168), (1000, 512), (2, 16400)])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_quantize_ragged(gpu_lib, shape, rounding):
    rng = np.random.default_rng(hash(shape) % 1000)
    x = _bf16(rng, shape, 3.0)
    got = gpu_lib.nvfp4q_quantize(to_dev(x), rounding=rounding, seed=77, offset=3)
    _check_rowwise(oracle.quantize_rowwise(x, rounding=rounding, seed=77, offset=3), got, shape[1])


def test_quantize_extremes(gpu_lib):
    # every finite bf16 value, including subnormals and the largest magnitudes
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(F.bf16_to_f32(bits))]
    bits = bits[: len(bits) // 16 * 16]
    rng = np.random.default_rng(5)
    x = rng.permutation(bits).reshape(-1, 256)
    for rounding in ("rtne", "sr"):
        got = gpu_lib.nvfp4q_quantize(to_dev(x), rounding=rounding, seed=9)
        _check_rowwise(oracle.quantize_rowwise(x, rounding=rounding, seed=9), got, 256, rounding)
    # one block per magnitude band: small blocks meet large global scales
    xs = (F.bf16_to_f32(x) * np.float32(1.0)).reshape(-1, 16)
    order = np.argsort(np.abs(xs).max(1))
    x2 = F.f32_to_bf16(xs[order]).reshape(-1, 256)
    got = gpu_lib.nvfp4q_quantize(to_dev(x2))
    _check_rowwise(oracle.quantize_rowwise(x2), got, 256, "sorted")


@pytest.mark.parametrize("amax", [2688.0, 1.0, 0.37, 1e-30, 1e-38, 3e38])
def test_quantize_given_amax(gpu_lib, amax):
    import torch

    rng = np.random.default_rng(6)
    x = _bf16(rng, (64, 256), 2.0)
    a = torch.tensor([amax], dtype=torch.float32, device="cuda")
    for rounding in ("rtne", "sr"):
        got = gpu_lib.nvfp4q_quantize(to_dev(x), amax=a, rounding=rounding, seed=1)
        q = oracle.quantize_rowwise(x, amax=np.float32(amax), rounding=rounding, seed=1)
        _check_rowwise(q, got, 256, f"amax={amax} {rounding}")


def test_quantize_zero_and_empty(gpu_lib):
    import torch

    x = np.zeros((4, 64), np.uint16)
    got = gpu_lib.nvfp4q_quantize(to_dev(x))
    _check_rowwise(oracle.quantize_rowwise(x), got, 64, "zeros")
    e = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    got = gpu_lib.nvfp4q_quantize(e)
    assert f32(got["amax"])[0] == 0.0 and f32(got["scale"])[0] == 1.0


def test_empty_inputs_on_every_path(gpu_lib):
    # no rows: every entry point reports amax 0 and S_dec 1 (per tensor, group or expert) and writes nothing
    import torch

    e = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    got = gpu_lib.rmsnorm_nvfp4q(e, g)
    assert f32(got["amax"])[0] == 0.0 and f32(got["scale"])[0] == 1.0
    got = gpu_lib.nvfp4q_quantize_2d(e, rounding="sr", seed=1)
    assert f32(got["amax"])[0] == 0.0 and f32(got["scale"])[0] == 1.0
    got = gpu_lib.nvfp4q_quantize_2d_grouped(e, 3)
    assert np.all(f32(got["amax"]) == 0.0) and np.all(f32(got["scale"]) == 1.0)
    offs = torch.zeros(5, dtype=torch.int32, device="cuda")
    codes = torch.full((64, 32), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full((64, 4), 0x55, dtype=torch.uint8, device="cuda")
    got = gpu_lib.nvfp4q_grouped(e, offs, rounding="sr", seed=1, codes=codes, scales=scales, rowwise=True)
    assert np.all(f32(got["amax"]) == 0.0) and np.all(f32(got["scale"]) == 1.0)
    assert np.all(f32(got["row_amax"]) == 0.0) and np.all(f32(got["row_scale"]) == 1.0)
    assert np.all(got["poff"].cpu().numpy() == 0)
    assert np.all(np_u8(codes) == 0xAA) and np.all(np_u8(scales) == 0x55)
    gpu_lib.nvfp4q_qk_norm(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda"), None,
                           torch.ones(128, dtype=torch.bfloat16, device="cuda"), None, 128)


def test_golden_blocks(gpu_lib):
    import json, os, torch

    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_blocks.json")))["cases"]
    for c in cases:
        x = F.f32_to_bf16(np.array(c["x"], np.float32)).reshape(1, 16)
        a = None if c["amax_in"] is None else torch.tensor([c["amax_in"]], dtype=torch.float32, device="cuda")
        got = gpu_lib.nvfp4q_quantize(to_dev(x), amax=a)
        assert np_u8(got["codes"], 8).tolist()[0] == c["bytes"], c["name"]
        assert int(np_u8(got["scales"], 1)[0, 0]) == c["scale"], c["name"]
        assert int(f32(got["scale"]).view(np.uint32)[0]) == c["s_dec_bits"], c["name"]


def test_repeated_calls_share_the_workspace(gpu_lib):
    rng = np.random.default_rng(7)
    xs = [_bf16(rng, (97, 528), s) for s in (1.0, 100.0, 0.01)]
    for _ in range(2):
        for x in xs:
            got = gpu_lib.nvfp4q_quantize(to_dev(x))
            _check_rowwise(oracle.quantize_rowwise(x), got, 528)


def test_graph_capture_replays(gpu_lib):
    import ctypes, torch
    q = gpu_lib
    rng = np.random.default_rng(8)
    x1, x2 = _bf16(rng, (128, 1024)), _bf16(rng, (128, 1024), 7.0)
    xd = to_dev(x1)
    codes = torch.empty((128, 512), dtype=torch.uint8, device="cuda")
    scales = torch.empty((128, 64), dtype=torch.uint8, device="cuda")
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    q.nvfp4q_quantize(xd, codes=codes, scales=scales)   # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            out = q.nvfp4q_quantize(xd, codes=codes, scales=scales)
    for rep, x in enumerate([x1, x2, x1, x2]):
        xd.copy_(to_dev(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.quantize_rowwise(x)
        assert_same_bits(f"replay {rep} codes", np_u8(codes), ref["codes"])
        assert_same_bits(f"replay {rep} scales", np_u8(scales), ref["scales"])
        assert_f32_bits(f"replay {rep} amax", f32(out["amax"])[0], ref["amax"])
        # eager work between replays
        e = q.nvfp4q_quantize(to_dev(x2))
        _check_rowwise(oracle.quantize_rowwise(x2), e, 1024, "eager")


def test_graph_capture_replays_other_entry_points(gpu_lib):
    # grouped (both planes, RHT, SR), stacked expert weights with tile scales, and the in-place QK norm,
    # each captured once and replayed on changing inputs, with eager calls between the replays; every
    # replay must equal an eager call on the same input
    import torch
    q = gpu_lib
    rng = np.random.default_rng(40)
    offs = torch.tensor([0, 5, 70, 70, 160], dtype=torch.int32, device="cuda")
    xs = [_bf16(rng, (160, 272), sc) for sc in (1.0, 9.0, 0.01)]
    ws = [np.concatenate([_bf16(rng, (48, 80), sc) for _ in range(3)]) for sc in (0.02, 3.0, 1e-3)]
    qs = [_bf16(rng, (9, 4 * 128), sc) for sc in (1.0, 50.0, 0.1)]
    wq = to_dev(workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(128)).astype(np.float32)))
    xg, xw, xq = to_dev(xs[0]), to_dev(ws[0]), to_dev(qs[0])

    def grouped(x):
        return q.nvfp4q_grouped(x, offs, apply_rht=True, rht_mask=0x6B1D, rounding="sr", seed=4, rowwise=True)

    def experts(x):
        return q.nvfp4q_quantize_2d_grouped(x, 3, rounding="sr", seed=5, tile16=True)

    grouped(xg), experts(xw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            og = grouped(xg)
            oe = experts(xw)
            q.nvfp4q_qk_norm(xq, None, wq, None, 128)
    for rep in range(4):
        i = rep % 3
        xg.copy_(to_dev(xs[i]))
        xw.copy_(to_dev(ws[i]))
        xq.copy_(to_dev(qs[i]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rg, re = grouped(to_dev(xs[i])), experts(to_dev(ws[i]))
        rq = to_dev(qs[i])
        q.nvfp4q_qk_norm(rq, None, wq, None, 128)
        torch.cuda.synchronize()
        mp = int(rg["poff"][-1])
        # planes compared over their written bytes (row padding of the allocations is never written)
        assert torch.equal(og["row_codes"][:, :136], rg["row_codes"][:, :136]), f"replay {rep}: grouped row codes"
        for k in ("row_scales", "amax", "row_amax", "poff"):
            assert torch.equal(og[k], rg[k]), f"replay {rep}: grouped {k}"
        assert torch.equal(og["codes"][:, :mp // 2], rg["codes"][:, :mp // 2]), f"replay {rep}: grouped codes"
        assert torch.equal(og["scales"][:, :mp // 16], rg["scales"][:, :mp // 16]), f"replay {rep}: grouped scales"
        for k, n in (("row_codes", 40), ("row_scales", 5), ("col_codes", 24), ("col_scales", 3), ("amax", 3)):
            assert torch.equal(oe[k][..., :n], re[k][..., :n]), f"replay {rep}: experts {k}"
        assert torch.equal(xq.view(torch.int16), rq.view(torch.int16)), f"replay {rep}: qk norm"


# ---------------------------------------------------------------- RMSNorm
def _check_rms(w, got, rounding="rtne", seed=0, offset=0, amax_given=None):
    """Contract rules for the fused path (see module docstring)."""
    cols = w.cols
    y_gpu = to_np_bf16(got["y"])
    y_ref, y64, _ = oracle.rmsnorm_bf16(w.x, w.gamma, w.beta, w.weight_offset, w.eps, return_f64=True)
    yg = F.bf16_to_f32(y_gpu).astype(np.float64)
    err = np.abs(yg - y64)
    assert np.all(err <= 1e-2 * np.abs(y64) + 2.0 ** -20), f"y error max {err.max()}"
    # y is the bf16 rounding of a value within the fp32 arithmetic's error bound of the exact one
    b64 = None if w.beta is None else F.bf16_to_f32(w.beta).astype(np.float64)[None, :]
    assert_rounded_output("y", y_gpu, y_ref, y64, "bf16", REL_ERR_RMSNORM, b64)
    # codes are the exact quantization of the GPU's own y
    amax = amax_given if amax_given is not None else np.float32(np.max(np.abs(yg)))
    q_own = oracle.quantize_rowwise(y_gpu, amax=amax, rounding=rounding, seed=seed, offset=offset)
    _check_rowwise(q_own, got, cols, "quantize(y_gpu)")
    # against the float64 oracle
    q_ref = oracle.quantize_rowwise(y_ref, amax=amax_given, rounding=rounding, seed=seed, offset=offset)
    n, ok = code_step_mismatch(np_u8(got["codes"], cols // 2), q_ref["codes"])
    assert ok, "a code differs by more than one step"
    assert n <= 1e-4 * w.rows * cols, f"{n} codes differ from the float64 oracle"
    assert_code_diffs_follow_y("codes", np_u8(got["codes"], cols // 2), q_ref["codes"], y_gpu, y_ref, amax,
                               q_ref["amax"])
    return n


@pytest.mark.parametrize("seed", [3, 224])
def test_rmsnorm_decode_8x7168(gpu_lib, seed):
    w = workloads.decode(seed=seed)
    got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), to_dev(w.beta), eps=w.eps, y_out=True)
    _check_rms(w, got)


def _one_launch_state(gpu_lib):
    """(calls completed, a wait gave up) of the workspace's one-launch state words (its first two int32)."""
    import torch

    st = gpu_lib.workspace()[:8].view(torch.int32).cpu().numpy()
    return int(st[0]), int(st[1])


@pytest.mark.parametrize("shape,bias,woff,rounding", [((1, 16), False, 0.0, "rtne"), ((8, 7168), True, 0.0, "sr"),
                                                      ((17, 4112), True, 1.0, "rtne"), ((64, 16384), False, 0.0, "sr"),
                                                      ((64, 1040), True, 0.0, "rtne"), ((63, 8192), False, 1.0, "rtne")])
def test_rmsnorm_one_launch_rows(gpu_lib, shape, bias, woff, rounding):
    """NVFP4Q_ONE_LAUNCH with at most 64 rows and no given amax: one launch whose workgroups meet on the amax
    inside it. Parity as for the two passes; the workspace's one-launch counter advances by one per call and
    no wait gave up."""
    rng = np.random.default_rng(sum(shape))
    T, H = shape
    w = workloads.Workload("t", _bf16(rng, shape, 1.3), gamma=_bf16(rng, (H,), 0.4),
                           beta=_bf16(rng, (H,), 0.1) if bias else None, weight_offset=woff, eps=1e-6)
    e0, _ = _one_launch_state(gpu_lib)
    got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), to_dev(w.beta) if bias else None,
                                 weight_offset=woff, eps=w.eps, y_out=True, rounding=rounding, seed=7, offset=1,
                                 one_launch=True)
    _check_rms(w, got, rounding, 7, 1)
    e1, err = _one_launch_state(gpu_lib)
    assert err == 0 and e1 == e0 + 1


@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("shape,bias,woff,rounding", [((8, 7168), True, 0.0, "sr"), ((37, 1040), False, 1.0, "rtne"),
                                                      ((5, 16384), True, 1.0, "sr")])
def test_rmsnorm_one_launch_fp16_fp32(gpu_lib, dtype, shape, bias, woff, rounding):
    """NVFP4Q_ONE_LAUNCH with fp16 and fp32 input: the fp16/fp32 contract rules (reading R-dtype)."""
    e0, _ = _one_launch_state(gpu_lib)
    test_rmsnorm_fp16_fp32_inputs(gpu_lib, dtype, shape, bias, woff, rounding, one_launch=True)
    e1, err = _one_launch_state(gpu_lib)
    assert err == 0 and e1 == e0 + 1


def test_rmsnorm_one_launch_equals_given_amax_pass(gpu_lib):
    """The one-launch result equals the single-pass encode given the amax it found, and the two-pass result:
    same y, codes and scales bit for bit (all normalize a row the same way; only where the amax comes from
    differs)."""
    import torch

    w = workloads.decode(seed=11)
    x, g, b = to_dev(w.x), to_dev(w.gamma), to_dev(w.beta)
    one = gpu_lib.rmsnorm_nvfp4q(x, g, b, eps=w.eps, y_out=True, rounding="sr", seed=3, offset=4, one_launch=True)
    passes = gpu_lib.rmsnorm_nvfp4q(x, g, b, eps=w.eps, y_out=True, rounding="sr", seed=3, offset=4)
    two = gpu_lib.rmsnorm_nvfp4q(x, g, b, eps=w.eps, y_out=True, rounding="sr", seed=3, offset=4,
                                 amax=one["amax"].clone())
    torch.cuda.synchronize()
    for k in ("y", "codes", "scales", "amax", "scale"):
        assert torch.equal(one[k].view(torch.uint8), two[k].view(torch.uint8)), k
        assert torch.equal(one[k].view(torch.uint8), passes[k].view(torch.uint8)), k


def test_rmsnorm_one_launch_between_other_calls(gpu_lib):
    """The one-launch state survives other entry points on the same workspace, and grids of different sizes
    follow each other (64, 5, 64 workgroups: slots a smaller grid left stale are waited for, not trusted)."""
    for k, rows in enumerate([64, 5, 64]):
        rng = np.random.default_rng(100 + k)
        w = workloads.Workload("t", _bf16(rng, (rows, 2048), 1.0), gamma=_bf16(rng, (2048,), 0.5), eps=1e-6)
        got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), eps=w.eps, y_out=True, one_launch=True)
        _check_rms(w, got)
        # other entry points write their partial maxima into the same workspace
        gpu_lib.nvfp4q_quantize_2d(to_dev(_bf16(rng, (1024, 2048), 2.0)))
        gpu_lib.rmsnorm_nvfp4q(to_dev(_bf16(rng, (300, 2048), 1.0)), to_dev(w.gamma), eps=1e-6)
    assert _one_launch_state(gpu_lib)[1] == 0


@pytest.mark.parametrize("seed", [2, 224])
def test_rmsnorm_prefill_4096x4096(gpu_lib, seed):
    w = workloads.prefill(seed=seed)
    got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), eps=w.eps, y_out=True)
    _check_rms(w, got)


@pytest.mark.parametrize("shape,bias,woff", [((5, 1040), True, 1.0), ((64, 16), False, 0.0), ((3, 16384), True, 0.0),
                                             ((33, 4096), False, 1.0), ((1, 7168), True, 0.0),
                                             ((300, 2560), True, 0.0)])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_rmsnorm_ragged(gpu_lib, shape, bias, woff, rounding):
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    T, H = shape
    w = workloads.Workload("t", _bf16(rng, shape, 2.0), gamma=_bf16(rng, (H,), 0.3),
                           beta=_bf16(rng, (H,), 0.05) if bias else None, weight_offset=woff, eps=1e-5)
    got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), to_dev(w.beta) if bias else None,
                                 weight_offset=woff, eps=w.eps, y_out=True, rounding=rounding, seed=11, offset=1)
    _check_rms(w, got, rounding, 11, 1)


@pytest.mark.parametrize("shape,bias,woff,rounding", [((3, 32768), False, 0.0, "rtne"), ((5, 20000), True, 1.0, "sr"),
                                                      ((2, 16400), True, 0.0, "rtne"), ((70, 18432), False, 0.0, "sr")])
def test_rmsnorm_wide_rows(gpu_lib, shape, bias, woff, rounding):
    """Rows of 16384 < hidden <= 32768: cooperative-row passes with eight superchunks per wave and gamma and
    beta read where they are used (also for a row count the streaming passes would take)."""
    import torch

    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    T, H = shape
    w = workloads.Workload("t", _bf16(rng, shape, 2.0), gamma=_bf16(rng, (H,), 0.3),
                           beta=_bf16(rng, (H,), 0.05) if bias else None, weight_offset=woff, eps=1e-5)
    args = (to_dev(w.x), to_dev(w.gamma), to_dev(w.beta) if bias else None)
    kw = dict(weight_offset=woff, eps=w.eps, y_out=True, rounding=rounding, seed=11, offset=1)
    got = gpu_lib.rmsnorm_nvfp4q(*args, **kw)
    _check_rms(w, got, rounding, 11, 1)
    valid = {"y": None, "codes": H // 2, "scales": H // 16, "amax": None, "scale": None}  # bytes past: padding
    u8 = lambda r, k: np_u8(r[k].view(torch.uint8), valid[k])
    # the one-launch option does not apply to rows this wide: the same two passes run
    one = gpu_lib.rmsnorm_nvfp4q(*args, one_launch=True, **kw)
    for k in valid:
        assert np.array_equal(u8(one, k), u8(got, k)), k
    # given the amax it found, the single-pass encode gives the same y, codes and scales
    giv = gpu_lib.rmsnorm_nvfp4q(*args, amax=got["amax"].clone(), **kw)
    for k in ("y", "codes", "scales"):
        assert np.array_equal(u8(giv, k), u8(got, k)), k


def test_rmsnorm_wide_rows_fp16(gpu_lib):
    """fp16 rows of 24576 with a bias, against the oracle in fp16 (reading R-dtype)."""
    test_rmsnorm_fp16_fp32_inputs(gpu_lib, "float16", (3, 24576), True, 0.0, "sr")


@pytest.mark.parametrize("shape,bias,woff,rounding", [((24579, 32), False, 0.0, "rtne"), ((8197, 1040), True, 1.0, "sr"),
                                                      ((8197, 1040), False, 1.0, "rtne")])
def test_rmsnorm_many_rows_per_wave(gpu_lib, shape, bias, woff, rounding):
    """Several rows per wave: the streaming passes refill their ring across rows."""
    rng = np.random.default_rng(shape[0] + shape[1])
    H = shape[1]
    w = workloads.Workload("t", _bf16(rng, shape, 1.5), gamma=_bf16(rng, (H,), 0.4),
                           beta=_bf16(rng, (H,), 0.1) if bias else None, weight_offset=woff, eps=1e-6)
    got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), to_dev(w.beta) if bias else None,
                                 weight_offset=woff, eps=w.eps, y_out=True, rounding=rounding, seed=5, offset=2)
    _check_rms(w, got, rounding, 5, 2)


def test_rmsnorm_rows_past_row_scale_slots(gpu_lib):
    """More rows than the workspace keeps per-row 1/rms for: the full-row passes."""
    rng = np.random.default_rng(77)
    shape = (258017, 16)
    w = workloads.Workload("t", _bf16(rng, shape, 1.0), gamma=_bf16(rng, (16,), 0.5), eps=1e-6)
    got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), eps=w.eps, y_out=True)
    _check_rms(w, got)


def test_rmsnorm_prefill_given_amax(gpu_lib):
    """Prefill size with a precomputed amax: the single-pass encode."""
    import torch

    w = workloads.prefill(seed=7)
    q = oracle.rmsnorm_quantize(w.x, w.gamma, None, 0.0, w.eps)
    a = torch.tensor([q["amax"]], dtype=torch.float32, device="cuda")
    got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), eps=w.eps, amax=a, y_out=True)
    _check_rms(w, got, amax_given=np.float32(q["amax"]))


@pytest.mark.parametrize("shape,dtype,bias,woff,rounding", [((2048, 4096), "bf16", False, 0.0, "rtne"),
                                                            ((2304, 3088), "bf16", True, 1.0, "sr"),
                                                            ((2050, 8192), "fp16", False, 0.0, "rtne"),
                                                            ((2100, 7184), "bf16", True, 0.0, "sr"),
                                                            ((2048, 4096), "fp32", False, 1.0, "rtne"),
                                                            ((4100, 4096), "bf16", False, 0.0, "sr")])
def test_rmsnorm_given_amax_large(gpu_lib, shape, dtype, bias, woff, rounding):
    """A given amax (one pass over x, each row's 1/rms taken in the same pass) on prefill-sized inputs:
    ragged last superchunks, rows of up to 8192 columns, several rows per workgroup, all input types."""
    import torch

    T, H = shape
    rng = np.random.default_rng(T * 3 + H)
    x32 = (rng.standard_normal(shape) * np.exp(rng.uniform(-2, 2, (T, 1)))).astype(np.float32)
    g32 = (1 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    b32 = (0.01 * rng.standard_normal(H)).astype(np.float32) if bias else None
    if dtype == "bf16":
        conv = lambda a: None if a is None else workloads.to_bf16_bits(a)
        dev = lambda a: None if a is None else to_dev(a)
    else:
        ndt = np.float16 if dtype == "fp16" else np.float32
        conv = lambda a: None if a is None else a.astype(ndt)
        dev = lambda a: None if a is None else torch.from_numpy(a).cuda()
    x, g, b = conv(x32), conv(g32), conv(b32)
    y_ref, y64, _ = oracle.rmsnorm_bf16(x, g, b, woff, 1e-6, return_f64=True, out_dtype=dtype)
    ref = oracle.quantize_rowwise(y_ref, rounding=rounding, seed=3, offset=1)
    a = torch.tensor([ref["amax"]], dtype=torch.float32, device="cuda")
    got = gpu_lib.rmsnorm_nvfp4q(dev(x), dev(g), dev(b), weight_offset=woff, eps=1e-6, amax=a, rounding=rounding,
                                 seed=3, offset=1, y_out=True)
    yg = to_np_bf16(got["y"]) if dtype == "bf16" else got["y"].cpu().numpy()
    b64 = None
    if b is not None:
        b64 = (F.bf16_to_f32(b) if dtype == "bf16" else b.astype(np.float32)).astype(np.float64)[None, :]
    assert_rounded_output("y", yg, y_ref, y64, dtype, REL_ERR_RMSNORM, b64)
    own = oracle.quantize_rowwise(yg, amax=np.float32(ref["amax"]), rounding=rounding, seed=3, offset=1)
    assert_same_bits("codes (own y)", np_u8(got["codes"], H // 2), own["codes"])
    assert_same_bits("scales (own y)", np_u8(got["scales"], H // 16), own["scales"])
    n, ok = code_step_mismatch(np_u8(got["codes"], H // 2), ref["codes"])
    assert ok and n <= 1e-4 * T * H, f"{n} codes differ from the float64 oracle"
    assert_code_diffs_follow_y("codes", np_u8(got["codes"], H // 2), ref["codes"], yg, y_ref, ref["amax"],
                               ref["amax"])


def test_rmsnorm_given_amax_and_y_only(gpu_lib):
    import torch

    w = workloads.decode(seed=9)
    q = oracle.rmsnorm_quantize(w.x, w.gamma, w.beta, 0.0, w.eps)
    a = torch.tensor([q["amax"]], dtype=torch.float32, device="cuda")
    got = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), to_dev(w.beta), eps=w.eps, amax=a, y_out=True)
    _check_rms(w, got, amax_given=np.float32(q["amax"]))
    y_only = gpu_lib.rmsnorm_nvfp4q(to_dev(w.x), to_dev(w.gamma), to_dev(w.beta), eps=w.eps, y_out=True,
                                    quantize=False)
    assert np.array_equal(to_np_bf16(y_only["y"]), to_np_bf16(got["y"]))


# The norm's codes without y output come from a separate compile-time branch of every RMSNorm encode (y is
# rounded there without being packed for a store); they must equal, bit for bit, the codes of the same call
# with y, which the tests above check against the oracle.
@pytest.mark.parametrize("rows,cols,bias,dtype,rounding,given,one", [
    (4096, 4096, False, "bfloat16", "rtne", False, False),  # streaming passes, one row per wave
    (4096, 4096, False, "bfloat16", "rtne", True, False),   # cooperative rows, given amax
    (2048, 8192, False, "bfloat16", "sr", True, False),     # cooperative rows, two superchunks per wave
    (2304, 5120, True, "bfloat16", "sr", False, False),     # bias amax pass, row-per-wave encode
    (300, 2560, True, "bfloat16", "rtne", False, False),    # few rows: superchunk-column encode
    (8, 7168, True, "bfloat16", "rtne", False, True),       # one launch
    (64, 20480, True, "bfloat16", "rtne", False, False),    # wide rows (parameters read where used)
    (2048, 4096, False, "float16", "sr", False, False),
    (1024, 3072, True, "float32", "rtne", True, False),
])
def test_rmsnorm_codes_without_y(gpu_lib, rows, cols, bias, dtype, rounding, given, one):
    import torch

    rng = np.random.default_rng(rows + cols)
    tdt = getattr(torch, dtype)
    x = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32)).to(tdt).cuda()
    g = torch.from_numpy((1 + 0.1 * rng.standard_normal(cols)).astype(np.float32)).to(tdt).cuda()
    b = torch.from_numpy((0.01 * rng.standard_normal(cols)).astype(np.float32)).to(tdt).cuda() if bias else None
    kw = dict(eps=1e-6, rounding=rounding, seed=5, offset=3, one_launch=one)
    with_y = gpu_lib.rmsnorm_nvfp4q(x, g, b, y_out=True, **kw)
    if given:
        kw["amax"] = with_y["amax"].clone()
        with_y = gpu_lib.rmsnorm_nvfp4q(x, g, b, y_out=True, **kw)
    no_y = gpu_lib.rmsnorm_nvfp4q(x, g, b, **kw)
    assert torch.equal(no_y["codes"][:, : cols // 2], with_y["codes"][:, : cols // 2]), "codes differ with and without y"
    assert torch.equal(no_y["scales"][:, : cols // 16], with_y["scales"][:, : cols // 16]), "scales differ"
    for k in ("amax", "scale"):
        assert torch.equal(no_y[k], with_y[k]), f"{k} differs between the calls with and without y"


# ---------------------------------------------------------------- fp16 / fp32 inputs
@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("shape", [(1, 16), (37, 272), (256, 1024), (5, 9232)])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_quantize_fp16_fp32_inputs(gpu_lib, dtype, shape, rounding):
    import torch

    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-4, 4, (shape[0], 1)))).astype(np.float32)
    x = x.astype(getattr(np, dtype))
    got = gpu_lib.nvfp4q_quantize(torch.from_numpy(x).cuda(), rounding=rounding, seed=0xD7, offset=3)
    q = oracle.quantize_rowwise(x, rounding=rounding, seed=0xD7, offset=3)
    R, C = shape
    assert_same_bits("codes", np_u8(got["codes"], C // 2), q["codes"])
    assert_same_bits("scales", np_u8(got["scales"], C // 16), q["scales"])
    assert_f32_bits("amax", f32(got["amax"])[0], q["amax"])
    assert_f32_bits("scale", f32(got["scale"])[0], q["s_dec"])


def test_quantize_fp32_given_amax_and_padded_rows(gpu_lib):
    import torch

    rng = np.random.default_rng(38)
    x = rng.standard_normal((64, 200)).astype(np.float32)
    xd = torch.from_numpy(x).cuda()[:, :192]           # rows of 200 floats (800 bytes, 16-byte aligned)
    a = torch.tensor([1.5], dtype=torch.float32, device="cuda")
    got = gpu_lib.nvfp4q_quantize(xd, amax=a, rounding="sr", seed=5)
    q = oracle.quantize_rowwise(x[:, :192], amax=np.float32(1.5), rounding="sr", seed=5)
    assert_same_bits("codes", np_u8(got["codes"], 96), q["codes"])
    assert_same_bits("scales", np_u8(got["scales"], 12), q["scales"])


@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("shape,bias,woff,rounding", [((8, 7168), True, 0.0, "rtne"), ((37, 1040), False, 1.0, "sr"),
                                                      ((300, 4096), True, 1.0, "sr"), ((5, 16384), False, 0.0, "rtne"),
                                                      ((2304, 1040), False, 0.0, "rtne"), ((2080, 2048), True, 1.0, "sr"),
                                                      ((2048, 2048), False, 0.0, "sr")])
def test_rmsnorm_fp16_fp32_inputs(gpu_lib, dtype, shape, bias, woff, rounding, one_launch=False):
    # reading R-dtype: gamma, beta and y in the input's type; y within the arithmetic tolerance of the
    # float64 value, codes the exact quantization of the GPU's own y, and almost all codes equal to the
    # quantization of the oracle's y
    import torch

    T, H = shape
    rng = np.random.default_rng(T + H)
    ndt = getattr(np, dtype)
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-3, 3, (T, 1)))).astype(ndt)
    g = (1 + 0.1 * rng.standard_normal(H)).astype(ndt)
    b = (0.01 * rng.standard_normal(H)).astype(ndt) if bias else None
    tdev = lambda a: torch.from_numpy(a).cuda()
    got = gpu_lib.rmsnorm_nvfp4q(tdev(x), tdev(g), tdev(b) if bias else None, weight_offset=woff, eps=1e-6,
                                 rounding=rounding, seed=11, offset=2, y_out=True, one_launch=one_launch)
    od = "fp16" if dtype == "float16" else "fp32"
    y_ref, y64, _ = oracle.rmsnorm_bf16(x, g, b, woff, 1e-6, return_f64=True, out_dtype=od)
    yg = got["y"].cpu().numpy()
    assert yg.dtype == ndt
    b64 = None if b is None else b.astype(np.float64)[None, :]
    assert_rounded_output("y", yg, y_ref, y64, od, REL_ERR_RMSNORM, b64)
    amax = np.float32(np.max(np.abs(yg.astype(np.float32))))
    assert_f32_bits("amax", f32(got["amax"])[0], amax)
    own = oracle.quantize_rowwise(yg, amax=amax, rounding=rounding, seed=11, offset=2)
    assert_same_bits("codes (own y)", np_u8(got["codes"], H // 2), own["codes"])
    assert_same_bits("scales (own y)", np_u8(got["scales"], H // 16), own["scales"])
    ref = oracle.quantize_rowwise(y_ref, rounding=rounding, seed=11, offset=2)
    n, ok = code_step_mismatch(np_u8(got["codes"], H // 2), ref["codes"])
    assert ok and n <= 1e-4 * T * H, f"{n} codes differ from the float64 oracle"
    assert_code_diffs_follow_y("codes", np_u8(got["codes"], H // 2), ref["codes"], yg, y_ref, amax, ref["amax"])


@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("head_dim", [64, 256])
@pytest.mark.parametrize("woff", [0.0, 1.0])
def test_qk_norm_fp16_fp32(gpu_lib, dtype, head_dim, woff):
    # reading R-dtype: the oracle's QK norm in the input's type; fp16 output within one step of the
    # oracle's rounding (and a rounding of a value within the fp32 arithmetic's bound), fp32 within that
    # bound of the exact value
    import torch

    w = workloads.qk_heads(seed=head_dim, tokens=33, q_heads=6, k_heads=2, head_dim=head_dim)
    tdt = getattr(torch, dtype)
    qf, kf = F.bf16_to_f32(w.x), F.bf16_to_f32(w.meta["k"])
    rng = np.random.default_rng(head_dim)
    qf = qf * (1 + 2.0 ** -9 * rng.standard_normal(qf.shape)).astype(np.float32)   # not bf16-exact
    qd, kd = torch.from_numpy(qf).to(tdt).cuda(), torch.from_numpy(kf).to(tdt).cuda()
    wq = torch.from_numpy(F.bf16_to_f32(w.gamma)).to(tdt).cuda()
    wk = torch.from_numpy(F.bf16_to_f32(w.meta["k_weight"])).to(tdt).cuda()
    q_in, k_in = qd.cpu().numpy(), kd.cpu().numpy()          # exactly the values the kernel reads
    wq_in, wk_in = wq.cpu().numpy(), wk.cpu().numpy()
    gpu_lib.nvfp4q_qk_norm(qd, kd, wq, wk, head_dim, weight_offset=woff, eps=w.eps)
    yq_ref, yk_ref = oracle.qk_norm(q_in, k_in, wq_in, wk_in, head_dim, weight_offset=woff, eps=w.eps)
    od = "fp16" if dtype == "float16" else "fp32"
    for name, got, ref, x_in, wv in (("q", qd, yq_ref, q_in, wq_in), ("k", kd, yk_ref, k_in, wk_in)):
        _, y64, _ = oracle.rmsnorm_bf16(x_in.reshape(-1, head_dim), wv, None, woff, w.eps, return_f64=True,
                                        out_dtype=od)
        yg = got.cpu().numpy().reshape(-1, head_dim)
        assert_rounded_output(name, yg, ref.reshape(-1, head_dim), y64, od, REL_ERR_QK)


# ---------------------------------------------------------------- QK norm (reading R-qk)
def _check_qk(y_gpu, x, w, head_dim, woff, eps):
    """bf16 QK norm: within 1e-2 of the exact value, and the bf16 rounding of a value within the fp32
    arithmetic's error bound, so within one bf16 step of the oracle's output."""
    _, y64, _ = oracle.rmsnorm_bf16(x.reshape(-1, head_dim), w, None, woff, eps, return_f64=True)
    yg = F.bf16_to_f32(y_gpu).astype(np.float64).reshape(-1, head_dim)
    err = np.abs(yg - y64)
    assert np.all(err <= 1e-2 * np.abs(y64) + 2.0 ** -20), f"QK norm error max {err.max()}"
    ref, _ = oracle.qk_norm(x, None, w, None, head_dim, woff, eps)
    assert ref.shape == x.shape
    assert_rounded_output("qk", np.asarray(y_gpu).reshape(-1, head_dim), ref.reshape(-1, head_dim), y64, "bf16",
                          REL_ERR_QK)


@pytest.mark.parametrize("head_dim", [64, 128, 256])
@pytest.mark.parametrize("tokens,hq,hk", [(1, 4, 0), (7, 5, 3), (129, 32, 8), (3, 0, 2)])
@pytest.mark.parametrize("woff", [0.0, 1.0])
def test_qk_norm_small(gpu_lib, head_dim, tokens, hq, hk, woff):
    import torch

    rng = np.random.default_rng(head_dim + 10 * tokens + hq)
    w = workloads.qk_heads(seed=int(rng.integers(1 << 20)), tokens=tokens, q_heads=max(hq, 1), k_heads=max(hk, 1),
                           head_dim=head_dim)
    q, k = w.x[:, :hq * head_dim], w.meta["k"][:, :hk * head_dim]
    # rows padded by 24 elements: the padding must stay untouched
    qd = torch.full((tokens, hq * head_dim + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    kd = torch.full((tokens, hk * head_dim + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    qd[:, :hq * head_dim] = to_dev(q)
    kd[:, :hk * head_dim] = to_dev(k)
    qv, kv = qd[:, :hq * head_dim], kd[:, :hk * head_dim]
    gpu_lib.nvfp4q_qk_norm(qv if hq else None, kv if hk else None, to_dev(w.gamma) if hq else None,
                           to_dev(w.meta["k_weight"]) if hk else None, head_dim, weight_offset=woff, eps=w.eps)
    if hq:
        _check_qk(to_np_bf16(qv), q, w.gamma, head_dim, woff, w.eps)
    if hk:
        _check_qk(to_np_bf16(kv), k, w.meta["k_weight"], head_dim, woff, w.eps)
    assert torch.all(qd[:, hq * head_dim:] == 7.0) and torch.all(kd[:, hk * head_dim:] == 7.0)


def test_qk_norm_4096_tokens_32q_8k_heads_of_128(gpu_lib):
    w = workloads.qk_heads()
    qd, kd = to_dev(w.x), to_dev(w.meta["k"])
    gpu_lib.nvfp4q_qk_norm(qd, kd, to_dev(w.gamma), to_dev(w.meta["k_weight"]), 128, eps=w.eps)
    rng = np.random.default_rng(15)
    rows = np.unique(np.concatenate([[0, 1, 4095], rng.choice(4096, 200, replace=False)]))
    _check_qk(to_np_bf16(qd)[rows], w.x[rows], w.gamma, 128, 0.0, w.eps)
    _check_qk(to_np_bf16(kd)[rows], w.meta["k"][rows], w.meta["k_weight"], 128, 0.0, w.eps)


# ---------------------------------------------------------------- 2D
@pytest.mark.parametrize("shape", [(16, 16), (64, 48), (256, 384), (144, 272), (16, 2064), (528, 16)])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_2d_small(gpu_lib, shape, rounding):
    rng = np.random.default_rng(shape[0] + 7 * shape[1])
    x = _bf16(rng, shape, 0.02)
    got = gpu_lib.nvfp4q_quantize_2d(to_dev(x), rounding=rounding, seed=0x5EED, offset=4)
    q = oracle.quantize_2d(x, rounding=rounding, seed=0x5EED, offset=4)
    R, C = shape
    assert_same_bits("row codes", np_u8(got["row_codes"], C // 2), q["row"]["codes"])
    assert_same_bits("row scales", np_u8(got["row_scales"], C // 16), q["row"]["scales"])
    assert_same_bits("col codes", np_u8(got["col_codes"], R // 2), q["col"]["codes"])
    assert_same_bits("col scales", np_u8(got["col_scales"], R // 16), q["col"]["scales"])
    assert_f32_bits("amax", f32(got["amax"])[0], q["amax"])
    assert_f32_bits("scale", f32(got["scale"])[0], q["s_dec"])


def test_2d_single_planes_and_given_amax(gpu_lib):
    import torch

    rng = np.random.default_rng(10)
    x = _bf16(rng, (96, 160))
    q = oracle.quantize_2d(x, rounding="sr", seed=3)
    a = torch.tensor([q["amax"]], dtype=torch.float32, device="cuda")
    r = gpu_lib.nvfp4q_quantize_2d(to_dev(x), rounding="sr", seed=3, colwise=False)
    c = gpu_lib.nvfp4q_quantize_2d(to_dev(x), rounding="sr", seed=3, rowwise=False, amax=a)
    assert_same_bits("row codes", np_u8(r["row_codes"], 80), q["row"]["codes"])
    assert_same_bits("col codes", np_u8(c["col_codes"], 48), q["col"]["codes"])
    assert_same_bits("col scales", np_u8(c["col_scales"], 6), q["col"]["scales"])
    assert_f32_bits("scale", f32(c["scale"])[0], q["s_dec"])


def test_2d_weight_8192x8192_sampled(gpu_lib):
    w = workloads.weight_2d()
    got = gpu_lib.nvfp4q_quantize_2d(to_dev(w.x), rounding="sr", seed=w.seed, offset=w.offset)
    amax = np.float32(np.max(np.abs(F.bf16_to_f32(w.x))))
    assert_f32_bits("amax", f32(got["amax"])[0], amax)
    rng = np.random.default_rng(11)
    # one row and one column in every 128-row and 128-column band of the tile grid, both edges of the
    # first band and of the tensor, and some more at random
    bands = np.arange(0, 8192, 128) + rng.integers(0, 128, 64)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 8191], bands, rng.choice(8192, 24, replace=False)]))
    bands = np.arange(0, 8192, 128) + rng.integers(0, 128, 64)
    cols = np.unique(np.concatenate([[0, 1, 127, 128, 8191], bands, rng.choice(8192, 24, replace=False)]))
    qr = oracle.quantize_rowwise(w.x[rows], amax=amax, rounding="sr", seed=w.seed, offset=w.offset, row_ids=rows)
    qc = oracle.quantize_colwise(w.x[:, cols], amax=amax, rounding="sr", seed=w.seed, offset=w.offset, col_ids=cols)
    assert_same_bits("row codes", np_u8(got["row_codes"], 4096)[rows], qr["codes"])
    assert_same_bits("row scales", np_u8(got["row_scales"], 512)[rows], qr["scales"])
    assert_same_bits("col codes", np_u8(got["col_codes"], 4096)[cols], qc["codes"])
    assert_same_bits("col scales", np_u8(got["col_scales"], 512)[cols], qc["scales"])
    assert_f32_bits("scale", f32(got["scale"])[0], qr["s_dec"])


def _tile16_input(rng, shape):
    # rows and columns of different magnitudes, so that tile scales differ from the 1D block scales
    R, C = shape
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(0.02)
    x *= np.exp(rng.uniform(-3, 3, (R, 1))).astype(np.float32) * np.exp(rng.uniform(-3, 3, (1, C))).astype(np.float32)
    return workloads.to_bf16_bits(x)


def _tile16_compare(got, q, R, C, rowwise=True, colwise=True):
    if rowwise:
        assert_same_bits("row codes", np_u8(got["row_codes"], C // 2), q["row"]["codes"])
        assert_same_bits("row scales", np_u8(got["row_scales"], C // 16), q["row"]["scales"])
    if colwise:
        assert_same_bits("col codes", np_u8(got["col_codes"], R // 2), q["col"]["codes"])
        assert_same_bits("col scales", np_u8(got["col_scales"], R // 16), q["col"]["scales"])


@pytest.mark.parametrize("shape", [(16, 16), (64, 48), (256, 384), (144, 272), (16, 2064), (528, 16)])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_2d_tile16_small(gpu_lib, shape, rounding):
    # NVFP4Q_SCALE_16X16 (reading R-2dblk): one scale per 16 x 16 tile in both planes; partial 128 x 128
    # work tiles at the right and bottom edges.
    rng = np.random.default_rng(shape[0] * 3 + shape[1])
    x = _tile16_input(rng, shape)
    got = gpu_lib.nvfp4q_quantize_2d(to_dev(x), rounding=rounding, seed=0x5EED, offset=4, tile16=True)
    q = oracle.quantize_2d_block(x, rounding=rounding, seed=0x5EED, offset=4)
    _tile16_compare(got, q, *shape)
    assert_f32_bits("amax", f32(got["amax"])[0], q["amax"])
    assert_f32_bits("scale", f32(got["scale"])[0], q["s_dec"])


def test_2d_tile16_single_planes_and_given_amax(gpu_lib):
    import torch

    rng = np.random.default_rng(20)
    x = _tile16_input(rng, (96, 160))
    q = oracle.quantize_2d_block(x, rounding="sr", seed=3)
    a = torch.tensor([q["amax"]], dtype=torch.float32, device="cuda")
    r = gpu_lib.nvfp4q_quantize_2d(to_dev(x), rounding="sr", seed=3, colwise=False, tile16=True)
    c = gpu_lib.nvfp4q_quantize_2d(to_dev(x), rounding="sr", seed=3, rowwise=False, amax=a, tile16=True)
    _tile16_compare(r, q, 96, 160, colwise=False)
    _tile16_compare(c, q, 96, 160, rowwise=False)
    assert_f32_bits("scale", f32(c["scale"])[0], q["s_dec"])
    # a zero tile next to a non-zero one, and a whole zero tensor
    z = x.copy()
    z[16:32, :] = 0
    z[:, 32:48] = 0
    got = gpu_lib.nvfp4q_quantize_2d(to_dev(z), rounding="rtne", tile16=True)
    _tile16_compare(got, oracle.quantize_2d_block(z), 96, 160)
    z[:] = 0
    got = gpu_lib.nvfp4q_quantize_2d(to_dev(z), rounding="sr", seed=1, tile16=True)
    _tile16_compare(got, oracle.quantize_2d_block(z, rounding="sr", seed=1), 96, 160)


def test_2d_tile16_weight_8192x8192_sampled(gpu_lib):
    # The weight workload with tile scales, checked on windows of 32 x 64 (two tile rows, four tile
    # columns) at the corners, at work-tile boundaries and at random places.
    w = workloads.weight_2d()
    got = gpu_lib.nvfp4q_quantize_2d(to_dev(w.x), rounding="sr", seed=w.seed, offset=w.offset, tile16=True)
    amax = np.float32(np.max(np.abs(F.bf16_to_f32(w.x))))
    assert_f32_bits("amax", f32(got["amax"])[0], amax)
    rc, rs = np_u8(got["row_codes"], 4096), np_u8(got["row_scales"], 512)
    cc, cs = np_u8(got["col_codes"], 4096), np_u8(got["col_scales"], 512)
    rng = np.random.default_rng(12)
    origins = [(0, 0), (8160, 8128), (96, 112), (128, 128), (4064, 0)]
    origins += [(int(a) * 16, int(b) * 16) for a, b in zip(rng.integers(0, 510, 6), rng.integers(0, 508, 6))]
    for r0, c0 in origins:
        q = oracle.quantize_2d_block(w.x[r0:r0 + 32, c0:c0 + 64], amax=amax, rounding="sr", seed=w.seed,
                                     offset=w.offset, origin=(r0, c0), full=(8192, 8192))
        where = f" at ({r0}, {c0})"
        assert_same_bits("row codes" + where, rc[r0:r0 + 32, c0 // 2:c0 // 2 + 32], q["row"]["codes"])
        assert_same_bits("row scales" + where, rs[r0:r0 + 32, c0 // 16:c0 // 16 + 4], q["row"]["scales"])
        assert_same_bits("col codes" + where, cc[c0:c0 + 64, r0 // 2:r0 // 2 + 16], q["col"]["codes"])
        assert_same_bits("col scales" + where, cs[c0:c0 + 64, r0 // 16:r0 // 16 + 2], q["col"]["scales"])


@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("shape", [(16, 16), (144, 272), (528, 16), (256, 384)])
@pytest.mark.parametrize("rounding,tile16", [("rtne", False), ("sr", False), ("sr", True)])
def test_2d_fp16_fp32_inputs(gpu_lib, dtype, shape, rounding, tile16):
    # reading R-dtype on the 2D path: both planes quantize the input values as given (fp32 tiles stage
    # 64 KiB in LDS); partial work tiles at the edges
    import torch

    rng = np.random.default_rng(shape[0] + 3 * shape[1] + (7 if tile16 else 0))
    R, C = shape
    x = (rng.standard_normal(shape) * np.exp(rng.uniform(-3, 3, (R, 1)))
         * np.exp(rng.uniform(-2, 2, (1, C)))).astype(getattr(np, dtype))
    got = gpu_lib.nvfp4q_quantize_2d(torch.from_numpy(x).cuda(), rounding=rounding, seed=0x2D, offset=6,
                                     tile16=tile16)
    fn = oracle.quantize_2d_block if tile16 else oracle.quantize_2d
    q = fn(x, rounding=rounding, seed=0x2D, offset=6)
    _tile16_compare(got, q, R, C)
    assert_f32_bits("amax", f32(got["amax"])[0], q["amax"])


def test_2d_experts_fp32(gpu_lib):
    import torch

    rng = np.random.default_rng(42)
    x = np.concatenate([(rng.standard_normal((64, 208)) * s).astype(np.float32) for s in (0.02, 5.0, 1e-3)])
    got = gpu_lib.nvfp4q_quantize_2d_grouped(torch.from_numpy(x).cuda(), 3, rounding="sr", seed=9, tile16=True)
    q = oracle.quantize_2d_experts(x, 3, rounding="sr", seed=9, tile16=True)
    _tile16_compare(got, q, 64, 208)
    for e in range(3):
        assert_f32_bits(f"expert {e} amax", f32(got["amax"])[e], q["amax"][e])


# ---------------------------------------------------------------- grouped 2D weights (reading R-experts)
@pytest.mark.parametrize("experts,shape", [(1, (48, 80)), (3, (144, 272)), (4, (16, 2064))])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
@pytest.mark.parametrize("tile16", [False, True])
def test_2d_experts_small(gpu_lib, experts, shape, rounding, tile16):
    rng = np.random.default_rng(experts * 100 + shape[1])
    x = np.concatenate([_tile16_input(rng, shape) for _ in range(experts)])
    got = gpu_lib.nvfp4q_quantize_2d_grouped(to_dev(x), experts, rounding=rounding, seed=0xE0, offset=5,
                                             tile16=tile16)
    q = oracle.quantize_2d_experts(x, experts, rounding=rounding, seed=0xE0, offset=5, tile16=tile16)
    R, C = shape
    _tile16_compare(got, q, R, C)
    for e in range(experts):
        assert_f32_bits(f"expert {e} amax", f32(got["amax"])[e], q["amax"][e])
        assert_f32_bits(f"expert {e} scale", f32(got["scale"])[e], q["s_dec"][e])


def test_2d_experts_given_amax_and_single_planes(gpu_lib):
    import torch

    rng = np.random.default_rng(21)
    x = np.concatenate([_tile16_input(rng, (64, 96)) for _ in range(4)])
    amax = np.array([0.5, 3.0, 0.0, 1e-3], np.float32)
    a = torch.tensor(amax, device="cuda")
    q = oracle.quantize_2d_experts(x, 4, amax=amax, rounding="sr", seed=2)
    r = gpu_lib.nvfp4q_quantize_2d_grouped(to_dev(x), 4, amax=a, rounding="sr", seed=2, colwise=False)
    c = gpu_lib.nvfp4q_quantize_2d_grouped(to_dev(x), 4, amax=a, rounding="sr", seed=2, rowwise=False)
    _tile16_compare(r, q, 64, 96, colwise=False)
    _tile16_compare(c, q, 64, 96, rowwise=False)
    for e in range(4):
        assert_f32_bits(f"expert {e} scale", f32(c["scale"])[e], q["s_dec"][e])


def test_2d_experts_4x4096x7168_sampled(gpu_lib):
    # The grouped-weight workload (four stacked 4096 x 7168 weights, SR), checked on sampled rows and
    # columns of every expert against the oracle's rowwise and columnwise planes with that expert's tags.
    w = workloads.experts_2d()
    E, R, C = w.experts, w.rows // w.experts, w.cols
    got = gpu_lib.nvfp4q_quantize_2d_grouped(to_dev(w.x), E, rounding="sr", seed=w.seed, offset=w.offset)
    rc, rs = np_u8(got["row_codes"], C // 2), np_u8(got["row_scales"], C // 16)
    cc, cs = np_u8(got["col_codes"], R // 2), np_u8(got["col_scales"], R // 16)
    rng = np.random.default_rng(13)
    for e in range(E):
        xe = w.x[e * R:(e + 1) * R]
        amax = np.float32(np.max(np.abs(F.bf16_to_f32(xe))))
        assert_f32_bits(f"expert {e} amax", f32(got["amax"])[e], amax)
        rows = np.unique(np.concatenate([[0, 127, 128, R - 1], rng.choice(R, 12, replace=False)]))
        cols = np.unique(np.concatenate([[0, 127, 128, C - 1], rng.choice(C, 12, replace=False)]))
        qr = oracle.quantize_rowwise(xe[rows], amax=amax, rounding="sr", seed=w.seed, offset=w.offset,
                                     tag=2 * e, row_ids=rows)
        qc = oracle.quantize_colwise(xe[:, cols], amax=amax, rounding="sr", seed=w.seed, offset=w.offset,
                                     col_ids=cols, tag=2 * e + 1)
        assert_same_bits(f"expert {e} row codes", rc[e * R + rows], qr["codes"])
        assert_same_bits(f"expert {e} row scales", rs[e * R + rows], qr["scales"])
        assert_same_bits(f"expert {e} col codes", cc[e * C + cols], qc["codes"])
        assert_same_bits(f"expert {e} col scales", cs[e * C + cols], qc["scales"])
        assert_f32_bits(f"expert {e} scale", f32(got["scale"])[e], qr["s_dec"])


# ---------------------------------------------------------------- grouped
def _grouped_check(gpu_lib, x, offsets, apply_rht, mask, rounding, seed=21, offset=2, groups=None, amax=None,
                   fast_math=False, colwise=True, rowwise=False, row_amax=None, pad=0, amax_all=False):
    import torch

    T, C = x.shape
    G = len(offsets) - 1
    cap = T + 15 * G
    cap16 = (cap + 15) // 16 * 16
    codes = torch.full((C, (cap16 // 2 + 15) // 16 * 16), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full((C, cap16 // 16), 0x55, dtype=torch.uint8, device="cuda")
    rcodes = torch.full((T, (C // 2 + 15) // 16 * 16), 0xAA, dtype=torch.uint8, device="cuda")
    rscales = torch.full((T, C // 16 + 3), 0x55, dtype=torch.uint8, device="cuda")
    a = None if amax is None else torch.tensor(amax, dtype=torch.float32, device="cuda")
    ra = None if row_amax is None else torch.tensor(row_amax, dtype=torch.float32, device="cuda")
    xd = to_dev(x) if x.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if pad:  # rows of x further apart than cols (a view into a wider buffer)
        wide = torch.full((x.shape[0], x.shape[1] + pad), 3.0, dtype=xd.dtype, device="cuda")
        wide[:, :x.shape[1]] = xd
        xd = wide[:, :x.shape[1]]
    got = gpu_lib.nvfp4q_grouped(xd, torch.tensor(offsets, dtype=torch.int32, device="cuda"),
                                 apply_rht=apply_rht, rht_mask=mask, amax=a, rounding=rounding, seed=seed,
                                 offset=offset, codes=codes, scales=scales, fast_math=fast_math, colwise=colwise,
                                 rowwise=rowwise, row_amax=ra, row_codes=rcodes, row_scales=rscales)
    ref = oracle.grouped_quantize(x, np.asarray(offsets, np.int32), apply_rht=apply_rht, rht_mask=mask,
                                  amax=None if amax is None else np.asarray(amax, np.float32),
                                  rounding=rounding, seed=seed, offset=offset, groups=groups, fast_math=fast_math,
                                  rowwise=rowwise,
                                  row_amax=None if row_amax is None else np.asarray(row_amax, np.float32))
    poff = ref["poff"]
    mpad = int(poff[-1])
    assert np.array_equal(got["poff"].cpu().numpy(), poff)
    gc, gs = np_u8(codes), np_u8(scales)
    rc, rs = np_u8(rcodes), np_u8(rscales)
    for g in (range(G) if groups is None else groups):
        if colwise:
            a0, a1 = int(poff[g]), int(poff[g + 1])
            assert_same_bits(f"group {g} codes", gc[:, a0 // 2:a1 // 2], ref["codes"][:, a0 // 2:a1 // 2])
            assert_same_bits(f"group {g} scales", gs[:, a0 // 16:a1 // 16], ref["scales"][:, a0 // 16:a1 // 16])
            assert_f32_bits(f"group {g} amax", f32(got["amax"])[g], ref["amax"][g])
            assert_f32_bits(f"group {g} scale", f32(got["scale"])[g], ref["s_dec"][g])
        if rowwise:
            r0, r1 = int(offsets[g]), int(offsets[g + 1])
            assert_same_bits(f"group {g} row codes", rc[r0:r1, :C // 2], ref["row_codes"][r0:r1])
            assert_same_bits(f"group {g} row scales", rs[r0:r1, :C // 16], ref["row_scales"][r0:r1])
            assert_f32_bits(f"group {g} row amax", f32(got["row_amax"])[g], ref["row_amax"][g])
            assert_f32_bits(f"group {g} row scale", f32(got["row_scale"])[g], ref["row_s_dec"][g])
    if amax_all:
        # every group's rowwise amax (a plain max |x|), and each group's S_dec as the scale rule of its amax
        xf = F.bf16_to_f32(x) if x.dtype == np.uint16 else x.astype(np.float32)
        for g in range(G):
            r0, r1 = int(offsets[g]), int(offsets[g + 1])
            a = np.float32(np.max(np.abs(xf[r0:r1]))) if r1 > r0 else np.float32(0.0)
            if rowwise:
                assert_f32_bits(f"group {g} row amax", f32(got["row_amax"])[g], a)
                assert_f32_bits(f"group {g} row scale", f32(got["row_scale"])[g],
                                oracle.global_scales(f32(got["row_amax"])[g])[1])
            if colwise:
                assert_f32_bits(f"group {g} scale", f32(got["scale"])[g],
                                oracle.global_scales(f32(got["amax"])[g])[1])
    if colwise:
        # the tail past the last padded column is never written
        assert np.all(gc[:, mpad // 2:] == 0xAA) and np.all(gs[:, mpad // 16:] == 0x55)
    else:
        assert np.all(gc == 0xAA) and np.all(gs == 0x55)
    if rowwise:
        # nothing past a row's C / 2 code bytes and C / 16 scale bytes
        assert np.all(rc[:, C // 2:] == 0xAA) and np.all(rs[:, C // 16:] == 0x55)


@pytest.mark.parametrize("apply_rht", [True, False])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_grouped_small(gpu_lib, apply_rht, rounding):
    rng = np.random.default_rng(12)
    x = _bf16(rng, (203, 272))
    offsets = [0, 0, 5, 21, 21, 150, 203]          # empty groups, short trailing groups
    _grouped_check(gpu_lib, x, offsets, apply_rht, 0x9C35, rounding)


def test_grouped_one_group_and_given_amax(gpu_lib):
    rng = np.random.default_rng(13)
    x = _bf16(rng, (300, 528), 4.0)
    _grouped_check(gpu_lib, x, [0, 300], True, 0xFFFF, "sr")
    _grouped_check(gpu_lib, x, [0, 7, 300], True, 0x0001, "rtne", amax=[1.5, 30.0])


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_grouped_extreme_group_scales(gpu_lib, rounding):
    # Groups whose amax lies below 2^-90, is exactly zero, is ordinary, and lies
    # above 2^120: the encode folds the transform's 0.25 into the block maximum
    # only inside [2^-90, 2^120] and must agree with the oracle on both sides.
    rng = np.random.default_rng(15)
    parts = [(_bf16(rng, (40, 288), 1e-30)), np.zeros((23, 288), np.uint16), _bf16(rng, (37, 288)),
             _bf16(rng, (50, 288), 1e37), _bf16(rng, (19, 288), 3e-28)]
    x = np.concatenate(parts, axis=0)
    offsets = np.concatenate([[0], np.cumsum([p.shape[0] for p in parts])]).tolist()
    _grouped_check(gpu_lib, x, offsets, True, 0x6A5C, rounding)


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_grouped_fast_math(gpu_lib, rounding):
    # NVFP4Q_FAST_MATH: the transform's fp32 output, without its bf16 round-through (reading R-fast),
    # bit-exact against the oracle's fast mode; ragged groups, an empty group, a given amax, and groups
    # outside the folding range of the encode.
    rng = np.random.default_rng(16)
    x = _bf16(rng, (203, 272))
    _grouped_check(gpu_lib, x, [0, 0, 5, 21, 21, 150, 203], True, 0x9C35, rounding, fast_math=True)
    _grouped_check(gpu_lib, x, [0, 7, 203], True, 0x0F0F, rounding, amax=[1.5, 30.0], fast_math=True)
    parts = [_bf16(rng, (40, 288), 1e-30), _bf16(rng, (37, 288)), _bf16(rng, (50, 288), 1e37)]
    x = np.concatenate(parts, axis=0)
    _grouped_check(gpu_lib, x, [0, 40, 77, 127], True, 0x6A5C, rounding, fast_math=True)


def test_grouped_moe_16384x7168_fast_math_sampled(gpu_lib):
    w = workloads.grouped_moe()
    G = len(w.offsets) - 1
    _grouped_check(gpu_lib, w.x, w.offsets.tolist(), w.apply_rht, w.rht_mask, "sr", seed=w.seed,
                   offset=w.offset, groups=[3, 33, G - 2], fast_math=True)


def test_grouped_moe_16384x7168_fast_math_sqnr(gpu_lib):
    """[PR] Fast math, acceptance: on the full grouped workload the fast mode's dequantized columnwise plane
    keeps an SQNR of at least 25 dB against the exact mode's, both from the HIP path (a sample of 512
    columns, every group), and under 3 % of their code bytes differ."""
    import torch

    w = workloads.grouped_moe()
    xd = to_dev(w.x)
    offs = torch.tensor(w.offsets, dtype=torch.int32, device="cuda")
    kw = dict(apply_rht=True, rht_mask=w.rht_mask, rounding="sr", seed=w.seed, offset=w.offset)
    ex = gpu_lib.nvfp4q_grouped(xd, offs, **kw)
    fa = gpu_lib.nvfp4q_grouped(xd, offs, fast_math=True, **kw)
    torch.cuda.synchronize()
    poff = ex["poff"].cpu().numpy().astype(np.int64)
    cols = np.arange(0, w.x.shape[1], 14)
    mpad = int(poff[-1])

    def deq(r):
        c, sc, sd = np_u8(r["codes"])[cols], np_u8(r["scales"])[cols], f32(r["scale"])
        return np.concatenate([oracle.dequantize_rowwise(c[:, poff[g] // 2:poff[g + 1] // 2],
                                                         sc[:, poff[g] // 16:poff[g + 1] // 16], sd[g])
                               for g in range(len(poff) - 1) if poff[g + 1] > poff[g]], axis=1)

    de, df = deq(ex), deq(fa)
    sqnr = 10 * np.log10(np.sum(de ** 2) / np.sum((df - de) ** 2))
    assert sqnr >= 25.0, sqnr
    differ = np.mean(np_u8(ex["codes"])[:, :mpad // 2] != np_u8(fa["codes"])[:, :mpad // 2])
    assert differ < 0.03, differ


def test_grouped_64_groups_many_empty(gpu_lib):
    rng = np.random.default_rng(14)
    counts = rng.multinomial(1000, np.full(64, 1 / 64))
    counts[::7] = 0
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = _bf16(rng, (int(offsets[-1]), 256))
    _grouped_check(gpu_lib, x, offsets.tolist(), True, 0x5A5A, "sr")


def test_grouped_moe_16384x7168_sampled(gpu_lib):
    w = workloads.grouped_moe()
    G = len(w.offsets) - 1
    _grouped_check(gpu_lib, w.x, w.offsets.tolist(), w.apply_rht, w.rht_mask, "sr", seed=w.seed,
                   offset=w.offset, groups=[0, 17, 40, G - 1])


@pytest.mark.timeout(400)
def test_grouped_moe_131072x7168_both_planes_sampled(gpu_lib):
    """131072 tokens x hidden 7168 (1.9 GB of bf16) in 64 groups, both planes with their amax passes: the
    workspace bounds no input size. Groups 0, 31 and 63 against the oracle (codes, scales, amax and S_dec of
    both planes), every group's rowwise amax, every S_dec against its amax, the untouched tails."""
    w = workloads.grouped_moe(tokens=131072)
    _grouped_check(gpu_lib, w.x, w.offsets.tolist(), w.apply_rht, w.rht_mask, "sr", seed=w.seed,
                   offset=w.offset, groups=[0, 31, 63], rowwise=True, amax_all=True)


def test_grouped_moe_16384x7168_every_group_ends(gpu_lib):
    """Every group of the full-size workload: its amax and S_dec, and the codes and scales of its first and
    last 16-token block (the blocks next to the group boundaries) in every column."""
    import torch

    w = workloads.grouped_moe()
    G = len(w.offsets) - 1
    got = gpu_lib.nvfp4q_grouped(to_dev(w.x), torch.tensor(w.offsets, dtype=torch.int32, device="cuda"),
                                 apply_rht=w.apply_rht, rht_mask=w.rht_mask, rounding="sr", seed=w.seed,
                                 offset=w.offset)
    ref = oracle.grouped_quantize(w.x, w.offsets, apply_rht=w.apply_rht, rht_mask=w.rht_mask, rounding="sr",
                                  seed=w.seed, offset=w.offset, ends_only=True)
    poff = ref["poff"]
    assert np.array_equal(got["poff"].cpu().numpy(), poff)
    gc, gs = np_u8(got["codes"]), np_u8(got["scales"])
    for g in range(G):
        assert_f32_bits(f"group {g} amax", f32(got["amax"])[g], ref["amax"][g])
        assert_f32_bits(f"group {g} scale", f32(got["scale"])[g], ref["s_dec"][g])
        a0, a1 = int(poff[g]), int(poff[g + 1])
        for t0 in sorted({a0, a1 - 16} if a1 > a0 else set()):
            assert_same_bits(f"group {g} block at {t0} codes", gc[:, t0 // 2:t0 // 2 + 8],
                             ref["codes"][:, t0 // 2:t0 // 2 + 8])
            assert_same_bits(f"group {g} block at {t0} scales", gs[:, t0 // 16], ref["scales"][:, t0 // 16])


@pytest.mark.parametrize("apply_rht", [True, False])
@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_grouped_rowwise_and_columnwise(gpu_lib, apply_rht, rounding):
    # Both planes of the grouped input in one call (reading R-rowcol): ragged and empty groups, the
    # rowwise plane without the transform under its own per-group amax.
    rng = np.random.default_rng(17)
    x = _bf16(rng, (203, 272))
    _grouped_check(gpu_lib, x, [0, 0, 5, 21, 21, 150, 203], apply_rht, 0x9C35, rounding, rowwise=True)


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_grouped_rowwise_only_and_given_amax(gpu_lib, rounding):
    rng = np.random.default_rng(18)
    x = _bf16(rng, (300, 528), 4.0)
    _grouped_check(gpu_lib, x, [0, 7, 300], True, 0x0001, rounding, colwise=False, rowwise=True)
    _grouped_check(gpu_lib, x, [0, 7, 300], True, 0x0001, rounding, colwise=False, rowwise=True,
                   row_amax=[1.5, 30.0])
    # one plane's amax given, the other's computed
    _grouped_check(gpu_lib, x, [0, 0, 131, 300], True, 0xF00F, rounding, amax=[0.0, 2.0, 5.0], rowwise=True)
    _grouped_check(gpu_lib, x, [0, 0, 131, 300], True, 0xF00F, rounding, rowwise=True, row_amax=[1.0, 2.0, 5.0],
                   fast_math=True)


def test_grouped_rowwise_extreme_group_scales(gpu_lib):
    rng = np.random.default_rng(19)
    parts = [_bf16(rng, (40, 288), 1e-30), np.zeros((23, 288), np.uint16), _bf16(rng, (37, 288)),
             _bf16(rng, (50, 288), 1e37)]
    x = np.concatenate(parts, axis=0)
    offsets = np.concatenate([[0], np.cumsum([p.shape[0] for p in parts])]).tolist()
    _grouped_check(gpu_lib, x, offsets, True, 0x6A5C, "sr", rowwise=True)


def test_grouped_moe_16384x7168_rowwise_sampled(gpu_lib):
    w = workloads.grouped_moe()
    G = len(w.offsets) - 1
    _grouped_check(gpu_lib, w.x, w.offsets.tolist(), w.apply_rht, w.rht_mask, "sr", seed=w.seed,
                   offset=w.offset, groups=[1, 30, G - 1], rowwise=True)


@pytest.mark.parametrize("rounding", ["rtne", "sr"])
def test_grouped_padded_rows_both_planes(gpu_lib, rounding):
    # x rows 40 elements apart beyond cols (the padding holds values that must not leak into any plane)
    rng = np.random.default_rng(39)
    x = _bf16(rng, (150, 272))
    _grouped_check(gpu_lib, x, [0, 3, 3, 70, 150], True, 0x1E3C, rounding, rowwise=True, pad=40)


@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("apply_rht,rounding,fast", [(True, "sr", False), (True, "rtne", False), (False, "sr", False),
                                                      (True, "sr", True)])
def test_grouped_fp16_fp32_inputs(gpu_lib, dtype, apply_rht, rounding, fast):
    # reading R-dtype on the grouped path: the transform's output rounded through fp16, or not at all for
    # fp32; both planes, ragged and empty groups, padded rows
    rng = np.random.default_rng(44)
    x = (rng.standard_normal((203, 272)) * np.exp(rng.uniform(-2, 2, (203, 1)))).astype(getattr(np, dtype))
    _grouped_check(gpu_lib, x, [0, 0, 5, 21, 21, 150, 203], apply_rht, 0x9C35, rounding, rowwise=True,
                   fast_math=fast, pad=24)


def test_grouped_fp16_small_and_large_groups(gpu_lib):
    # fp16 groups near the ends of its range (no fold of the 0.25 through an fp16 round-through): the
    # transform's outputs of the small group are fp16 subnormals
    rng = np.random.default_rng(45)
    parts = [(rng.standard_normal((40, 96)) * 2e-5).astype(np.float16),
             (rng.standard_normal((37, 96)) * 1e4).astype(np.float16),
             rng.standard_normal((19, 96)).astype(np.float16)]
    x = np.concatenate(parts)
    _grouped_check(gpu_lib, x, [0, 40, 77, 96], True, 0x6A5C, "sr", rowwise=True)


def test_ceiling_probes_run(gpu_lib):
    """The probe kernels of bench.py --ceilings on a small input: the read pass leaves its output alone
    (written only for one particular value), the mix and row-layout passes write what they load, and the
    one-launch barriers' waits end without giving up (each call counter advances once per launch) and
    every workgroup stores with the grid's maximum (with each workgroup's own in the form without a wait)."""
    import ctypes
    import os

    import torch

    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.abspath(gpu_lib.__file__)), "libnvfp4q_ceilings.so"))
    vp, u64, u32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
    lib.ceil_read.argtypes = [vp, u64, vp, vp]
    lib.ceil_mix.argtypes = [vp, u64, vp, vp, vp]
    lib.ceil_rowmix.argtypes = [vp, u32, vp, vp, vp]
    lib.ceil_fused.argtypes = [vp, u32, vp, vp, vp, u32, vp]
    lib.ceil_fused_ws_bytes.restype = u64
    rows = 64
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.integers(0, 1 << 16, size=rows * 4096, dtype=np.uint16).view(np.int16)).cuda()
    nblk = rows * 256
    st = torch.cuda.current_stream().cuda_stream
    out = torch.zeros(4096, dtype=torch.int32, device="cuda")
    assert lib.ceil_read(x.data_ptr(), x.numel() * 2, out.data_ptr(), st) == 0
    codes = torch.zeros(nblk * 8, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(nblk, dtype=torch.uint8, device="cuda")
    assert lib.ceil_mix(x.data_ptr(), nblk, codes.data_ptr(), scales.data_ptr(), st) == 0
    torch.cuda.synchronize()
    w = x.view(torch.int32).cpu().numpy().view(np.uint32).reshape(nblk, 8)
    hi = w[:, 0] ^ w[:, 1] ^ w[:, 4] ^ w[:, 5]
    lo = w[:, 2] ^ w[:, 3] ^ w[:, 6] ^ w[:, 7]
    expect = (hi.astype(np.uint64) << np.uint64(32)) | lo.astype(np.uint64)
    assert np.array_equal(codes.cpu().numpy().view(np.uint64), expect)
    c2 = torch.zeros_like(codes)
    assert lib.ceil_rowmix(x.data_ptr(), rows, c2.data_ptr(), scales.data_ptr(), st) == 0
    torch.cuda.synchronize()
    assert torch.equal(c2, codes)   # the same blocks, loaded in the row layout
    ws = torch.zeros(lib.ceil_fused_ws_bytes(), dtype=torch.uint8, device="cuda")
    c3 = torch.zeros_like(codes)
    for k in range(3):
        assert lib.ceil_fused(x.data_ptr(), rows, c3.data_ptr(), scales.data_ptr(), ws.data_ptr(), 1 << 20, st) == 0
    torch.cuda.synchronize()
    epoch, err = ws[:8].view(torch.int32).cpu().numpy()
    assert err == 0 and epoch == 3
    # the other forms of the grid-wide maximum: each stored code word carries the maximum it used
    lib.ceil_fused_count.argtypes = [vp, u32, vp, vp, vp, u32, ctypes.c_int, vp]
    lib.ceil_fused_count_ws_bytes.restype = u64
    mag = (x.view(torch.int16).cpu().numpy().view(np.uint16) & 0x7FFF).astype(np.uint32).reshape(rows, 4096)
    g_all = np.uint64(mag.max())
    g_wg = np.repeat(mag.reshape(rows // 4, -1).max(axis=1), 4 * 256).astype(np.uint64)  # 4 rows per workgroup
    wc = torch.zeros(lib.ceil_fused_count_ws_bytes(), dtype=torch.uint8, device="cuda")
    calls = 0
    for mode in (0, 2, 3, 4, 1):
        c4 = torch.zeros_like(codes)
        for k in range(3):
            assert lib.ceil_fused_count(x.data_ptr(), rows, c4.data_ptr(), scales.data_ptr(), wc.data_ptr(), 1 << 20,
                                        mode, st) == 0
            calls += mode != 1
        torch.cuda.synchronize()
        g = g_wg if mode == 1 else g_all
        assert np.array_equal(c4.cpu().numpy().view(np.uint64), expect ^ (g << np.uint64(32))), mode
        epoch, err = wc[:8].view(torch.int32).cpu().numpy()
        assert err == 0 and epoch == calls, mode
    # the issue-rate kernels (registers only) run for every instruction kind
    lib.ceil_rate.argtypes = [ctypes.c_int, u32, u32, vp, vp]
    rout = torch.zeros(8 * 256, dtype=torch.int32, device="cuda")
    for kind in range(lib.ceil_rate_kinds()):
        assert lib.ceil_rate(kind, 8, 16, rout.data_ptr(), st) == 0
    torch.cuda.synchronize()

"""Benchmark: achieved HBM bandwidth of RMSNorm + NVFP4 quantization on one MI355X.

Default workload (the one the metric is quoted on): prefill, 4096 tokens x
hidden 4096 bf16, RMSNorm (eps 1e-6, gamma, no bias) feeding rowwise NVFP4 with
round-to-nearest-even. One step = one full ``rmsnorm_nvfp4q`` call: the tensor
amax, the normalization and the quantized output. Other workloads
(``--config quantize|decode|weight|grouped``) are available for measurement.

Bytes are the compulsory bytes of the format: every input read once and every
output written once (x, gamma[, beta], codes, scales, amax, S_dec). Inputs sit in
HBM before timing starts; the step rotates over enough copies of the input and
output buffers (>= 512 MiB in total) that no step finds its data in the 256 MB
Infinity Cache left behind by the previous steps.

Output: one JSON line on stdout (rank 0 only; this benchmark is one GPU).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, published peak
ROTATE_BYTES = 512 << 20   # total bytes cycled between steps (twice the 256 MB Infinity Cache)
METRIC = "achieved HBM GB/s and % of peak, RMSNorm+NVFP4 quantize (tokens×hidden)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- workloads
class Case:
    """Device buffers and launch closures for one workload."""

    def __init__(self, name, torch, q, workloads, fast_math=False, planes="col", tile16=False, dtype="bf16",
                 one_launch=False):
        import numpy as np

        self.name = name
        self.fast_math = fast_math
        self.planes = planes  # grouped: which planes a step writes
        self.one_launch = one_launch
        self.tile16 = tile16  # weight: one scale per 16 x 16 tile
        self.dtype = dtype    # element type of the input
        tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
        es = {"bf16": 2, "fp16": 2, "fp32": 4}[dtype]
        self.colwise = name != "grouped" or planes in ("col", "both")
        self.rowwise = name == "grouped" and planes in ("row", "both")
        self.w = w = workloads.make(name)
        dev = torch.device("cuda", 0)

        def d(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        def din(bits):  # an input of the requested type, from the workload's bf16 values (exact conversion)
            return d(bits).to(tdt)

        R, C = w.x.shape
        self.rows, self.cols = R, C
        x_bytes = R * C * es
        if name in ("quantize", "prefill", "decode"):
            out_bytes = R * C // 2 + R * C // 16
            param_bytes = (C * es if w.gamma is not None else 0) + (C * es if w.beta is not None else 0)
        elif name == "qknorm":           # in place: q and k read and written once, two weights read
            out_bytes = R * C * es + w.meta["k"].size * 2 * es
            param_bytes = 2 * es * w.meta["head_dim"]
        elif name in ("weight", "experts"):
            out_bytes = 2 * (R * C // 2 + R * C // 16)
            param_bytes = 0
            if name == "experts":      # per-expert amax and S_dec (the 2D call's 8 bytes are added below)
                out_bytes += 8 * (w.experts - 1)
        else:  # grouped
            G = len(w.offsets) - 1
            counts = np.diff(w.offsets)
            mpad = int(np.sum((counts + 15) // 16 * 16))
            self.mpad = mpad
            out_bytes = 4 * (G + 1)                     # padded offsets
            if self.colwise:  # the columnwise plane and its per-group amax and S_dec
                out_bytes += C * mpad // 2 + C * mpad // 16 + 8 * G
            if self.rowwise:  # the rowwise plane and its per-group amax and S_dec
                out_bytes += R * C // 2 + R * C // 16 + 8 * G
            param_bytes = 4 * (G + 1)
        self.bytes = x_bytes + out_bytes + param_bytes + (8 if name not in ("grouped", "qknorm") else 0)
        set_bytes = x_bytes + out_bytes
        self.nsets = max(1, math.ceil(ROTATE_BYTES / set_bytes))
        x0 = din(w.x)
        self.xs = [x0] + [x0.clone() for _ in range(self.nsets - 1)]
        self.gamma = din(w.gamma) if w.gamma is not None else None
        self.beta = din(w.beta) if w.beta is not None else None
        self.q = q
        self.torch = torch
        if name == "grouped":
            self.offsets = torch.tensor(w.offsets, dtype=torch.int32, device=dev)
            G = len(w.offsets) - 1
            cap16 = (R + 15 * G + 15) // 16 * 16
            self.outs = [(torch.empty((C, (cap16 // 2 + 15) // 16 * 16), dtype=torch.uint8, device=dev),
                          torch.empty((C, cap16 // 16), dtype=torch.uint8, device=dev)) for _ in range(self.nsets)]
            ldr = (C // 2 + 15) // 16 * 16
            self.row_outs = [(torch.empty((R, ldr), dtype=torch.uint8, device=dev),
                              torch.empty((R, C // 16), dtype=torch.uint8, device=dev)) if self.rowwise else (None, None)
                             for _ in range(self.nsets)]
        elif name in ("weight", "experts"):
            self.outs = [None] * self.nsets
        elif name == "qknorm":
            k0 = din(w.meta["k"])
            self.ks = [k0] + [k0.clone() for _ in range(self.nsets - 1)]
            self.outs = [None] * self.nsets
            self.wk = din(w.meta["k_weight"])
        else:
            ldc = (C // 2 + 15) // 16 * 16
            self.outs = [(torch.empty((R, ldc), dtype=torch.uint8, device=dev),
                          torch.empty((R, C // 16), dtype=torch.uint8, device=dev)) for _ in range(self.nsets)]

    def describe(self):
        w = self.w
        d = {"workload": self.name, "rows": self.rows, "cols": self.cols, "rounding": w.rounding,
             "compulsory_bytes_per_step": self.bytes, "rotated_buffer_sets": self.nsets}
        d["input_dtype"] = self.dtype
        if self.name in ("prefill", "decode"):
            d.update({"tokens": self.rows, "hidden": self.cols, "op": "rmsnorm+nvfp4 rowwise",
                      "bias": w.beta is not None, "eps": w.eps})
            if self.one_launch:
                d["one_launch"] = "NVFP4Q_ONE_LAUNCH: the amax found inside one launch (at most 64 tokens)"
        elif self.name == "qknorm":
            d.update({"op": "per-head RMSNorm of q and k in place (QK norm)", "tokens": self.rows,
                      "q_heads": self.cols // w.meta["head_dim"], "k_heads": w.meta["k"].shape[1] // w.meta["head_dim"],
                      "head_dim": w.meta["head_dim"], "eps": w.eps})
        elif self.name in ("weight", "experts"):
            d.update({"op": "nvfp4 rowwise+columnwise (2D weight)", "seed": w.seed})
            if self.name == "experts":
                d.update({"op": "grouped 2D weights: nvfp4 rowwise+columnwise of stacked expert weights, "
                                "per-expert amax", "experts": w.experts, "rows": self.rows // w.experts})
            if self.tile16:
                d["op"] = "nvfp4 rowwise+columnwise (2D weight), one scale per 16x16 tile"
        elif self.name == "grouped":
            d.update({"op": "grouped columnwise nvfp4 after 16-pt RHT", "groups": len(w.offsets) - 1,
                      "padded_tokens": self.mpad})
            if self.planes == "both":
                d["op"] = "grouped rowwise nvfp4 + columnwise nvfp4 after 16-pt RHT, one pass"
            elif self.planes == "row":
                d["op"] = "grouped rowwise nvfp4 (per-group amax)"
            if self.fast_math:
                d["fast_math"] = "transform output quantized in fp32 (no bf16 round-through)"
        else:
            d.update({"op": "nvfp4 rowwise"})
        return d

    def given(self, out):
        """The amax arguments that make a call skip its amax pass, from a call's outputs."""
        g = {"amax": out["amax"].clone()} if self.colwise else {}
        if self.rowwise:
            g["row_amax"] = out["row_amax"].clone()
        return g

    def step(self, i, given=None):
        q, w = self.q, self.w
        given = given or {}
        amax = given.get("amax")
        x = self.xs[i % self.nsets]
        o = self.outs[i % self.nsets]
        if self.name in ("prefill", "decode"):
            return q.rmsnorm_nvfp4q(x, self.gamma, self.beta, eps=w.eps, amax=amax, codes=o[0], scales=o[1],
                                    one_launch=self.one_launch)
        if self.name == "quantize":
            return q.nvfp4q_quantize(x, amax=amax, codes=o[0], scales=o[1])
        if self.name == "weight":
            return q.nvfp4q_quantize_2d(x, amax=amax, rounding=w.rounding, seed=w.seed, offset=w.offset,
                                        tile16=self.tile16)
        if self.name == "qknorm":
            return q.nvfp4q_qk_norm(x, self.ks[i % self.nsets], self.gamma, self.wk, w.meta["head_dim"], eps=w.eps)
        if self.name == "experts":
            return q.nvfp4q_quantize_2d_grouped(x, w.experts, amax=amax, rounding=w.rounding, seed=w.seed,
                                                offset=w.offset, tile16=self.tile16)
        return q.nvfp4q_grouped(x, self.offsets, apply_rht=w.apply_rht, rht_mask=w.rht_mask, amax=amax,
                                rounding=w.rounding, seed=w.seed, offset=w.offset, codes=o[0], scales=o[1],
                                fast_math=self.fast_math, colwise=self.colwise, rowwise=self.rowwise,
                                row_amax=given.get("row_amax"),
                                row_codes=self.row_outs[i % self.nsets][0],
                                row_scales=self.row_outs[i % self.nsets][1])


# ----------------------------------------------------------------------------- timing
def time_steps(case, steps, warmup, given=None, eager=False, passes=3):
    """Median over `passes` timed passes of the average ms per step over `steps` steps.

    The steps are captured once in a HIP graph (the library allocates nothing and
    records no memsets, so a call is capture-safe). A pass replays a graph of
    `warmup` untimed steps and then the graph of `steps` timed steps between two
    synchronizations, with HIP events around the timed replay on the stream the
    kernels run on. This removes the Python and launch overhead of each call,
    which would otherwise exceed the GPU time of a step. `eager` times plain
    calls instead. Returns (median ms per step, the passes' ms per step).
    """
    torch = case.torch
    per_pass = []
    if eager:
        for _ in range(passes):
            for i in range(warmup):
                case.step(i, given)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                case.step(warmup + i, given)
            e1.record()
            torch.cuda.synchronize()
            per_pass.append(e0.elapsed_time(e1) / steps)
        return sorted(per_pass)[len(per_pass) // 2], per_pass
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):                      # eager warm-up before capture
            case.step(i, given)
        torch.cuda.synchronize()
        gw, gt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=s):
            for i in range(max(warmup, 1)):
                case.step(i, given)
        with torch.cuda.graph(gt, stream=s):
            for i in range(steps):
                case.step(i, given)
        torch.cuda.synchronize()
        for _ in range(passes):
            gw.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            gt.replay()
            e1.record(s)
            torch.cuda.synchronize()
            per_pass.append(e0.elapsed_time(e1) / steps)
    return sorted(per_pass)[len(per_pass) // 2], per_pass


def compare_builds(case, libs, steps, warmup, reps, stage=False):
    """Median us per step of each library build on the same case, in one process: the library is swapped
    in the binding, a warm-up graph and a timed graph of `steps` steps are captured per library, and the
    timed replays alternate between libraries `reps` times (order reversed every other round), so that
    slow drifts of the box fall on every build alike. Box-to-box spread is several percent; the spread
    within one such run is well under one."""
    import statistics

    torch, q = case.torch, case.q
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    for lp in libs:
        q._lib = None
        q.lib_path = os.path.abspath(lp)
        q.load()
        with torch.cuda.stream(s):
            given = case.given(case.step(0)) if stage else None
            for i in range(3):
                case.step(i, given)
            torch.cuda.synchronize()
            gw, gt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(gw, stream=s):
                for i in range(max(warmup, 1)):
                    case.step(i, given)
            with torch.cuda.graph(gt, stream=s):
                for i in range(steps):
                    case.step(i, given)
            torch.cuda.synchronize()
        graphs.append((lp, gw, gt))
    times = {lp: [] for lp in libs}
    with torch.cuda.stream(s):
        for r in range(reps):
            for lp, gw, gt in (graphs if r % 2 == 0 else graphs[::-1]):
                gw.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                gt.replay()
                e1.record(s)
                torch.cuda.synchronize()
                times[lp].append(e0.elapsed_time(e1) / steps * 1e3)
    print(json.dumps({"compare": case.describe()["workload"], "timed": "roofline kernel, given amax" if stage
                      else "full step", "unit": "us per step", "steps": steps, "reps": reps,
                      "median": {lp: round(statistics.median(v), 3) for lp, v in times.items()},
                      "all": {lp: [round(x, 3) for x in v] for lp, v in times.items()}}))


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s=12.0):
    """The CPU oracle on a bounded sample of the same workload (rows of the tensor)."""
    import numpy as np

    import oracle

    w = case.w
    name = case.name
    t0 = time.perf_counter()
    done_bytes = 0
    passes = 0
    R, C = w.x.shape
    chunk = max(16, min(R, (1 << 22) // C // 16 * 16))    # about 4 M elements per oracle call
    r0 = 0
    while time.perf_counter() - t0 < budget_s:
        if name == "grouped":
            G = len(w.offsets) - 1
            g = passes % G
            oracle.grouped_quantize(w.x, w.offsets, apply_rht=w.apply_rht, rht_mask=w.rht_mask, rounding=w.rounding,
                                    seed=w.seed, offset=w.offset, groups=[g], fast_math=case.fast_math,
                                    colwise=case.colwise, rowwise=case.rowwise)
            n = int(w.offsets[g + 1] - w.offsets[g])
            done_bytes += case.bytes * n / R
        elif name == "experts":
            # a band of rows of one expert (rowwise plane) and the same share of its columns (columnwise)
            Re = R // w.experts
            e = r0 // Re
            rows = np.arange(r0, min((e + 1) * Re, r0 + chunk))
            xe = w.x[e * Re:(e + 1) * Re]
            lr = rows - e * Re
            ncol = max(16, len(rows) * C // Re)
            c0 = (lr[0] * C // Re) // 16 * 16
            cols = np.arange(c0, min(C, c0 + ncol))
            if case.tile16:
                b0 = lr[0] // 16 * 16
                oracle.quantize_2d_block(xe[b0:b0 + len(rows) // 16 * 16 or 16], amax=np.float32(1.0),
                                         rounding=w.rounding, seed=w.seed, origin=(b0, 0), full=xe.shape,
                                         tags=(2 * e, 2 * e + 1))
            else:
                oracle.quantize_rowwise(xe[lr], amax=np.float32(1.0), rounding=w.rounding, seed=w.seed,
                                        tag=2 * e, row_ids=lr)
                oracle.quantize_colwise(xe[:, cols], amax=np.float32(1.0), rounding=w.rounding, seed=w.seed,
                                        col_ids=cols, tag=2 * e + 1)
            done_bytes += case.bytes * len(rows) / R
            r0 = (rows[-1] + 1) % R
        else:
            rows = np.arange(r0, min(R, r0 + chunk))
            xs = w.x[rows]
            if name in ("prefill", "decode"):
                if case.dtype == "bf16":
                    oracle.rmsnorm_quantize(xs, w.gamma, w.beta, w.weight_offset, w.eps)
                else:
                    ndt = np.float16 if case.dtype == "fp16" else np.float32
                    conv = lambda a: None if a is None else oracle.bf16_to_f32(a).astype(ndt)
                    oracle.rmsnorm_quantize(conv(xs), conv(w.gamma), conv(w.beta), w.weight_offset, w.eps,
                                            out_dtype=case.dtype)
            elif name == "quantize":
                if case.dtype == "bf16":
                    oracle.quantize_rowwise(xs)
                else:
                    oracle.quantize_rowwise(oracle.bf16_to_f32(xs).astype(np.float16 if case.dtype == "fp16"
                                                                          else np.float32))
            elif name == "qknorm":
                oracle.qk_norm(xs, w.meta["k"][rows], w.gamma, w.meta["k_weight"], w.meta["head_dim"], eps=w.eps)
            else:
                if case.tile16:
                    b0 = rows[0] // 16 * 16
                    oracle.quantize_2d_block(w.x[b0:b0 + len(rows)], amax=np.float32(1.0), rounding=w.rounding,
                                             seed=w.seed, origin=(b0, 0), full=w.x.shape)
                else:
                    oracle.quantize_rowwise(xs, amax=np.float32(1.0), rounding=w.rounding, seed=w.seed,
                                            row_ids=rows)
                    oracle.quantize_colwise(w.x[:, rows], amax=np.float32(1.0), rounding=w.rounding, seed=w.seed,
                                            col_ids=rows)
            done_bytes += case.bytes * len(rows) / R
            r0 = (r0 + chunk) % R
        passes += 1
    el = time.perf_counter() - t0
    if name == "grouped":
        sample = f"{passes} groups of the grouped workload, one oracle call each"
    elif name == "weight":
        sample = f"{passes} calls of {chunk} rows + {chunk} columns of the 2D workload (both planes)"
    elif name == "experts":
        sample = (f"{passes} calls of up to {chunk} rows of one expert + the same share of its columns "
                  f"(both planes)")
    else:
        sample = f"{passes} calls of {min(chunk, R)} consecutive rows of the {name} workload"
    if case.dtype != "bf16":
        sample += (f" ({case.dtype} input" + ("" if name in ("quantize", "prefill", "decode") else
                                            "; the oracle run on the bf16 values it was converted from") + ")")
    threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": sample + f"; {el:.1f} s, {done_bytes / 1e6:.1f} MB of compulsory bytes",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


# ----------------------------------------------------------------------------- roofline
# The kernel each workload's roofline entry describes, how it is timed, and the
# pattern of its kernel names in a rocprofv3 trace. "stage": the encode kernel
# alone, launched with the amax the full step produced (for quantize, weight
# and grouped the same kernel the full step runs; for RMSNorm the single-pass
# encode that a given amax selects, since the full step's encode pass reads the
# amax pass's per-row 1/rms). "step": both passes timed together.
DOMINANT = {
    "prefill": ("stage", "k_rms_coop (encode mode)", r"k_rms_coop<\d+, \d+, \w+, \w+, 1, \w+(, \d+)?(, \w+)?>"),
    "decode": ("stage", "k_rms_coop (encode mode)", r"k_rms_coop<\d+, \d+, \w+, \w+, 1, \w+(, \d+)?(, \w+)?>"),
    "quantize": ("stage", "k_quant_rows", r"k_quant_rows"),
    "weight": ("stage", "k_quant_2d", r"k_quant_2d"),
    "experts": ("stage", "k_quant_2d", r"k_quant_2d"),
    "qknorm": ("step", "k_qk_norm", r"k_qk_norm"),
    "grouped": ("stage", "k_grouped_quant", r"k_grouped_quant"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def _code_only(text):
    """Source text without // comments, trailing blanks and empty lines (a comment edit keeps the digest)."""
    out = []
    for line in text.splitlines():
        i = line.find("//")
        line = (line if i < 0 else line[:i]).rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


# The kernel sources each workload's passes are built from; the shared device headers (*.hpp) count for all.
DIGEST_SOURCES = {
    "prefill": ("kernels_rms_stream.hip", "kernels_rms_coop.hip"),
    "decode": ("kernels_rms_stream.hip", "kernels_rms_coop.hip"),
    "quantize": ("kernels_rows.hip",),
    "weight": ("kernels_2d.hip", "kernels_rows.hip"),
    "experts": ("kernels_2d.hip", "kernels_rows.hip"),
    "grouped": ("kernels_grouped.hip",),
    "qknorm": ("kernels_qk.hip",),
}


def source_digest(workload=None):
    """sha256 of the device code a workload's kernels come from (its kernels_*.hip files and the shared
    headers, comments left out; with no workload, every kernels_*.hip): traffic figures are valid only for the
    kernels they were taken on. Host-only files (api.hip, the C header) do not enter."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rmsnorm_nvfp4_block_amd", "csrc")
    names = DIGEST_SOURCES[workload] if workload else None
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc)
                   if f.endswith(".hpp") or (f.startswith("kernels_") and f.endswith(".hip")
                                             and (names is None or f in names)))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def read_pmc(directory, counter):
    """{kernel name: [value per dispatch]} for one counter from a rocprofv3 --pmc csv directory."""
    import csv
    import glob
    import re

    out = {}
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    per = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                name = re.sub(r"\(anonymous namespace\)::", "", row["Kernel_Name"])
                key = (name, row["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def traffic_key(config, fast_math=False, planes="col", tile16=False, dtype="bf16"):
    """The profiles/traffic.json entry of a workload variant."""
    return (config + ("" if planes == "col" else "_" + planes) + ("_fast" if fast_math else "")
            + ("_tile16" if tile16 else "") + ("" if dtype == "bf16" else "_" + dtype))


def ingest_pmc(config, fetch_dir, write_dir, command, key=None):
    """Per-step FETCH_SIZE / WRITE_SIZE (KiB) of the dominant kernel(s) into profiles/traffic.json."""
    import re

    pat = re.compile(DOMINANT[config][2])
    entry = {"kernels": {}, "source_sha256": source_digest(config), "command": command}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for name, vals in read_pmc(d, counter).items():
            if pat.search(name):
                k = entry["kernels"].setdefault(name.split("(")[0], {})
                k[counter.lower() + "_kib"] = sum(vals) / len(vals)
                k["dispatches"] = len(vals)
    # the library's other kernels of the same run (the full step's passes), for reference only
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for name, vals in read_pmc(d, counter).items():
            if "nvfp4q::" in name and not pat.search(name):
                k = entry.setdefault("other_kernels", {}).setdefault(name.split("(")[0], {})
                k[counter.lower() + "_kib"] = sum(vals) / len(vals)
                k["dispatches"] = len(vals)
    if not entry["kernels"]:
        raise SystemExit("no dispatch of the dominant kernel in the counter files")
    if DOMINANT[config][0] == "stage" and len(entry["kernels"]) != 1:
        raise SystemExit(f"expected one kernel, found {list(entry['kernels'])}")
    entry["fetch_kib"] = sum(k.get("fetch_size_kib", 0.0) for k in entry["kernels"].values())
    entry["write_kib"] = sum(k.get("write_size_kib", 0.0) for k in entry["kernels"].values())
    _update_traffic(key or config, entry)


def ingest_copy(fetch_dir, write_dir, nbytes, command):
    """Counter readings of a plain device-to-device copy of `nbytes`: the calibration of FETCH/WRITE_SIZE."""
    best = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        cands = [(n, sorted(v)[len(v) // 2]) for n, v in read_pmc(d, counter).items() if "copy" in n.lower()]
        if not cands:
            raise SystemExit("no copy kernel in the counter files")
        # the calibration copies are the largest copy dispatches of the run
        best[counter] = max(cands, key=lambda t: t[1])[1]
    kib = nbytes / 1024.0
    _update_traffic("copy_calibration", {
        "bytes": nbytes, "fetch_kib": best["FETCH_SIZE"], "write_kib": best["WRITE_SIZE"],
        "fetch_factor": kib / best["FETCH_SIZE"], "write_factor": kib / best["WRITE_SIZE"], "command": command})


def _update_traffic(key, entry):
    d = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            d = json.load(fh)
    d[key] = entry
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(d, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({key: entry}))


def traffic_bytes(config):
    """Calibrated HBM bytes per launch of the dominant kernel(s), or None (no figures, or the code changed since)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        d = json.load(fh)
    e, cal = d.get(config), d.get("copy_calibration")
    if not e or not cal or e.get("source_sha256") != source_digest(config.split("_")[0]):
        return None
    return e["fetch_kib"] * 1024.0 * cal["fetch_factor"] + e["write_kib"] * 1024.0 * cal["write_factor"]


def copy_calibration(torch, nbytes, reps):
    """Plain copies of a known size, for the FETCH_SIZE / WRITE_SIZE calibration runs."""
    n = nbytes // 4
    bufs = [torch.full((n,), float(i), dtype=torch.float32, device="cuda") for i in range(4)]
    torch.cuda.synchronize()
    for r in range(reps):
        bufs[(2 * r + 1) % 4].copy_(bufs[(2 * r) % 4])
    torch.cuda.synchronize()
    log(f"[bench] {reps} copies of {nbytes} bytes done")


# ----------------------------------------------------------------------------- main
# ----------------------------------------------------------------------------- ceilings
def _graph_time(torch, step, steps, warmup, passes=3):
    """Median over `passes` of the ms per call of `step(i)`, captured `steps` times in a HIP graph
    (the same protocol as time_steps)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    per = []
    with torch.cuda.stream(s):
        for i in range(3):
            step(i, s)
        torch.cuda.synchronize()
        gw, gt = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=s):
            for i in range(max(warmup, 1)):
                step(i, s)
        with torch.cuda.graph(gt, stream=s):
            for i in range(steps):
                step(i, s)
        torch.cuda.synchronize()
        for _ in range(passes):
            gw.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            gt.replay()
            e1.record(s)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / steps)
    return sorted(per)[len(per) // 2], per


def ceilings(torch, steps, warmup):
    """Probe kernels with the traffic of the library's passes and none of their arithmetic
    (libnvfp4q_ceilings.so): what a pass of that shape can reach here. Prints one JSON line."""
    import ctypes

    path = os.path.join(ROOT, "rmsnorm_nvfp4_block_amd", "libnvfp4q_ceilings.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} not found: build it with `python -m rmsnorm_nvfp4_block_amd.build`")
    lib = ctypes.CDLL(path)
    vp, u64, u32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32
    lib.ceil_read.argtypes = [vp, u64, vp, vp]
    lib.ceil_mix.argtypes = [vp, u64, vp, vp, vp]
    lib.ceil_fused.argtypes = [vp, u32, vp, vp, vp, u32, vp]
    lib.ceil_rowmix.argtypes = [vp, u32, vp, vp, vp]
    lib.ceil_fused_ws_bytes.restype = u64
    lib.ceil_fused_count.argtypes = [vp, u32, vp, vp, vp, u32, ctypes.c_int, vp]
    lib.ceil_fused_count_ws_bytes.restype = u64
    lib.ceil_empty.argtypes = [u32, u32, ctypes.c_int, vp]
    for f in (lib.ceil_read, lib.ceil_mix, lib.ceil_rowmix, lib.ceil_fused, lib.ceil_fused_count, lib.ceil_empty):
        f.restype = ctypes.c_int

    def ok(rc, what):
        if rc != 0:
            raise SystemExit(f"{what}: hip error {rc}")

    out = torch.zeros(4096, dtype=torch.int32, device="cuda")
    results = []

    def record(name, shape, nbytes, ms, per, **extra):
        r = {"probe": name, "shape": shape, "bytes": nbytes, "us": round(ms * 1e3, 3),
             "pass_us": [round(t * 1e3, 3) for t in per], "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
             "frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        r.update(extra)
        results.append(r)
        log(f"[ceilings] {name:9s} {shape:12s} {r['us']:9.2f} us  {r['GBps']:8.1f} GB/s  ({r['frac']:.3f} of peak)")

    for rows, cols in ((4096, 4096), (8192, 8192), (16384, 7168)):
        shape = f"{rows}x{cols}"
        xb = rows * cols * 2
        nsets = max(2, -(-ROTATE_BYTES // xb))
        xs = [torch.empty(xb // 2, dtype=torch.int16, device="cuda").random_(-32768, 32767) for _ in range(nsets)]
        nblk = rows * cols // 16
        cs = [torch.empty(nblk * 8, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
        ss = [torch.empty(nblk, dtype=torch.uint8, device="cuda") for _ in range(nsets)]

        def rd(i, st):
            ok(lib.ceil_read(xs[i % nsets].data_ptr(), xb, out.data_ptr(), st.cuda_stream), "ceil_read")

        def mx(i, st):
            j = i % nsets
            ok(lib.ceil_mix(xs[j].data_ptr(), nblk, cs[j].data_ptr(), ss[j].data_ptr(), st.cuda_stream), "ceil_mix")

        def two(i, st):
            rd(i, st)
            mx(i, st)

        ms, per = _graph_time(torch, rd, steps, warmup)
        record("read", shape, xb, ms, per, pattern="one 8 KiB span per wave (64 lanes x 8 loads of 16 B)")
        ms, per = _graph_time(torch, mx, steps, warmup)
        record("mix", shape, nblk * 41, ms, per,
               pattern="per 16-element block: 2 x 16 B loads, 8 B + 1 B non-temporal stores")
        if (rows, cols) == (4096, 4096):
            ms, per = _graph_time(torch, two, steps, warmup)
            record("two-pass", shape, xb + nblk * 41, ms, per,
                   pattern="read, then mix over the same x (two launches per step)")

            def rmx(i, st):
                j = i % nsets
                ok(lib.ceil_rowmix(xs[j].data_ptr(), rows, cs[j].data_ptr(), ss[j].data_ptr(), st.cuda_stream),
                   "ceil_rowmix")

            def two_rows(i, st):
                rd(i, st)
                rmx(i, st)

            ms, per = _graph_time(torch, rmx, steps, warmup)
            record("rowmix", shape, nblk * 41, ms, per,
                   pattern="the mix traffic in the rowwise encode's layout (one row per wave, 8 loads in flight)")
            ms, per = _graph_time(torch, two_rows, steps, warmup)
            record("two-pass-rows", shape, xb + nblk * 41, ms, per,
                   pattern="read, then rowmix over the same x: each row on the same wave (and XCD) in both")
            ws = torch.zeros(lib.ceil_fused_ws_bytes(), dtype=torch.uint8, device="cuda")

            def fused(i, st):
                j = i % nsets
                ok(lib.ceil_fused(xs[j].data_ptr(), rows, cs[j].data_ptr(), ss[j].data_ptr(), ws.data_ptr(),
                                  1 << 20, st.cuda_stream), "ceil_fused")

            ms, per = _graph_time(torch, fused, steps, warmup)
            err = int(ws[4:8].view(torch.int32).item())
            record("fused", shape, xb + nblk * 9, ms, per, wait_gave_up=bool(err),
                   pattern="one launch: rows in registers, grid-wide maximum through per-workgroup slots, stores")
            wc = torch.zeros(lib.ceil_fused_count_ws_bytes(), dtype=torch.uint8, device="cuda")
            for mode, name, pat in ((0, "fused-count", "one launch: grid-wide maximum through one arrival counter "
                                     "and one atomic maximum (release / acquire), stores"),
                                    (2, "fused-count-relaxed", "as fused-count with relaxed atomics (the arrival "
                                     "issued after the maximum's atomic returned)"),
                                    (3, "fused-slots-all", "per-workgroup slots, each workgroup polling all of "
                                     "them with every load of a round in flight"),
                                    (4, "fused-flags", "per-workgroup slots read by workgroup 0, which raises one "
                                     "flag per 64 workgroups; the others poll their flag"),
                                    (1, "fused-nowait", "one launch, no grid-wide wait (each workgroup's own "
                                     "maximum): the shape's floor")):
                def fc(i, st, mode=mode):
                    j = i % nsets
                    ok(lib.ceil_fused_count(xs[j].data_ptr(), rows, cs[j].data_ptr(), ss[j].data_ptr(),
                                            wc.data_ptr(), 1 << 20, mode, st.cuda_stream), "ceil_fused_count")

                ms, per = _graph_time(torch, fc, steps, warmup)
                err = int(wc[4:8].view(torch.int32).item())
                record(name, shape, xb + nblk * 9, ms, per, wait_gave_up=bool(err), pattern=pat)
        del xs, cs, ss
        torch.cuda.empty_cache()

    # issue cost of single VALU instructions: 2048 x 256 threads (8 waves per SIMD), 4096 iterations of
    # 8 independent instructions per lane
    lib.ceil_rate_kinds.restype = ctypes.c_int
    lib.ceil_rate_name.restype = ctypes.c_char_p
    lib.ceil_rate_name.argtypes = [ctypes.c_int]
    lib.ceil_rate.argtypes = [ctypes.c_int, u32, u32, vp, vp]
    lib.ceil_rate.restype = ctypes.c_int
    grid, iters = 2048, 4096
    rout = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    simds = torch.cuda.get_device_properties(0).multi_processor_count * 4
    winst = grid * 4 * iters * 8
    rates = []
    for kind in range(lib.ceil_rate_kinds()):  # one untimed round first (clocks settle)
        ok(lib.ceil_rate(kind, grid, iters, rout.data_ptr(), torch.cuda.current_stream().cuda_stream), "ceil_rate")
    torch.cuda.synchronize()
    for kind in range(lib.ceil_rate_kinds()):
        name = lib.ceil_rate_name(kind).decode()
        ms, per = _graph_time(torch, lambda i, st, kind=kind: ok(lib.ceil_rate(kind, grid, iters, rout.data_ptr(),
                                                                                st.cuda_stream), "ceil_rate"), 5, 1)
        rates.append({"instruction": name, "ns_per_wave_instruction_per_simd": round(ms * 1e6 * simds / winst, 4)})
    base = rates[0]["ns_per_wave_instruction_per_simd"]
    for r in rates:
        r["vs_v_add_u32"] = round(r["ns_per_wave_instruction_per_simd"] / base, 2)
        log(f"[ceilings] issue {r['instruction']:30s} {r['ns_per_wave_instruction_per_simd']:.3f} ns per wave "
            f"instruction and SIMD ({r['vs_v_add_u32']:.2f} x v_add_u32)")

    # launch cost of an empty 1024 x 256 kernel: in a graph, and eager (plain vs cooperative)
    n = 200
    ms, per = _graph_time(torch, lambda i, st: ok(lib.ceil_empty(1, 1024, 0, st.cuda_stream), "ceil_empty"),
                          n, warmup)
    launches = {"graph_plain_us": round(ms * 1e3, 3)}
    for coop in (0, 1):
        st = torch.cuda.Stream()
        ok(lib.ceil_empty(8, 1024, coop, st.cuda_stream), "ceil_empty")
        torch.cuda.synchronize()
        t = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            ok(lib.ceil_empty(n, 1024, coop, st.cuda_stream), "ceil_empty")
            e1.record(st)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) / n)
        launches["eager_cooperative_us" if coop else "eager_plain_us"] = round(sorted(t)[1] * 1e3, 3)
    log(f"[ceilings] empty 1024x256 kernel per launch: {launches}")
    print(json.dumps({"ceilings": results, "valu_issue": rates, "empty_kernel_launch": launches, "steps": steps,
                      "warmup": warmup,
                      "timing": "median of 3 passes of a graph of `steps` calls (launch costs: see keys)"}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="prefill", choices=["quantize", "prefill", "decode", "weight", "grouped", "experts", "qknorm"])
    ap.add_argument("--fast-math", action="store_true",
                    help="grouped: NVFP4Q_FAST_MATH (no bf16 round-through of the transform's output)")
    ap.add_argument("--planes", default="col", choices=["col", "row", "both"],
                    help="grouped: the columnwise plane, the rowwise plane, or both in one pass")
    ap.add_argument("--tile16", action="store_true",
                    help="weight: NVFP4Q_SCALE_16X16 (one block scale per 16x16 tile, shared by both planes)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16", "fp32"],
                    help="element type of the input (the workload's values, converted exactly)")
    ap.add_argument("--one-launch", action="store_true",
                    help="prefill/decode: NVFP4Q_ONE_LAUNCH (one launch meeting on the amax inside it, <= 64 tokens)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-only", action="store_true",
                    help="time only the roofline kernel with a given amax (for kernel traces); no metric line")
    ap.add_argument("--eager", action="store_true", help="time plain calls instead of a HIP graph replay")
    ap.add_argument("--ceilings", action="store_true",
                    help="only run the probe kernels (read, traffic mix, two-pass, one-launch barrier, launch cost)")
    ap.add_argument("--copy-calibration", type=int, metavar="BYTES",
                    help="only run plain copies of BYTES (for the counter calibration runs)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="record the dominant kernel's FETCH_SIZE/WRITE_SIZE from two rocprofv3 --pmc runs")
    ap.add_argument("--ingest-copy", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="record the copy calibration from two rocprofv3 --pmc runs of --copy-calibration")
    ap.add_argument("--command", default="", help="the command the ingested counter runs used")
    ap.add_argument("--compare", nargs="+", metavar="LIB",
                    help="time this build's library against other builds of it (paths to libnvfp4q.so) in one "
                         "process: a graph per library, replays alternated --reps times (with --stage-only: "
                         "the roofline kernel with a given amax); one JSON line of per-library medians")
    ap.add_argument("--reps", type=int, default=9, help="--compare: alternated replays per library")
    args = ap.parse_args()

    if args.ingest_pmc:
        ingest_pmc(args.config, *args.ingest_pmc, command=args.command,
                   key=traffic_key(args.config, args.fast_math, args.planes, args.tile16, args.dtype))
        return
    if args.ingest_copy:
        ingest_copy(*args.ingest_copy, nbytes=args.copy_calibration or (256 << 20), command=args.command)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path has no multi-GPU "
                                   "component (a sharded run would add one amax all-reduce, not built)"}))
        sys.exit(2)

    # the CPU oracle is single-threaded numpy; pin BLAS/OpenMP pools before numpy loads
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"

    import torch

    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration, 8)
        return
    if args.ceilings:
        torch.cuda.set_device(0)
        ceilings(torch, args.steps, args.warmup)
        return

    import rmsnorm_nvfp4_block_amd as q
    import workloads

    q.load()
    torch.cuda.set_device(0)
    if args.fast_math and args.config != "grouped":
        raise SystemExit("--fast-math applies to the grouped workload (the only one with the transform)")
    if args.planes != "col" and args.config != "grouped":
        raise SystemExit("--planes applies to the grouped workload (the others name their planes already)")
    if args.fast_math and args.planes == "row":
        raise SystemExit("--fast-math concerns the transform, which the rowwise plane does not take")
    if args.tile16 and args.config not in ("weight", "experts"):
        raise SystemExit("--tile16 applies to the weight and experts workloads (the 2D path)")
    if args.one_launch and args.config not in ("prefill", "decode"):
        raise SystemExit("--one-launch applies to the RMSNorm workloads (prefill, decode)")
    case = Case(args.config, torch, q, workloads, fast_math=args.fast_math, planes=args.planes, tile16=args.tile16,
                dtype=args.dtype, one_launch=args.one_launch)
    log(f"[bench] {case.describe()}")

    how, kname, _ = DOMINANT[args.config]
    if args.compare:
        compare_builds(case, [q.lib_path] + args.compare, args.steps, args.warmup, args.reps,
                       stage=args.stage_only and how == "stage")
        return
    if args.stage_only:
        # for a kernel trace of the roofline kernel alone: one eager call for the amax, then its graph
        if how != "stage":
            raise SystemExit("--stage-only needs a workload whose roofline kernel is timed alone")
        given = case.given(case.step(0))
        torch.cuda.synchronize()
        kms, kpass = time_steps(case, args.steps, args.warmup, given=given, eager=args.eager)
        log(f"[bench] {kname} alone (given amax): {kms * 1e3:.2f} us/launch (median of {len(kpass)} passes)")
        print(json.dumps({"stage_only": True, "config": case.describe(), "kernel": kname,
                          "launch_us": round(kms * 1e3, 3), "pass_us": [round(t * 1e3, 3) for t in kpass],
                          "bytes_per_launch": case.bytes}), flush=True)
        return

    # whole step (amax + quantize), the figure the metric is quoted on
    ms, spass = time_steps(case, args.steps, args.warmup, eager=args.eager)
    log(f"[bench] full step: {ms * 1e3:.2f} us/step (median of {len(spass)} passes: "
        + ", ".join(f"{t * 1e3:.2f}" for t in spass) + ")")
    value = case.bytes / (ms * 1e-3) / 1e9

    if how == "stage":
        # the encode kernel alone against the amax the full step produced
        given = case.given(case.step(0))
        torch.cuda.synchronize()
        kms, kpass = time_steps(case, args.steps, args.warmup, given=given, eager=args.eager)
        log(f"[bench] {kname} alone (given amax): {kms * 1e3:.2f} us/launch (median of {len(kpass)} passes: "
            + ", ".join(f"{t * 1e3:.2f}" for t in kpass) + ")")
    else:
        kms, kpass = ms, spass
    achieved = case.bytes / (kms * 1e-3) / 1e9
    traffic = traffic_bytes(traffic_key(args.config, args.fast_math, args.planes, args.tile16, args.dtype))
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "config": dict(case.describe(), timing=("median of 3 passes; a pass replays a graph of `warmup` steps, "
                                                "then times a graph of `steps` steps between syncs")
                       if not args.eager else "median of 3 passes of `warmup` + `steps` eager calls"),
        "pass_ms_per_step": [round(t, 5) for t in spass],
        "roofline": {
            "bound": "hbm",
            "kernel": kname + (" (one step)" if how == "step" else ", launched with a precomputed amax"),
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": round(traffic) if traffic is not None else None,
            "launch_us": round(kms * 1e3, 3),
            "pass_launch_us": [round(t * 1e3, 3) for t in kpass],
            "bytes_per_launch": case.bytes,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

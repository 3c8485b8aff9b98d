"""Calls whose outputs must not depend on launch geometry (grid sizes, tile order, encode mapping).

Used by tests/test_gpu_geometry.py in the test process and, with other NVFP4Q_* launch settings, in a
child process (run as a script: `python tests/geometry_calls.py OUT.npz`). Inputs are seeded and small
but span several workgroups and ragged tails. Only launch geometry differs between the two runs; the
arithmetic of every element is the same, so the outputs must agree bit for bit (block indices and SR
draws are functions of tile coordinates, not of the launch).
"""
import os
import sys

import numpy as np

if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import workloads  # noqa: E402

# child-process launch settings (every one only changes grid sizes, order or mapping)
CHILD_ENV = {
    "NVFP4Q_RMS_STREAM_WGS": "37",
    "NVFP4Q_RMS_ENCODE_WGS": "5",
    "NVFP4Q_RMS_COOP_WGS": "3",
    "NVFP4Q_XCD_ORDER": "0",
    "NVFP4Q_RMS_ROWWAVE_MIN": "1",
    "NVFP4Q_AMAX_WGS": "7",
}


def _bf16(rng, shape, scale=1.0):
    return workloads.to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def run_all(q):
    import torch

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()

    def host(t):
        return t.cpu().numpy() if t is not None else None

    def plane(t, width):
        # plane rows are padded to a multiple of 16 bytes; the padding is never written
        return host(t)[:, :width]

    out = {}
    rng = np.random.default_rng(31)
    x = _bf16(rng, (1536, 2048))
    g = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(2048)).astype(np.float32))
    r = q.rmsnorm_nvfp4q(dev(x), dev(g), eps=1e-6, y_out=True)
    out["rms_codes"], out["rms_scales"] = plane(r["codes"], 1024), plane(r["scales"], 128)
    for k in ("amax", "scale"):
        out["rms_" + k] = host(r[k]).view(np.uint8)
    out["rms_y"] = host(r["y"].view(torch.int16))
    x = _bf16(rng, (300, 1024), 2.0)
    g = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(1024)).astype(np.float32))
    b = workloads.to_bf16_bits((0.01 * rng.standard_normal(1024)).astype(np.float32))
    r = q.rmsnorm_nvfp4q(dev(x), dev(g), dev(b), eps=1e-6, rounding="sr", seed=9, offset=4)
    out["rmsb_codes"], out["rmsb_scales"] = plane(r["codes"], 512), plane(r["scales"], 64)
    for k in ("amax", "scale"):
        out["rmsb_" + k] = host(r[k]).view(np.uint8)
    x = _bf16(rng, (700, 4096))
    g = workloads.to_bf16_bits((1 + 0.1 * rng.standard_normal(4096)).astype(np.float32))
    r = q.rmsnorm_nvfp4q(dev(x), dev(g), eps=1e-6, amax=torch.tensor([5.5], device="cuda"))
    out["rmsa_codes"], out["rmsa_scales"] = plane(r["codes"], 2048), plane(r["scales"], 256)
    for dt in ("float16", "float32"):
        tdt = getattr(torch, dt)
        x = torch.from_numpy((rng.standard_normal((520, 1040)) * 2).astype(np.float32)).to(tdt).cuda()
        g = torch.from_numpy((1 + 0.1 * rng.standard_normal(1040)).astype(np.float32)).to(tdt).cuda()
        b = torch.from_numpy((0.01 * rng.standard_normal(1040)).astype(np.float32)).to(tdt).cuda()
        for bias in (False, True):
            r = q.rmsnorm_nvfp4q(x, g, b if bias else None, eps=1e-6, y_out=True, rounding="sr", seed=2, offset=6)
            key = f"rms_{dt}_{int(bias)}_"
            out[key + "codes"], out[key + "scales"] = plane(r["codes"], 520), plane(r["scales"], 65)
            for k in ("amax", "scale"):
                out[key + k] = host(r[k]).view(np.uint8)
            out[key + "y"] = host(r["y"]).view(np.uint8)
    x = _bf16(rng, (777, 1536), 3.0)
    r = q.nvfp4q_quantize(dev(x), rounding="sr", seed=3, offset=1)
    out["q_codes"], out["q_scales"] = plane(r["codes"], 768), plane(r["scales"], 96)
    out["q_amax"] = host(r["amax"]).view(np.uint8)
    x = _bf16(rng, (640, 384))
    r = q.nvfp4q_quantize_2d(dev(x), rounding="sr", seed=5, offset=2)
    out["2d_row_codes"], out["2d_row_scales"] = plane(r["row_codes"], 192), plane(r["row_scales"], 24)
    out["2d_col_codes"], out["2d_col_scales"] = plane(r["col_codes"], 320), plane(r["col_scales"], 40)
    out["2d_amax"] = host(r["amax"]).view(np.uint8)
    counts = rng.multinomial(1000, np.full(8, 1 / 8))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = _bf16(rng, (1000, 512))
    r = q.nvfp4q_grouped(dev(x), torch.tensor(offsets, device="cuda"), apply_rht=True, rht_mask=0x3C5A,
                         rounding="sr", seed=7, offset=3)
    mpad = int(host(r["poff"])[-1])  # plane storage past the last padded column is never written
    out["g_codes"] = host(r["codes"])[:, : mpad // 2]
    out["g_scales"] = host(r["scales"])[:, : mpad // 16]
    for k in ("amax", "poff"):
        out["g_" + k] = host(r[k]).view(np.uint8)
    r = q.nvfp4q_grouped(dev(x), torch.tensor(offsets, device="cuda"), apply_rht=True, rht_mask=0x3C5A,
                         rounding="sr", seed=7, offset=3, rowwise=True)
    out["gr_row_codes"], out["gr_row_scales"] = plane(r["row_codes"], 256), plane(r["row_scales"], 32)
    out["gr_row_amax"] = host(r["row_amax"]).view(np.uint8)
    x = _bf16(rng, (3 * 160, 272))
    r = q.nvfp4q_quantize_2d_grouped(dev(x), 3, rounding="sr", seed=6, offset=1, tile16=True)
    out["e_row_codes"], out["e_row_scales"] = plane(r["row_codes"], 136), plane(r["row_scales"], 17)
    out["e_col_codes"], out["e_col_scales"] = plane(r["col_codes"], 80), plane(r["col_scales"], 10)
    out["e_amax"] = host(r["amax"]).view(np.uint8)
    xf = (rng.standard_normal((513, 1040)) * 4).astype(np.float32)
    r = q.nvfp4q_quantize(torch.from_numpy(xf).cuda(), rounding="sr", seed=8)
    out["qf_codes"], out["qf_scales"] = plane(r["codes"], 520), plane(r["scales"], 65)
    out["qf_amax"] = host(r["amax"]).view(np.uint8)
    return out


if __name__ == "__main__":
    import rmsnorm_nvfp4_block_amd as q

    np.savez(sys.argv[1], **run_all(q))

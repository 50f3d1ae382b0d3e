"""Benchmark of the FFN block hot path on one MI355X.

One step = one pass of the whole hot path over the Qwen2-7B-shaped FP8
workload: the prefill block over N=8192 token rows (C=3584, H=18944, eps 1e-6):
fused residual RMSNorm with abs-max, e4m3 quantisation, fused gate+up GEMM with
the SwiGLU epilogue, e4m3 quantisation of h, down GEMM; then the 16-token FP8
decode FFN (dual gate/up GEMV with SiLU, down GEMV) over the same e4m3 weights
with per-row scales.  Inputs are seeded synthetic tensors already resident in
HBM when the timed region starts.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]

Prints one JSON line.  value = whole-step algorithmic FLOP/s (the block's dense
contractions: 6*N*C*H for the prefill, 6*M*C*H for the decode).  "roofline"
describes the dominant kernel (the FP8 gate+up GEMM) from HIP events recorded
on its own stream around every launch in the timed steps; "cpu_baseline" times
the CPU oracle on a bounded sample of the same workload.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FFN-block TFLOP/s (fp8/bf16 prefill) and decode GEMV HBM GB/s, % of peak"
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
WORKLOAD = "qwen7b8"
DECODE_COPIES = 3           # rotating decode weight copies: 3 x 204 MB > 256 MB MALL
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SRC = os.path.join(ROOT, "transformer_ffn_block_residual_amd", "csrc", "gemm.hip")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=256, help="prefill rows in the CPU oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (HBM counter calibration under rocprofv3 --pmc)")
    return p.parse_args()


def gemm_traffic():
    """HBM bytes per gate+up launch from committed rocprofv3 counter runs, or
    None when the GEMM source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        src = hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()
        if rec.get("gemm_src_sha256") != src:
            return None
        return rec.get("gateup_bytes_per_launch")
    except (OSError, ValueError):
        return None


def cpu_baseline(w, d, dec_x, rows):
    """The oracle, untuned, on a bounded sample: a prefill block over `rows` of
    the workload's token rows plus the full 16-token decode, weights quantised
    beforehand (outside the timed region, as on the device)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default
        threads = os.cpu_count() or 1
    qw_gu, s_gu, _ = O.quant_absmax(d["w_gu"])
    qw_d, s_d, _ = O.quant_absmax(d["w_d"])
    H, C = w.H, w.C
    sgv = np.full(H, s_gu, np.float32)
    sdv = np.full(C, s_d, np.float32)
    inp, add = d["inp"][:rows], d["addend"][:rows]
    t0 = time.perf_counter()
    r, y, rstd, am_y = O.rmsnorm_fwd(inp, add, d["w_norm"], w.eps)
    qy, sy, _ = O.quant_absmax(y, am_y)
    h, am_h = O.swiglu(O.gemm_fp8(qy, sy, qw_gu, s_gu))
    qh, sh, _ = O.quant_absmax(h, am_h)
    O.gemm_fp8(qh, sh, qw_d, s_d)
    O.decode_gemv(dec_x, qw_gu[:H], sgv, qw_gu[H:], sgv, qw_d, sdv)
    dt = time.perf_counter() - t0
    flops = 6.0 * rows * C * H + 6.0 * w.decode_M * C * H
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"prefill block over the first {rows} of {w.N} token rows + the full {w.decode_M}-token "
                      f"decode, FP8 weights quantised beforehand; {dt:.2f} s wall"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the FFN block path here has no "
              "multi-GPU mode.", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from transformer_ffn_block_residual_amd import block, binding as B, workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = W.WORKLOADS[WORKLOAD]
    N, C, H, M = w.N, w.C, w.H, w.decode_M
    print(f"[bench] generating {WORKLOAD} inputs (seed {w.seed})", file=sys.stderr, flush=True)
    d = W.block_inputs(N, C, H, w.seed, w.w_std, w.outliers)
    dec_x = W.decode_inputs(M, C, H, w.seed, with_weights=False)["x"]

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    pre = block.PrefillBlock(N, C, H, w.eps, True)
    pre.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    inp, addend = dev(d["inp"]), dev(d["addend"])
    x_dec = dev(dec_x)
    decs = []
    for _ in range(DECODE_COPIES):
        db = block.DecodeBlock(M, C, H)
        wgu = pre.w_gu.clone()
        sg = pre.s_gu.expand(H).contiguous()
        db.set_fp8_weights(wgu[:H], sg, wgu[H:], sg.clone(), pre.w_d.clone(), pre.s_d.expand(C).contiguous())
        decs.append(db)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = {k: [] for k in ("rms", "q_y", "gateup", "q_h", "down", "decode")}

    def step(i, record):
        def mark():
            e = torch.cuda.Event(enable_timing=True)
            e.record(stream)
            return e
        e0 = mark() if record else None
        B.ffn_rmsnorm_fwd(pre.y, pre.rstd, pre.r, pre.am_y, inp, addend, pre.w_norm, pre.eps, N, C, stream)
        e1 = mark() if record else None
        B.ffn_quant_absmax(pre.qy, pre.s_y, pre.am_y, pre.y, N * C, 0, stream)
        e2 = mark() if record else None
        B.ffn_gateup(pre.h, pre.am_h, pre.qy, pre.s_y, pre.w_gu, pre.s_gu, B.FFN_E4M3, 1, N, C, H, stream)
        e3 = mark() if record else None
        B.ffn_quant_absmax(pre.qh, pre.s_h, pre.am_h, pre.h, N * H, 0, stream)
        e4 = mark() if record else None
        B.ffn_down(pre.out, pre.qh, pre.s_h, pre.w_d, pre.s_d, B.FFN_E4M3, N, H, C, stream)
        e5 = mark() if record else None
        decs[i % DECODE_COPIES].forward(x_dec, M, stream)
        e6 = mark() if record else None
        if record:
            for k, (s, t) in zip(ev, [(e0, e1), (e1, e2), (e2, e3), (e3, e4), (e4, e5), (e5, e6)]):
                ev[k].append((s, t))

    for i in range(a.warmup):
        step(i, False)
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {a.steps} steps", file=sys.stderr, flush=True)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(a.steps):
        step(i, True)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / a.steps

    kern_ms = {k: float(np.mean([s.elapsed_time(t) for s, t in v])) for k, v in ev.items()}
    flops_gateup = 4.0 * N * C * H
    flops_step = 6.0 * N * C * H + 6.0 * M * C * H
    gu_tflops = flops_gateup / (kern_ms["gateup"] * 1e-3) / 1e12
    traffic = gemm_traffic()
    dec_bytes = 3.0 * H * C + (2 * H + C) * 4 + 2.0 * M * (C + H) * 2
    kernels = {
        "rmsnorm_fwd": {"ms": kern_ms["rms"], "GB/s": (4 * N * C * 2 + N * 4 + C * 2) / kern_ms["rms"] / 1e6},
        "quant_y": {"ms": kern_ms["q_y"], "GB/s": (N * C * 3) / kern_ms["q_y"] / 1e6},
        "gateup_fp8_swiglu": {"ms": kern_ms["gateup"], "TFLOP/s": gu_tflops},
        "quant_h": {"ms": kern_ms["q_h"], "GB/s": (N * H * 3) / kern_ms["q_h"] / 1e6},
        "down_fp8": {"ms": kern_ms["down"], "TFLOP/s": 2.0 * N * C * H / (kern_ms["down"] * 1e-3) / 1e12},
        "decode_m16": {"ms": kern_ms["decode"], "GB/s": dec_bytes / kern_ms["decode"] / 1e6,
                       "frac_hbm": dec_bytes / kern_ms["decode"] / 1e6 / PEAK_HBM_GBS},
    }
    out = {
        "metric": METRIC,
        "value": flops_step / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {"workload": "qwen2-7b-shaped FFN block, FP8: prefill N=8192 C=3584 H=18944 eps=1e-6 "
                               "+ 16-token FP8 row-scaled decode on the same weights",
                   "N": N, "C": C, "H": H, "decode_M": M, "seed": w.seed,
                   "quant": "per-tensor abs-max e4m3 activations and weights; decode: e4m3 weights, "
                            "per-row fp32 scales, bf16 activations"},
        "roofline": {"bound": "mfma", "kernel": "ffn_gateup (e4m3, fused SwiGLU)",
                     "achieved": gu_tflops, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": gu_tflops / PEAK_FP8_TFLOPS, "traffic": traffic},
        "kernels": kernels,
    }
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, d, dec_x, a.cpu_rows)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())

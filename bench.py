"""Benchmark of the FFN block hot path on one MI355X.

Default step (--workload qwen7b8): one pass of the whole hot path over the
Qwen2-7B-shaped FP8 workload: the prefill block over N=8192 token rows
(C=3584, H=18944, eps 1e-6): fused residual RMSNorm with abs-max, e4m3
quantisation, fused gate+up GEMM with the SwiGLU epilogue, e4m3 quantisation of
h, down GEMM; then the 16-token FP8 decode FFN (dual gate/up GEMV with SiLU,
down GEMV) over the same e4m3 weights with per-row scales.  Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts.

The default run also times the other configurations, each in the same way,
and puts them in the line's "configs" record (each with its own roofline line
and CPU baseline); --workload prints one of them as the line itself:
  prefill   bf16 block, N=4096, C=4096, H=14336
  prefill8  FP8 block, same shape, 0.1% x50 outliers
  decode    single-token FP8 decode, C=4096, H=14336 (value in GB/s);
            --decode-arm picks the arm (split SiLU, fused SiLU input,
            per projection, or bf16 weights), --decode-m the tokens (1..32)

    python bench.py [--gpus 1] [--steps 20] [--warmup 25] [--workload W] [--no-configs] [--no-cpu-baseline]

Prints one JSON line.  For block workloads value = whole-step algorithmic
FLOP/s (the block's dense contractions: 6*N*C*H for the prefill, 6*M*C*H for
the decode); for the decode workload value = algorithmic HBM bytes (weights +
scales + activations, each once) per second.  "roofline" describes the
dominant kernel from HIP events recorded on its launch stream around every
launch of a second pass of the same steps (the timed region itself carries
only its two bracketing events); "cpu_baseline" times the CPU oracle on a bounded
sample of the same workload: the C++ oracle (fp32, std::thread over rows)
for the forward and the FP8 decode, with the CPU model and core counts.
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
PEAK = {"fp8": 5000.0, "bf16": 2500.0}   # MI355X dense MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0                    # MI355X HBM3E
DECODE_COPIES = 3                        # rotating decode weight copies: > 256 MB MALL
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# decode arms: (ffn_decode_gemv_arm arm, or None for ffn_decode_gemv / "bf16"
# for ffn_decode_gemv_bf16; description)
DECODE_ARMS = {
    "split": (None, "split SiLU: dual gate/up GEMV with silu_mul in its epilogue, then the down GEMV"),
    "silu_input": (1, "fused SiLU input: dual gate/up GEMV to g|u, then the down GEMV forming silu(g)*u itself"),
    "per_projection": (2, "per projection: gate GEMV, up GEMV, silu_mul, down GEMV"),
    "bf16": ("bf16", "bf16 weights: dense gate/up GEMV with silu_mul, then the dense down GEMV"),
}
CSRC = os.path.join(ROOT, "transformer_ffn_block_residual_amd", "csrc")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=25)
    p.add_argument("--workload", default=None, choices=["qwen7b8", "prefill", "prefill8", "decode"],
                   help="one workload's line only (default: the qwen7b8 step, with the other configurations "
                        "in its 'configs' record)")
    p.add_argument("--no-configs", action="store_true",
                   help="default run: leave out the 'configs' record of the other configurations")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="prefill rows in the CPU oracle sample (default: all N rows, 10-30 s on 16 threads)")
    p.add_argument("--cpu-decodes", type=int, default=30,
                   help="decode calls in the CPU oracle sample of the decode workload (about 10 s)")
    p.add_argument("--decode-arm", default="split", choices=list(DECODE_ARMS),
                   help="decode workload: which arm of the decode FFN runs")
    p.add_argument("--decode-m", type=int, default=1,
                   help="decode workload: tokens per call (1..32 on the split arm, 1..4 on the others)")
    p.add_argument("--backward", action="store_true",
                   help="block workloads: time the FFN block backward (after one forward) instead of the forward")
    p.add_argument("--decode-layout", default="auto", choices=["auto", "rows", "packed"],
                   help="FP8 decode weights: row-major (ffn_decode_gemv) or the packed decode layout "
                        "(ffn_decode_gemv_packed); auto: packed from 4 tokens on, row-major below")
    p.add_argument("--decode-at", default="end", choices=["end", "start", "mid"],
                   help="qwen7b8: where the decode runs in the step's one stream: after the down GEMM, "
                        "before the RMSNorm, or between the quantisation of y and the gate+up GEMM")
    p.add_argument("--decode-overlap", default="none", choices=["none", "tail", "start"],
                   help="qwen7b8: where the step's decode runs.  none: after the down GEMM on the same stream; "
                        "tail: on a second stream from the end of the h quantisation on, beside the down GEMM "
                        "(whose persistent grid leaves 32 CUs free); start: on a second stream from the start of "
                        "the step.  Each step joins the second stream before it ends.  Both overlaps measure "
                        "slower than none (the decode needs more than the free CUs)")
    p.add_argument("--concurrent-backward", action="store_true",
                   help="backward: each projection's weight gradient on a second stream beside its data gradient, "
                        "one workgroup per tile (measured no faster than the default single stream); the per-phase "
                        "times always come from the serial order")
    p.add_argument("--unfused-swiglu-bwd", action="store_true",
                   help="backward: the down projection's data gradient and the SwiGLU backward as two calls "
                        "(ffn_matmul_tn, ffn_swiglu_bwd) instead of ffn_matmul_tn_swiglu_bwd")
    p.add_argument("--grad-dtype", default="e4m3", choices=["e4m3", "e5m2"],
                   help="FP8 backward: the format of the quantised gradients (weights and activations stay e4m3)")
    p.add_argument("--gemm-layout", default="tiled", choices=["tiled", "rows"],
                   help="block workloads: the GEMM operands (weights; y and h, or their e4m3 codes) in the tiled "
                        "layout (ffn_tile_pack; every GEMM load one contiguous KiB) or row-major")
    p.add_argument("--known-h-absmax", action="store_true",
                   help="FP8 block workloads: quantise h in the gate+up epilogue with the previous step's abs-max "
                        "(ffn_gateup_swiglu_quant, the recompute form) instead of bf16 h + ffn_quant_absmax")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (HBM counter calibration under rocprofv3 --pmc)")
    p.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no benchmark: turn the counter_collection.csv files of a FETCH_SIZE and a WRITE_SIZE "
                        "rocprofv3 run of this script (--copy-calibration) into the workload's entry of "
                        "profiles/traffic.json")
    a = p.parse_args()
    if a.grad_dtype != "e4m3" and not a.backward:
        p.error("--grad-dtype applies to the backward (--backward)")
    return a


def src_digest(name):
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()


def measured_traffic(key, src):
    """HBM bytes per launch of kernel `key` from committed rocprofv3 counter
    runs, or None when its source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[key]
        if rec.get("src_sha256") != src_digest(src):
            return None
        return rec.get("bytes_per_launch")
    except (OSError, ValueError, KeyError):
        return None


# kernels with counter entries per workload: traffic.json key, source file,
# the kernel name fragments whose per-dispatch counters make up one launch of
# the entry point, which dispatches are that launch, and its algorithmic bytes
def traffic_specs(workload, known_h_absmax=False, backward=False, grad_dtype="e4m3", rows_layout=False):
    """[(traffic.json key, source file, kernel-name fragments of one launch,
    description, algorithmic bytes of one launch, (skip, stride, offset))],
    the dominant kernel first.  Matching dispatches are taken from the
    skip-th on, every stride-th from offset: the backward's two
    weight-gradient GEMMs share one kernel (the up projection's is the second
    of each step), and the forward's two row-major activation quantisations
    share one kernel after the two weight quantisations of the set-up.  The
    forward's GEMMs (and FP8 quantisations) run on tiled operands unless
    rows_layout; the row-major forms' keys carry "_rows"."""
    from transformer_ffn_block_residual_amd import workloads as W
    w = W.WORKLOADS[workload]
    N, C, H = w.N, w.C, w.H
    if backward:
        e = 1 if w.fp8 else 2
        fp8 = "true" if w.fp8 else "false"
        e5 = w.fp8 and grad_dtype == "e5m2"
        what = ("e5m2 x e4m3" if e5 else "e4m3") if w.fp8 else "bf16"
        # the FP8 backward's products read tiled operands unless rows_layout
        btl = w.fp8 and not rows_layout
        # reads dgu^T [2H, N] and y^T [C, N] once, reads and writes dW_gu [2H, C]
        return [(f"dwup{'5' if e5 else ''}{'_rows' if w.fp8 and rows_layout else ''}_{workload}", "gemm.hip",
                 [f"gemm_kernel<{fp8}, false, false, true, {'true' if e5 else 'false'}, false, "
                  f"{'true' if btl else 'false'}>"],
                 f"gemm_kernel ({what}, accumulating{', tiled operands' if btl else ''}) of the up projection's weight "
                 f"gradient, [2H, C] = [{2 * H}, {C}], K = N = {N}",
                 2 * H * N * e + C * N * e + 2 * (2 * H * C * 2), (0, 2, 1))]
    if workload == "decode":
        return [("decode_decode", "decode.hip", ["gemv_small_kernel<0, false, 1,", "gemv_small_kernel<2, false, 1,"],
                 f"gemv_small_kernel<dual SiLU> + gemv_small_kernel<single> (one ffn_decode_gemv), M=1 C={C} H={H}",
                 3 * H * C + (2 * H + C) * 4 + 2 * (C + H) * 2, (0, 1, 0))]
    elt = 1 if w.fp8 else 2
    fp8 = "true" if w.fp8 else "false"
    dt = "e4m3" if w.fp8 else "bf16"
    tiled = not rows_layout
    tl = "true" if tiled else "false"
    lay = ", tiled operands" if tiled else ""
    tag = "_rows" if rows_layout else ""
    every = (0, 1, 0)
    if known_h_absmax:
        # reads x and w, writes the e4m3 codes of h
        return [(f"gateupq{tag}_{workload}", "gemm.hip", [f"gemm_kernel<{fp8}, true, true, false, false, false, {tl}>"],
                 f"gemm_kernel (e4m3, fused SwiGLU + e4m3 quantisation{lay}) of ffn_gateup_swiglu_quant"
                 f"{'_tiled' if tiled else ''}, N={N} C={C} H={H}", N * C * elt + 2 * H * C * elt + N * H, every)]
    specs = [
        (f"gateup{tag}_{workload}", "gemm.hip", [f"gemm_kernel<{fp8}, true, false, false, false, false, {tl}>"],
         f"gemm_kernel ({dt}, fused SwiGLU{lay}) of ffn_gateup"
         f"{('_acc_tiled' if w.fp8 else '_tiled_bf16') if tiled else ''}, N={N} C={C} H={H}",
         N * C * elt + 2 * H * C * elt + N * H * 2, every),
        (f"down{tag}_{workload}", "gemm.hip", [f"gemm_kernel<{fp8}, false, false, false, false, false, {tl}>"],
         f"gemm_kernel ({dt}{lay}) of ffn_down{('_tiled' if w.fp8 else '_tiled_bf16') if tiled else ''}, "
         f"N={N} H={H} C={C}",
         N * H * elt + C * H * elt + N * C * 2, every),
        # reads inp and addend, writes r and y, rstd; the weight once
        # (the bf16 block's RMSNorm stores y for the tiled GEMM: a form of its own)
        (f"rmsnorm{'' if w.fp8 else tag}_{workload}", "norm_quant.hip", ["rmsnorm_kernel<"],
         f"rmsnorm_kernel (residual add + RMSNorm + rstd{' + abs-max' if w.fp8 else ''}) of ffn_rmsnorm_fwd, "
         f"N={N} C={C}",
         4 * N * C * 2 + N * 4 + C * 2, every),
    ]
    if w.fp8:
        # row-major: after the two weight quantisations, y and h alternate on
        # quant_kernel; tiled: y and h alternate on quant_tiled_kernel
        qk = "quant_tiled_kernel(" if tiled else "quant_kernel("
        specs += [(f"quant_{t}{tag}_{workload}", "norm_quant.hip", [qk],
                   f"{qk[:-1]} (per-tensor e4m3 with a given abs-max{', tiled codes' if tiled else ''}) of {t}, "
                   f"{N} x {K}", 3 * N * K, (0 if tiled else 2, 2, o)) for t, K, o in (("y", C, 0), ("h", H, 1))]
    if w.decode_M:
        M = w.decode_M
        specs.append((f"decode{M}_{workload}", "decode.hip",
                      ["decode_dual_wave_kernel<", "decode_down_split_kernel<", "decode_down_reduce_kernel("],
                      f"decode_dual_wave_kernel + decode_down_split_kernel + decode_down_reduce_kernel (one "
                      f"ffn_decode_gemv_packed), M={M} C={C} H={H}",
                      3 * H * C + (2 * H + C) * 4 + 2 * M * (C + H) * 2, every))
    return specs


def traffic_spec(workload, known_h_absmax=False, backward=False, grad_dtype="e4m3", rows_layout=False):
    """The dominant kernel's entry of traffic_specs."""
    return traffic_specs(workload, known_h_absmax, backward, grad_dtype, rows_layout)[0]


def ingest_pmc(a):
    """HBM bytes per launch of the workload's kernels (traffic_specs) from two
    rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each
    scaled by what the counter reads for the 1 GiB calibration copy."""
    import csv
    tables = {}
    for counter, path in (("FETCH_SIZE", a.ingest_pmc[0]), ("WRITE_SIZE", a.ingest_pmc[1])):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not copies:
            raise SystemExit(f"{path}: no calibration copy (run bench.py with --copy-calibration)")
        tables[counter] = (rows, (1 << 20) / max(copies))
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    for key, src, frags, desc, algo, (skip, stride, offset) in traffic_specs(
            a.workload, a.known_h_absmax, a.backward, a.grad_dtype, rows_layout=a.gemm_layout == "rows"):
        rec = {"kernel": desc, "src": f"transformer_ffn_block_residual_amd/csrc/{src}",
               "src_sha256": src_digest(src)}
        total = 0.0
        for counter, (rows, factor) in tables.items():
            per_launch = 0.0
            for f in frags:
                vals = [float(r["Counter_Value"]) for r in rows if f in r["Kernel_Name"]]
                vals = vals[skip:][offset::stride]
                if not vals:
                    raise SystemExit(f"no dispatch of {f} with {counter}")
                per_launch += sum(vals) / len(vals)
            tag = counter.split("_")[0].lower()
            rec[f"{tag}_kb_raw"] = per_launch
            rec[f"{tag}_factor"] = factor
            total += per_launch * factor * 1024
        rec["bytes_per_launch"] = total
        rec["algorithmic_bytes"] = algo
        data[key] = rec
        print(json.dumps({key: rec}))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    return 0


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default
        return os.cpu_count() or 1


def host_desc():
    """The host the CPU baseline runs on: CPU model, logical CPUs this process
    may use, physical cores of the machine."""
    from oracle import cpp
    model, _, physical = cpp.cpu_info()
    return {"cpu_model": model, "logical_cpus": cpp.threads(), "physical_cores": physical}


def cpu_block_sample(w, d, rows, dec_x=None):
    """The C++ oracle (fp32, std::thread over rows on every CPU this process
    may use), untuned, on one block over the first `rows` token rows (plus
    the full decode batch when given); FP8 weights quantised beforehand,
    outside the timed region, as on the device."""
    import numpy as np
    from oracle import cpp as P
    H, C = w.H, w.C
    if w.fp8:
        qw_gu, s_gu, _ = P.quant_absmax(d["w_gu"])
        qw_d, s_d, _ = P.quant_absmax(d["w_d"])
    inp, add = d["inp"][:rows], d["addend"][:rows]
    t0 = time.perf_counter()
    r, y, rstd, am_y = P.rmsnorm_fwd(inp, add, d["w_norm"], w.eps)
    if w.fp8:
        qy, sy, _ = P.quant_absmax(y, am_y)
        h, am_h = P.swiglu(P.gemm_fp8(qy, sy, qw_gu, s_gu))
        qh, sh, _ = P.quant_absmax(h, am_h)
        P.gemm_fp8(qh, sh, qw_d, s_d)
    else:
        h, _ = P.swiglu(P.gemm_bf16(y, d["w_gu"]))
        P.gemm_bf16(h, d["w_d"])
    flops = 6.0 * rows * C * H
    what = f"prefill block over {'all' if rows == w.N else 'the first'} {rows} of {w.N} token rows"
    if dec_x is not None:
        sgv = np.full(H, s_gu, np.float32)
        sdv = np.full(C, s_d, np.float32)
        P.decode_gemv(dec_x, qw_gu[:H], sgv, qw_gu[H:], sgv, qw_d, sdv)
        flops += 6.0 * dec_x.shape[0] * C * H
        what += f" + the full {dec_x.shape[0]}-token decode"
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": P.threads(), "kind": "oracle",
            "impl": "C++ oracle, fp32, 16-way fixed-order sums, std::thread over rows",
            "sample": f"{what}; weights quantised beforehand; {dt:.2f} s wall", **host_desc()}


def cpu_decode_sample(d_q, x, calls):
    """The C++ oracle decode of x's M tokens over the full weights (already
    quantised), `calls` times, in GB/s of algorithmic bytes."""
    from oracle import cpp as P
    qg, sg, qu, su, qd, sd = d_q
    H, C = qg.shape
    M = x.shape[0]
    t0 = time.perf_counter()
    for _ in range(calls):
        P.decode_gemv(x, qg, sg, qu, su, qd, sd)
    dt = time.perf_counter() - t0
    nbytes = calls * (3.0 * H * C + (2 * H + C) * 4 + 2.0 * M * (C + H) * 2)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": P.threads(), "kind": "oracle",
            "impl": "C++ oracle, fp32, 16-way fixed-order sums, std::thread over rows",
            "sample": f"{calls} full {M}-token FP8 decodes (C={C}, H={H}); {dt:.2f} s wall", **host_desc()}


def cpu_decode_sample_bf16(d, calls):
    """The numpy oracle's bf16-weight decode, `calls` times, in GB/s of
    algorithmic bytes (the C++ oracle has no bf16-weight arm)."""
    import oracle as O
    H, C = d["w_gate"].shape
    M = d["x"].shape[0]
    t0 = time.perf_counter()
    for _ in range(calls):
        O.decode_gemv_bf16(d["x"], d["w_gate"], d["w_up"], d["w_down"])
    dt = time.perf_counter() - t0
    nbytes = calls * (6.0 * H * C + 2.0 * M * (C + H) * 2)
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": int(blas_threads()), "kind": "oracle",
            "impl": "numpy oracle, fp64 BLAS", "sample": f"{calls} full {M}-token bf16-weight decodes (C={C}, H={H}); "
            f"{dt:.2f} s wall", **host_desc()}


def graph_step_ms(torch, issue, steps):
    """Average duration of one step when `steps` steps are captured in one HIP
    graph and replayed: the path without host launch gaps.  issue(stream)
    issues the steps on the capturing stream; the path launches kernels only
    (its abs-max clearing is a kernel, not a memset), so the graph replays
    them exactly."""
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=side):
        issue(torch.cuda.current_stream())
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    t0.record()
    for _ in range(reps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * steps)


class Timer:
    """HIP events on the launch stream around each named part of a step
    (created before the timed region, so that a mark costs one record)."""

    def __init__(self, torch, stream, n_marks):
        self.torch, self.stream, self.ev = torch, stream, {}
        self.pool = [torch.cuda.Event(enable_timing=True) for _ in range(n_marks)]
        self.used = 0

    def mark(self, stream=None):
        e = self.pool[self.used]
        self.used += 1
        e.record(self.stream if stream is None else stream)
        return e

    def add(self, name, a, b):
        self.ev.setdefault(name, []).append((a, b))

    def mean_ms(self):
        import numpy as np
        return {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in self.ev.items()}

    def median_min_ms(self):
        import numpy as np
        out = {}
        for k, v in self.ev.items():
            t = [a.elapsed_time(b) for a, b in v]
            out[k] = {"median": float(np.median(t)), "min": float(np.min(t))}
        return out


def run_steps(torch, stream, step, a, marks_per_step=8):
    """W warmup steps, then the timed region: exactly K steps between two
    events, synchronised on both sides, with nothing else on the stream.  A
    second pass of K steps records events around every launch for the
    per-kernel times (each event pair costs the stream a few microseconds,
    which would distort a short step's total if it were in the timed region)."""
    for i in range(a.warmup):
        step(i, None)
    torch.cuda.synchronize()
    print(f"[bench] warmup done; timing {a.steps} steps", file=sys.stderr, flush=True)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(a.steps):
        step(i, None)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / a.steps
    timer = Timer(torch, stream, marks_per_step * a.steps)
    for i in range(a.steps):
        step(a.steps + i, timer)
    torch.cuda.synchronize()
    run_steps.spread = timer.median_min_ms()
    return ms, timer.mean_ms()


def decode_packed(a, M):
    """Whether the FP8 split-SiLU decode of M tokens runs on packed weights."""
    return a.decode_layout == "packed" or (a.decode_layout == "auto" and M >= 3)


def bench_block(a, torch, np, B, block, W):
    w = W.WORKLOADS[a.workload]
    N, C, H = w.N, w.C, w.H
    M = w.decode_M
    dt = "fp8" if w.fp8 else "bf16"
    print(f"[bench] generating {a.workload} inputs (seed {w.seed})", file=sys.stderr, flush=True)
    d = W.block_inputs(N, C, H, w.seed, w.w_std, w.outliers)
    dec_x = W.decode_inputs(M, C, H, w.seed, with_weights=False)["x"] if M else None

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    tiled = a.gemm_layout == "tiled"
    pre = block.PrefillBlock(N, C, H, w.eps, w.fp8, tiled=tiled)
    pre.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    inp, addend = dev(d["inp"]), dev(d["addend"])
    decs = []
    if M:
        x_dec = dev(dec_x)
        packed = decode_packed(a, M)
        for _ in range(DECODE_COPIES):
            db = (block.DecodeBlockPacked if packed else block.DecodeBlock)(M, C, H)
            wgu = pre.w_gu_rows.clone()
            sg = pre.s_gu.expand(H).contiguous()
            db.set_fp8_weights(wgu[:H], sg, wgu[H:], sg, pre.w_d_rows.clone(), pre.s_d.expand(C).contiguous())
            decs.append(db)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    E = B.FFN_E4M3 if w.fp8 else B.FFN_BF16
    known = a.known_h_absmax and w.fp8
    # the decode is independent of the prefill block: with an overlap it runs
    # on a second stream (the default priority, like every stream here)
    overlap = a.decode_overlap if M else "none"
    side = torch.cuda.Stream() if overlap != "none" else None
    fork_ev, join_ev = torch.cuda.Event(), torch.cuda.Event()
    if known:
        # ping-pong abs-max buffers: step i quantises with am[i % 2] and
        # records its own abs-max in am[(i + 1) % 2]; one ordinary forward
        # provides the first known value
        pre.forward_zero_once(inp, addend, stream)
        am_pp = [pre.am_h.clone(), torch.empty_like(pre.am_h)]
        torch.cuda.synchronize()

    def decode_on_side(i, tm, stream, forked=False):
        # forked: fork_ev was recorded on `stream` already (before the launch
        # that the decode is to run beside, so that that launch is queued first)
        if not forked:
            fork_ev.record(stream)
        side.wait_event(fork_ev)
        d0 = tm.mark(side) if tm else None
        decs[i % DECODE_COPIES].forward(x_dec, M, side)
        if tm:
            tm.add("decode", d0, tm.mark(side))
        join_ev.record(side)

    serial_at = a.decode_at if (M and overlap == "none") else None

    def decode_serial(i, tm, stream):
        d0 = tm.mark() if tm else None
        decs[i % DECODE_COPIES].forward(x_dec, M, stream)
        d1 = tm.mark() if tm else None
        if tm:
            tm.add("decode", d0, d1)
        return d1

    def step(i, tm, stream=stream):
        first = tm.mark() if tm else None
        if overlap == "start":
            decode_on_side(i, tm, stream)
        m0 = decode_serial(i, tm, stream) if serial_at == "start" else first
        # the abs-max words follow the zero-once convention: the FP8 chain
        # accumulates into words that the previous consumer cleared, so no
        # launch in the step exists only to clear one; bf16 takes no abs-max
        if known:
            B.ffn_rmsnorm_fwd(pre.y, pre.rstd, pre.r, pre.am_y, inp, addend, pre.w_norm, pre.eps, N, C, stream)
        elif w.fp8:
            B.ffn_rmsnorm_fwd_acc(pre.y, pre.rstd, pre.r, pre.am_y, inp, addend, pre.w_norm, pre.eps, N, C, stream)
        elif tiled:
            B.ffn_rmsnorm_fwd_tiled(pre.y, pre.rstd, pre.r, None, inp, addend, pre.w_norm, pre.eps, N, C, stream)
        else:
            B.ffn_rmsnorm_fwd(pre.y, pre.rstd, pre.r, None, inp, addend, pre.w_norm, pre.eps, N, C, stream)
        m1 = tm.mark() if tm else None
        if known:
            if tiled:
                B.ffn_quant_absmax_clear_tiled(pre.qy, pre.s_y, pre.am_y, pre.y, N, C, None, stream)
            else:
                B.ffn_quant_absmax(pre.qy, pre.s_y, pre.am_y, pre.y, N * C, 0, stream)
            m2 = tm.mark() if tm else None
            if tiled:
                B.ffn_gateup_swiglu_quant_tiled(pre.qh, pre.s_h, am_pp[(i + 1) % 2], am_pp[i % 2], pre.qy,
                                                pre.s_y, pre.w_gu, pre.s_gu, N, C, H, stream)
            else:
                B.ffn_gateup_swiglu_quant(pre.qh, pre.s_h, am_pp[(i + 1) % 2], am_pp[i % 2], pre.qy, pre.s_y,
                                          pre.w_gu, pre.s_gu, E, N, C, H, stream)
            m3 = tm.mark() if tm else None
            m4 = m3
            if overlap == "tail":
                fork_ev.record(stream)
            if tiled:
                B.ffn_down_tiled(pre.out, pre.qh, pre.s_h, pre.w_d, pre.s_d, N, H, C, stream)
            else:
                B.ffn_down(pre.out, pre.qh, pre.s_h, pre.w_d, pre.s_d, E, N, H, C, stream)
        elif w.fp8:
            if tiled:
                B.ffn_quant_absmax_clear_tiled(pre.qy, pre.s_y, pre.am_y, pre.y, N, C, pre.am_h, stream)
            else:
                B.ffn_quant_absmax_clear(pre.qy, pre.s_y, pre.am_y, pre.y, N * C, pre.am_h, stream)
            m2 = tm.mark() if tm else None
            m2q = m2
            if serial_at == "mid":
                m2 = decode_serial(i, tm, stream)
            if tiled:
                B.ffn_gateup_acc_tiled(pre.h, pre.am_h, pre.qy, pre.s_y, pre.w_gu, pre.s_gu, N, C, H, stream)
            else:
                B.ffn_gateup_acc(pre.h, pre.am_h, pre.qy, pre.s_y, pre.w_gu, pre.s_gu, E, N, C, H, stream)
            m3 = tm.mark() if tm else None
            if tiled:
                B.ffn_quant_absmax_clear_tiled(pre.qh, pre.s_h, pre.am_h, pre.h, N, H, pre.am_y, stream)
            else:
                B.ffn_quant_absmax_clear(pre.qh, pre.s_h, pre.am_h, pre.h, N * H, pre.am_y, stream)
            m4 = tm.mark() if tm else None
            if overlap == "tail":
                fork_ev.record(stream)
            if tiled:
                B.ffn_down_tiled(pre.out, pre.qh, pre.s_h, pre.w_d, pre.s_d, N, H, C, stream)
            else:
                B.ffn_down(pre.out, pre.qh, pre.s_h, pre.w_d, pre.s_d, E, N, H, C, stream)
        else:
            m2 = m1
            if serial_at == "mid":
                m2 = decode_serial(i, tm, stream)
            if tiled:
                B.ffn_gateup_tiled_bf16(pre.h, None, pre.y, pre.w_gu, N, C, H, stream)
            else:
                B.ffn_gateup(pre.h, None, pre.y, None, pre.w_gu, None, E, 1, N, C, H, stream)
            m3 = tm.mark() if tm else None
            m4 = m3
            if overlap == "tail":
                fork_ev.record(stream)
            if tiled:
                B.ffn_down_tiled_bf16(pre.out, pre.h, pre.w_d, N, H, C, stream)
            else:
                B.ffn_down(pre.out, pre.h, None, pre.w_d, None, E, N, H, C, stream)
        if overlap == "tail":
            decode_on_side(i, tm, stream, forked=True)
        m5 = tm.mark() if tm else None
        last = m5
        if serial_at == "end":
            last = decode_serial(i, tm, stream)
        elif M and overlap != "none":
            stream.wait_event(join_ev)
            last = tm.mark() if tm else None
        if tm:
            tm.add("step", first, last)
            tm.add("rmsnorm", m0, m1)
            if w.fp8:
                tm.add("quant_y", m1, m2q if (w.fp8 and not known) else m2)
                if not known:
                    tm.add("quant_h", m3, m4)
            tm.add("gateup", m2, m3)
            tm.add("down", m4, m5)

    ms, km = run_steps(torch, stream, step, a, marks_per_step=10)
    spread = run_steps.spread

    def issue(cur):
        for i in range(a.steps):
            step(i, None, cur)
    graph_ms = graph_step_ms(torch, issue, a.steps)
    peak = PEAK[dt]
    gu_tflops = 4.0 * N * C * H / (km["gateup"] * 1e-3) / 1e12
    kernels = {
        "rmsnorm_fwd": {"ms": km["rmsnorm"], "GB/s": (4 * N * C * 2 + N * 4 + C * 2) / km["rmsnorm"] / 1e6},
        "gateup_swiglu": {"ms": km["gateup"], "TFLOP/s": gu_tflops, "frac_peak": gu_tflops / peak},
        "down": {"ms": km["down"], "TFLOP/s": 2.0 * N * C * H / (km["down"] * 1e-3) / 1e12,
                 "frac_peak": 2.0 * N * C * H / (km["down"] * 1e-3) / 1e12 / peak},
    }
    if w.fp8:
        kernels["quant_y"] = {"ms": km["quant_y"], "GB/s": N * C * 3 / km["quant_y"] / 1e6}
        if not known:
            kernels["quant_h"] = {"ms": km["quant_h"], "GB/s": N * H * 3 / km["quant_h"] / 1e6}
    flops = 6.0 * N * C * H
    cfg = {"workload": {"qwen7b8": "qwen2-7b-shaped FFN block, FP8: prefill N=8192 C=3584 H=18944 eps=1e-6 "
                                   "+ 16-token FP8 row-scaled decode on the same weights",
                        "prefill": "llama-shaped FFN block, bf16: prefill N=4096 C=4096 H=14336 eps=1e-5",
                        "prefill8": "llama-shaped FFN block, FP8: prefill N=4096 C=4096 H=14336 eps=1e-5, "
                                    "0.1% x50 outliers"}[a.workload],
           "N": N, "C": C, "H": H, "decode_M": M, "seed": w.seed,
           **({"decode_overlap": overlap, "decode_at": serial_at,
               "decode_layout": "packed" if decode_packed(a, M) else "rows"} if M else {}),
           "gemm_operands": "tiled" if tiled else "row-major",
           "quant": ("per-tensor abs-max e4m3 activations and weights" if w.fp8 else "none (bf16)")
           + ("; h quantised in the gate+up epilogue with the previous step's abs-max" if known else "")
           + ("; decode: e4m3 weights, per-row fp32 scales, bf16 activations" if M else "")}
    if M:
        dec_bytes = 3.0 * H * C + (2 * H + C) * 4 + 2.0 * M * (C + H) * 2
        kernels["decode"] = {"ms": km["decode"], "GB/s": dec_bytes / km["decode"] / 1e6,
                             "frac_hbm": dec_bytes / km["decode"] / 1e6 / PEAK_HBM_GBS}
        flops += 6.0 * M * C * H
    # HBM-side bytes per launch from the committed counter runs, where the
    # kernel's source is unchanged since they were taken
    names = {"gateup": "gateup_swiglu", "gateupq": "gateup_swiglu", "down": "down", "rmsnorm": "rmsnorm_fwd",
             "quant_y": "quant_y", "quant_h": "quant_h", f"decode{M}": "decode"}
    specs = traffic_specs(a.workload, known, rows_layout=not tiled)
    for key, src, _, _, algo, _ in specs:
        name = names.get(key[:-len(a.workload) - 1].replace("_rows", ""))
        if name in kernels:
            t = measured_traffic(key, src)
            kernels[name]["traffic"] = t
            kernels[name]["traffic_over_algorithmic"] = None if t is None else t / algo
    out = {
        "metric": METRIC, "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": cfg,
        "roofline": {"bound": "mfma", "kernel": ("ffn_gateup_swiglu_quant (e4m3, SwiGLU + e4m3 h)" if known else
                                                  f"ffn_gateup ({'e4m3' if w.fp8 else 'bf16'}, fused SwiGLU)")
                     + (", tiled operands" if tiled else ""),
                     "achieved": gu_tflops, "peak": peak, "unit": "TFLOP/s", "frac": gu_tflops / peak,
                     "traffic": measured_traffic(specs[0][0], "gemm.hip")},
        "kernels": kernels,
        "spread_ms": spread,
        "ms_per_step_in_hip_graph": graph_ms,
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_block_sample(w, d, a.cpu_rows or N, dec_x)
    return out


BWD_PHASES = {
    # phase: (kind, work) with work in flop ("mfma") or bytes ("hbm") given N, C, H, element bytes e
    # FP8: codes in both layouts from one read (abs-max handed over by its producer)
    "quant_dout": ("hbm", lambda N, C, H, e: 4 * N * C),
    # both weights transposed; made once per weight update, so only in the
    # first warmup step (listed if a timed step ever remakes them)
    "transpose_weights": ("hbm", lambda N, C, H, e: 6 * C * H * e),
    "dx_down": ("mfma", lambda N, C, H, e: 2 * N * C * H),
    # the same product with the SwiGLU backward in its epilogue (dh never stored)
    "dx_down_swiglu_bwd": ("mfma", lambda N, C, H, e: 2 * N * C * H),
    # bf16: the gradient and h transposed; FP8: the forward's codes of h
    "transpose_down_operands": ("hbm", lambda N, C, H, e: (4 * N * C if e == 2 else 0) + 2 * N * H * e),
    "dw_down": ("mfma", lambda N, C, H, e: 2 * N * C * H),
    "swiglu_bwd": ("hbm", lambda N, C, H, e: 10 * N * H),
    "quant_dgu": ("hbm", lambda N, C, H, e: 8 * N * H),
    "dx_up": ("mfma", lambda N, C, H, e: 4 * N * C * H),
    "transpose_up_operands": ("hbm", lambda N, C, H, e: (8 * N * H if e == 2 else 0) + 2 * N * C * e),
    "dw_up": ("mfma", lambda N, C, H, e: 4 * N * C * H),
    "rmsnorm_bwd": ("hbm", lambda N, C, H, e: 5 * N * C * 2 + N * 4),
}


def cpu_backward_sample(w, d, rows, grad_fmt="e4m3"):
    """The oracle forward + backward of the block over the first `rows` token
    rows (full weights; FP8 weights quantised beforehand, as in the forward
    sample); only the backward is timed."""
    import oracle as O
    import numpy as np
    d_out = _bwd_dout(np, w, rows)
    fwd = O.block_forward(d["inp"][:rows], d["addend"][:rows], d["w_norm"], d["w_gu"], d["w_d"], w.eps, fp8=w.fp8)
    t0 = time.perf_counter()
    O.block_backward(fwd, d_out, d["w_norm"], d["w_gu"], d["w_d"], fp8=w.fp8, grad_fmt=grad_fmt)
    dt = time.perf_counter() - t0
    flops = 12.0 * rows * w.C * w.H
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "impl": "numpy oracle, fp64 BLAS (the C++ oracle covers the forward only)",
            "sample": f"block backward over the first {rows} of {w.N} token rows (full weights); {dt:.2f} s wall",
            **host_desc()}


def _bwd_dout(np, w, rows):
    """The incoming gradient of the block output: ~N(0, 1) bf16, seeded."""
    from transformer_ffn_block_residual_amd import workloads as W
    g = np.random.default_rng([w.seed, 99]).standard_normal((rows, w.C), dtype=np.float32)
    return W.to_bf16_bits(g)


def bench_backward(a, torch, np, B, block, W):
    w = W.WORKLOADS[a.workload]
    N, C, H = w.N, w.C, w.H
    dt = "fp8" if w.fp8 else "bf16"
    e = 1 if w.fp8 else 2
    print(f"[bench] generating {a.workload} inputs (seed {w.seed}) for the backward", file=sys.stderr, flush=True)
    d = W.block_inputs(N, C, H, w.seed, w.w_std, w.outliers)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    pre = block.PrefillBlock(N, C, H, w.eps, w.fp8)
    pre.load_weights(d["w_norm"], d["w_gu"], d["w_d"])
    gd = a.grad_dtype if w.fp8 else "e4m3"
    # the zero-once abs-max convention, as in the forward step: no clearing launches in a step
    btiled = w.fp8 and a.gemm_layout == "tiled"
    bb = block.BackwardBlock(pre, in_place=False, grad_dtype=gd, fuse_swiglu_bwd=not a.unfused_swiglu_bwd,
                             concurrent=a.concurrent_backward, zero_once=True, tiled=btiled)
    bb.forward(dev(d["inp"]), dev(d["addend"]))
    d_out = dev(_bwd_dout(np, w, N))
    # the abs-max of d_out, as its producer (the next block's RMSNorm backward)
    # would hand it over
    am_dout = torch.empty(1, dtype=torch.float32, device="cuda")
    B.ffn_quant_absmax(bb.qdout if w.fp8 else torch.empty(N * C, dtype=torch.uint8, device="cuda"),
                       torch.empty(1, dtype=torch.float32, device="cuda"), am_dout, d_out, N * C, 1)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    names = list(BWD_PHASES)

    def step(i, tm, stream=stream):
        if tm is None:
            bb.backward(d_out, stream, d_out_absmax=am_dout)
            return
        marks = [tm.mark()]
        seen = []

        def mark(label):
            marks.append(tm.mark())
            seen.append(label)
        bb.backward(d_out, stream, mark, d_out_absmax=am_dout)
        tm.add("step", marks[0], marks[-1])
        for k, label in enumerate(seen):
            tm.add(label, marks[k], marks[k + 1])

    ms, km = run_steps(torch, stream, step, a, marks_per_step=16)
    spread = run_steps.spread

    def issue(cur):
        for i in range(a.steps):
            step(i, None, cur)
    graph_ms = graph_step_ms(torch, issue, a.steps)
    peak = PEAK[dt]
    kernels = {}
    for name in names:
        if name not in km:
            continue
        kind, work = BWD_PHASES[name]
        wv = work(N, C, H, e)
        if kind == "mfma":
            tf = wv / (km[name] * 1e-3) / 1e12
            kernels[name] = {"ms": km[name], "TFLOP/s": tf, "frac_peak": tf / peak}
        else:
            kernels[name] = {"ms": km[name], "GB/s": wv / km[name] / 1e6,
                             "frac_hbm": wv / km[name] / 1e6 / PEAK_HBM_GBS}
    flops = 12.0 * N * C * H
    dw_tf = kernels["dw_up"]["TFLOP/s"]
    out = {
        "metric": METRIC, "value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": f"FFN block backward of the {a.workload} workload: N={N} C={C} H={H}, "
                               + (("FP8 (per-tensor e4m3 weights, activations and gradients)" if gd == "e4m3" else
                                   "FP8 (per-tensor e4m3 weights and activations, e5m2 gradients)") if w.fp8
                                  else "bf16")
                               + "; down and up backward_qmm (data and weight gradients), SwiGLU and RMSNorm "
                                 "backward; the transposed weights are made once per weight update (before the timed steps) and "
                                 "reused; the abs-max of the incoming gradient comes "
                                 "with it (its producer, the next block's RMSNorm backward, writes it)",
                   "N": N, "C": C, "H": H, "seed": w.seed, "backward": True,
                   "swiglu_bwd": "two calls" if a.unfused_swiglu_bwd else "fused into the down data gradient",
                   "schedule": ("weight gradients on a second stream beside the data gradients"
                                if a.concurrent_backward else "one stream"),
                   "absmax": ("zero-once: dMlpUp's and d_res's words accumulated into, each cleared by the other's "
                              "consumer" if w.fp8 else "none (no quantised gradient)"),
                   **({"grad_dtype": gd, "gemm_operands": "tiled" if btiled else "row-major"} if w.fp8 else {})},
        "roofline": {"bound": "mfma", "kernel": f"ffn_matmul_tn ({(gd if w.fp8 else 'bf16')}, accumulate): "
                                                 "the up projection's weight gradient [2H, C], K = N",
                     "achieved": dw_tf, "peak": peak, "unit": "TFLOP/s", "frac": dw_tf / peak,
                     "traffic": measured_traffic(traffic_spec(a.workload, backward=True, grad_dtype=gd,
                                                              rows_layout=not btiled)[0], "gemm.hip")},
        "kernels": kernels,
        "spread_ms": spread,
        "ms_per_step_in_hip_graph": graph_ms,
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_backward_sample(w, d, a.cpu_rows or min(N, 256), gd)
    return out


def bench_decode(a, torch, np, B, block, W):
    w = W.WORKLOADS["decode"]
    M, C, H = a.decode_m, w.C, w.H
    arm, arm_what = DECODE_ARMS[a.decode_arm]
    bf16w = arm == "bf16"
    print(f"[bench] generating decode inputs (seed {w.seed}), arm {a.decode_arm}, M={M}", file=sys.stderr,
          flush=True)
    d = W.decode_inputs(M, C, H, w.seed, w.w_std)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    decs = []
    packed = False
    if bf16w:
        wts = [dev(d[k]) for k in ("w_gate", "w_up", "w_down")]
        for i in range(DECODE_COPIES):
            db = block.DecodeBlockBf16(M, C, H)
            db.load_weights(*(wts if i == 0 else [t.clone() for t in wts]))
            decs.append(db)
    else:
        packed = arm is None and decode_packed(a, M)
        first = block.DecodeBlock(M, C, H)
        first.load_master_weights(d["w_gate"], d["w_up"], d["w_down"])
        for i in range(DECODE_COPIES):
            if i == 0 and not packed:
                decs.append(first)
                continue
            # each copy its own weights (packed ones are packed from the first's rows)
            db = (block.DecodeBlockPacked if packed else block.DecodeBlock)(M, C, H)
            db.set_fp8_weights(first.wg.clone(), first.sg.clone(), first.wu.clone(), first.su.clone(),
                               first.wd.clone(), first.sd.clone())
            decs.append(db)
        if packed:
            del first
    x = dev(d["x"])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def bind_all(cur):
        if bf16w or arm is None:
            return [db.bind(x, M, cur) for db in decs]
        return [db.bind(x, M, cur, arm=arm) for db in decs]

    calls = bind_all(stream)

    def step(i, tm):
        m0 = tm.mark() if tm else None
        calls[i % DECODE_COPIES]()
        if tm:
            tm.add("decode", m0, tm.mark())

    ms, km = run_steps(torch, stream, step, a)
    spread = run_steps.spread
    # algorithmic bytes: each weight (and row scale) once, x, h and out once
    wbytes = (6.0 * H * C) if bf16w else (3.0 * H * C + (2 * H + C) * 4)
    nbytes = wbytes + 2.0 * M * (C + H) * 2
    gbs = nbytes / (ms * 1e-3) / 1e9

    def issue(cur):
        calls_g = bind_all(cur)
        for i in range(a.steps):
            calls_g[i % len(calls_g)]()
    graph_ms = graph_step_ms(torch, issue, a.steps)
    # a step is exactly one decode call (all of its kernels), so the call's
    # average duration is the timed region's; the event-bracketed pass reads
    # longer by the events' own cost and is reported beside it
    call_ms = ms
    wdesc = ("bf16" if bf16w else "e4m3 with per-row fp32 scales")
    entry = {None: "ffn_decode_gemv", "bf16": "ffn_decode_gemv_bf16"}.get(arm, "ffn_decode_gemv_arm")
    if not bf16w and arm is None and packed:
        entry = "ffn_decode_gemv_packed"
    default = a.decode_arm == "split" and M == 1 and not packed
    out = {
        "metric": METRIC, "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16w else "fp8", "data": "synthetic",
        "config": {"workload": f"{'single' if M == 1 else str(M)}-token decode FFN: x[{M},{C}] bf16, gate/up "
                               f"[{H},{C}] and down [{C},{H}] {wdesc}; {arm_what}",
                   "M": M, "C": C, "H": H, "seed": w.seed, "weight_copies": DECODE_COPIES, "arm": a.decode_arm,
                   **({} if bf16w else {"weight_layout": "packed" if packed else "rows"})},
        "roofline": {"bound": "hbm", "kernel": f"{entry} ({arm_what})",
                     "achieved": nbytes / (call_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": nbytes / (call_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": measured_traffic("decode_decode", "decode.hip") if default else None},
        "kernels": {"decode": {"ms": call_ms, "GB/s": nbytes / call_ms / 1e6,
                               "ms_between_events": km["decode"], "median_min_between_events": spread["decode"],
                               "ms_in_hip_graph": graph_ms, "GB/s_in_hip_graph": nbytes / graph_ms / 1e6}},
    }
    if not a.no_cpu_baseline:
        import oracle as O
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        if bf16w:
            out["cpu_baseline"] = cpu_decode_sample_bf16(d, a.cpu_decodes)
        else:
            qg, sg = O.quant_rows(d["w_gate"])
            qu, su = O.quant_rows(d["w_up"])
            qd, sd = O.quant_rows(d["w_down"])
            out["cpu_baseline"] = cpu_decode_sample((qg, sg, qu, su, qd, sd), d["x"], a.cpu_decodes)
    return out


# the per-configuration figures of the default run: (workload, decode tokens)
SUB_CONFIGS = (("decode", 1), ("prefill", 0), ("prefill8", 0))
SUB_KEYS = ("metric", "value", "unit", "ms_per_step", "dtype", "config", "roofline", "kernels", "spread_ms",
            "ms_per_step_in_hip_graph", "ms_in_hip_graph", "cpu_baseline")


def main():
    a = parse()
    if a.ingest_pmc:
        if a.workload is None:
            a.workload = "qwen7b8"
        return ingest_pmc(a)
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); this FFN block path has no "
              "multi-GPU mode.", file=sys.stderr)
        return 2

    import copy
    import gc

    import numpy as np
    import torch
    from transformer_ffn_block_residual_amd import block, binding as B, workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    all_configs = a.workload is None and not a.backward and not a.no_configs
    if a.workload is None:
        a.workload = "qwen7b8"
    if a.workload == "decode":
        out = bench_decode(a, torch, np, B, block, W)
    elif a.backward:
        out = bench_backward(a, torch, np, B, block, W)
    else:
        out = bench_block(a, torch, np, B, block, W)
    if all_configs:
        # the other configurations, each timed the same way (its own warmup
        # and K steps), with its own roofline line and CPU baseline
        out["configs"] = {}
        for name, m in SUB_CONFIGS:
            gc.collect()
            torch.cuda.empty_cache()
            sa = copy.copy(a)
            sa.workload, sa.decode_m, sa.decode_arm = name, (m or a.decode_m), "split"
            print(f"[bench] configuration {name}", file=sys.stderr, flush=True)
            sub = bench_decode(sa, torch, np, B, block, W) if name == "decode" else \
                bench_block(sa, torch, np, B, block, W)
            out["configs"][name] = {k: sub[k] for k in SUB_KEYS if k in sub}
        # and the FP8 block's backward at the same shape
        gc.collect()
        torch.cuda.empty_cache()
        sa = copy.copy(a)
        sa.workload, sa.backward = "qwen7b8", True
        print("[bench] configuration backward", file=sys.stderr, flush=True)
        sub = bench_backward(sa, torch, np, B, block, W)
        out["configs"]["backward"] = {k: sub[k] for k in SUB_KEYS if k in sub}
    if a.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())

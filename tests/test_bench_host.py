"""bench.py's host logic without a GPU: the one-GPU contract, the algorithmic
byte counts behind each roofline line, and the reduction of rocprofv3
counter files to per-launch HBM traffic."""

import csv
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from transformer_ffn_block_residual_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("wl", ["qwen7b8", "prefill", "prefill8"])
def test_block_traffic_specs(wl):
    w = W.WORKLOADS[wl]
    N, C, H = w.N, w.C, w.H
    e = 1 if w.fp8 else 2
    specs = {s[0]: s for s in bench.traffic_specs(wl)}
    first = bench.traffic_specs(wl)[0]
    assert first[0] == f"gateup_{wl}"                       # the dominant kernel comes first
    assert specs[f"gateup_{wl}"][4] == N * C * e + 2 * H * C * e + N * H * 2
    assert specs[f"down_{wl}"][4] == N * H * e + C * H * e + N * C * 2
    assert specs[f"rmsnorm_{wl}"][4] == 4 * N * C * 2 + 4 * N + 2 * C
    if w.fp8:
        # tiled operands by default: y and h alternate on the tiled quantiser
        assert specs[f"quant_y_{wl}"][4] == 3 * N * C and specs[f"quant_y_{wl}"][5] == (0, 2, 0)
        assert specs[f"quant_h_{wl}"][4] == 3 * N * H and specs[f"quant_h_{wl}"][5] == (0, 2, 1)
        assert specs[f"quant_y_{wl}"][2] == ["quant_tiled_kernel("]
        assert specs[f"gateup_{wl}"][2] == ["gemm_kernel<true, true, false, false, false, false, true>"]
        # row-major operands: keys of their own; after the two weight
        # quantisations, y and h alternate on the row-major quantiser
        rows = {s[0]: s for s in bench.traffic_specs(wl, rows_layout=True)}
        assert rows[f"quant_y_rows_{wl}"][5] == (2, 2, 0) and rows[f"quant_h_rows_{wl}"][5] == (2, 2, 1)
        assert rows[f"gateup_rows_{wl}"][2] == ["gemm_kernel<true, true, false, false, false, false, false>"]
        assert rows[f"gateup_rows_{wl}"][4] == specs[f"gateup_{wl}"][4]
    else:
        assert f"quant_y_{wl}" not in specs
        assert specs[f"gateup_{wl}"][2] == ["gemm_kernel<false, true, false, false, false, false, true>"]
        rows = {s[0]: s for s in bench.traffic_specs(wl, rows_layout=True)}
        assert rows[f"gateup_rows_{wl}"][2] == ["gemm_kernel<false, true, false, false, false, false, false>"]
        assert f"rmsnorm_rows_{wl}" in rows                    # the bf16 RMSNorm stores y tiled or not
    if w.decode_M:
        M = w.decode_M
        assert specs[f"decode{M}_{wl}"][4] == 3 * H * C + 4 * (2 * H + C) + 2 * M * (C + H) * 2
    src_files = {s[1] for s in specs.values()}
    assert src_files <= set(os.listdir(bench.CSRC))


def test_decode_and_backward_specs():
    w = W.WORKLOADS["decode"]
    (key, src, frags, _, algo, sel), = bench.traffic_specs("decode")
    assert key == "decode_decode" and src == "decode.hip" and len(frags) == 2
    assert algo == 3 * w.H * w.C + 4 * (2 * w.H + w.C) + 2 * (w.C + w.H) * 2
    q = W.WORKLOADS["qwen7b8"]
    (key, _, frags, _, algo, sel), = bench.traffic_specs("qwen7b8", backward=True)
    assert key == "dwup_qwen7b8" and sel == (0, 2, 1)        # the second weight-gradient GEMM of each step
    assert algo == 2 * q.H * q.N + q.C * q.N + 2 * (2 * q.H * q.C * 2)
    (key5, _, frags5, _, _, _), = bench.traffic_specs("qwen7b8", backward=True, grad_dtype="e5m2")
    assert key5 == "dwup5_qwen7b8" and frags5 != frags
    # the FP8 backward's products read tiled operands by default
    assert frags == ["gemm_kernel<true, false, false, true, false, false, true>"]
    (keyr, _, fragsr, _, _, _), = bench.traffic_specs("qwen7b8", backward=True, rows_layout=True)
    assert keyr == "dwup_rows_qwen7b8" and fragsr == ["gemm_kernel<true, false, false, true, false, false, false>"]


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, val) in enumerate(rows):
            wr.writerow([i + 1, name, counter, val])


def test_ingest_scales_by_the_copy_and_selects_dispatches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    gu = "void ffn::gemm_kernel<true, true, false, false, false, false, true>(ffn::GemmArgs)"
    dn = "void ffn::gemm_kernel<true, false, false, false, false, false, true>(ffn::GemmArgs)"
    rn = "void ffn::rmsnorm_kernel<8, true>(...)"
    qk = "ffn::quant_kernel(unsigned char*, float*, float const*, unsigned short const*, long, float*)"
    qt = "ffn::quant_tiled_kernel(unsigned char*, float*, float const*, unsigned short const*, long, long, float*)"
    dd = ["void ffn::decode_dual_wave_kernel<8, 8>(...)", "void ffn::decode_down_split_kernel<8>(...)",
          "ffn::decode_down_reduce_kernel(...)"]

    def rows(scale):
        r = [(qk, 1000.0 * scale), (qk, 2000.0 * scale)]                 # the two weight quantisations
        for step in range(3):
            r += [(rn, 10.0 * scale), (qt, 3.0 * scale), (gu, 100.0 * scale + step), (qt, 30.0 * scale),
                  (dn, 50.0 * scale)]
            r += [(d, (7.0 + k) * scale) for k, d in enumerate(dd)]
        r.append(("__amd_rocclr_copyBuffer", 524288.0 if scale == 1 else 1048576.0))
        return r

    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", rows(1))
    _counter_csv(write, "WRITE_SIZE", rows(2))
    a = types.SimpleNamespace(workload="qwen7b8", known_h_absmax=False, backward=False, grad_dtype="e4m3",
                              gemm_layout="tiled", ingest_pmc=(str(fetch), str(write)))
    assert bench.ingest_pmc(a) == 0
    data = json.load(open(tmp_path / "traffic.json"))
    # FETCH raw KiB scaled by 2 (the 1 GiB copy read as 512 MiB), WRITE by 1
    g = data["gateup_qwen7b8"]
    assert g["fetch_factor"] == 2.0 and g["write_factor"] == 1.0
    assert g["fetch_kb_raw"] == pytest.approx(101.0) and g["write_kb_raw"] == pytest.approx(201.0)
    assert g["bytes_per_launch"] == pytest.approx((101.0 * 2 + 201.0) * 1024)
    assert data["quant_y_qwen7b8"]["fetch_kb_raw"] == 3.0 and data["quant_h_qwen7b8"]["fetch_kb_raw"] == 30.0
    assert data["decode16_qwen7b8"]["fetch_kb_raw"] == 7.0 + 8.0 + 9.0    # the three kernels of one call
    assert data["rmsnorm_qwen7b8"]["src_sha256"] == bench.src_digest("norm_quant.hip")
    assert bench.measured_traffic("gateup_qwen7b8", "gemm.hip") == pytest.approx(g["bytes_per_launch"])
    # an entry taken from another version of the source is not reported
    data["gateup_qwen7b8"]["src_sha256"] = "0" * 64
    json.dump(data, open(tmp_path / "traffic.json", "w"))
    assert bench.measured_traffic("gateup_qwen7b8", "gemm.hip") is None


def test_ingest_needs_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    f = tmp_path / "f.csv"
    _counter_csv(f, "FETCH_SIZE", [("ffn::gemv_small_kernel<0, false, 1, 1, 2, 4, 2>(...)", 1.0)])
    a = types.SimpleNamespace(workload="decode", known_h_absmax=False, backward=False, grad_dtype="e4m3",
                              gemm_layout="tiled", ingest_pmc=(str(f), str(f)))
    with pytest.raises(SystemExit, match="calibration"):
        bench.ingest_pmc(a)


def test_committed_traffic_entries_match_their_sources():
    # bench.py reports a counter entry only while its kernel's source is the
    # one the counters were taken from; every committed entry is current
    data = json.load(open(bench.TRAFFIC_FILE))
    assert data
    for key, e in data.items():
        assert e["src_sha256"] == bench.src_digest(os.path.basename(e["src"])), key

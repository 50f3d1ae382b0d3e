"""bench.py on the GPU: short runs of several of its modes, each checked for
the one-line JSON record it must print (the keys, units and the roofline and
per-kernel entries), so that a mode that is rarely run cannot break unseen.
Each run is a subprocess with few steps and no CPU baseline."""

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[gpu] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "2",
                        "--no-cpu-baseline", *args], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _common(d, unit):
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "kernels"):
        assert k in d, k
    assert d["unit"] == unit and d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"] == "synthetic" and "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] in ("mfma", "hbm") and rf["peak"] > 0
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"])
    assert 0 < rf["frac"] < 1


@pytest.mark.timeout(600)
def test_decode_line():
    d = _run("--workload", "decode")
    _common(d, "GB/s")
    assert d["roofline"]["bound"] == "hbm" and d["dtype"] == "fp8"


@pytest.mark.timeout(600)
def test_decode_line_other_arms_and_tokens():
    for args in (("--decode-arm", "bf16"), ("--decode-m", "4"), ("--decode-m", "16", "--decode-layout", "rows")):
        d = _run("--workload", "decode", *args)
        _common(d, "GB/s")


@pytest.mark.timeout(600)
def test_prefill8_line_and_decode_position():
    d = _run("--workload", "prefill8")
    _common(d, "TFLOP/s")
    assert set(d["kernels"]) >= {"rmsnorm_fwd", "gateup_swiglu", "down", "quant_y", "quant_h"}
    d = _run("--workload", "qwen7b8", "--no-configs", "--decode-at", "start")
    _common(d, "TFLOP/s")
    assert d["config"]["decode_at"] == "start" and "decode" in d["kernels"]


@pytest.mark.timeout(600)
def test_backward_line():
    d = _run("--workload", "prefill8", "--backward")
    _common(d, "TFLOP/s")
    assert {"dw_up", "dx_up", "rmsnorm_bwd"} <= set(d["kernels"])

"""bench.py on the GPU: the fields of its JSON line, for the prefill workload (with
the CPU baseline) and for a decode workload's own line.  Short runs (2 timed steps)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    print(f"bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _common(d):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"] == "synthetic" and "workload" in d["config"]
    rf = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rf, key
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3


def test_prefill_line_with_cpu_baseline():
    d = _run("--steps", "2", "--warmup", "1", "--no-extra", "--no-decode", "--no-breakdown", "--cpu-budget", "2")
    _common(d)
    assert d["unit"] == "TFLOP/s" and d["config"]["workload"] == "prefill_32k_b2_bf16"
    assert d["roofline"]["bound"] == "mfma" and d["roofline"]["unit"] == "TFLOP/s"
    cb = d["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["gpu_rows_match"]["selection_equal"] is True


def test_decode_workload_line():
    d = _run("--workload", "7", "--steps", "2", "--warmup", "1", "--no-breakdown", "--no-cpu")
    _common(d)
    assert d["unit"] == "GB/s" and d["config"]["workload"] == "decode_paged_varlen_b64_bf16"
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["unit"] == "GB/s"
    assert d["cache_tokens"]["total"] > 0

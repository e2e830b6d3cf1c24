"""bench.py end to end on the GPU, a few steps of the default run: one JSON
line with the fields the measurement contract names, the largest graded
workload (the speculative-decode batch) as the headline, a roofline object
for its split kernel, the CPU-oracle baseline with the host's core count and
CPU model, and a sub-result with its own roofline for each other graded
workload and launch configuration."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _roofline_ok(roof):
    assert roof["bound"] in ("hbm", "mfma") and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["kernel_avg_ms"] > 0 and roof["path_frac"] > 0


def test_bench_json_line():
    print("bench.py default run, 3 steps", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--cpu-budget", "1"],
                       capture_output=True, text=True, timeout=400, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline", "sub_results"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == "spec_decode_bf16"
    _roofline_ok(d["roofline"])
    assert d["roofline"]["bound"] == "mfma"
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["nproc"] >= 1 and cpu["cpu_model"]
    subs = {(s["workload"], s["plan"].split(",")[0]) for s in d["sub_results"]}
    assert {w for w, _ in subs} == {"deepseek_v3_bf16", "agentic_long_bf16", "fp8_kv"}
    assert ("agentic_long_bf16", "uniform") in subs and ("agentic_long_bf16", "balanced work list") in subs
    for s in d["sub_results"]:
        _roofline_ok(s["roofline"])
        assert s["tokens_per_s"] > 0 and s["kv_gbs"] > 0

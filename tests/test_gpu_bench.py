"""bench.py on one GPU: the single JSON line it prints carries every field of the benchmark contract.

Runs the 4096-token single-request workload (small, a few seconds) in a child process, two timed steps.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_contract():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "3", "--steps", "2", "--warmup", "1",
                        "--cpu-seconds", "1"], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int), ("warmup", int),
                     ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                     ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)]:
        assert isinstance(d[key], typ), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"] and d["config"]["heads"] == 64 and d["config"]["kv_lora"] == 512
    roof = d["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof   # counters belong to the long-context workload: null here
    assert 0 < roof["frac_of_measured_mfma_loop"]
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["sample"]
    assert cpu["host_cpus"] >= 1 and cpu["blas_threads"] == cpu["cores"] and "cpu_model" in cpu
    ref = d["reference_rates"]
    assert ref["gemm_bf16_tflops"] > 0 and ref["copy_gbps"] > 0
    # the box's own ceilings: a back-to-back MFMA loop and a read-only stream, below the vendor peaks
    assert 0 < ref["mfma_loop_bf16_tflops"] <= 2600 and 0 < ref["stream_read_gbps"] <= 8500

"""GPU: bench.py's output contract.

A short run of the benchmark in a child process (the one-JSON-line contract:
field names, types and units, the roofline and CPU-baseline objects), and its
refusal of more than one GPU.  The timings themselves are not checked.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=240):
    print(f"[bench] {' '.join(args)}", flush=True)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_bench_prints_one_json_line_with_the_contract_fields():
    r = _bench("--steps", "3", "--warmup", "1", "--no-calibration")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "sampled points/s" and d["dtype"] == "f32"
    assert d["config"]["workload"] == "detr_encoder"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert roof["traffic"] is None or roof["traffic"] > 0
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0
    assert cpu["single_core"]["cores"] == 1
    single = d["kernel_us_single"]
    assert 0 < single["min"] <= single["median"] <= single["p90"] <= single["max"]
    # the encoder's visit order is built once, outside value, and said so
    assert d["config"]["query_order"] != "none" and d["query_order_build_us"] > 0
    assert d["value_includes_query_order_build"] is False
    assert 0 < d["value_with_query_order_build_every_step"] < d["value"]


def test_bench_refuses_more_than_one_gpu():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("op", ["backward", "forward_fused", "forward_pruned"])
def test_bench_other_ops_report_their_metric(op):
    r = _bench("--op", op, "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
               "--no-calibration")
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["config"]["op"] == op and d["value"] > 0
    assert d["roofline"]["frac"] > 0

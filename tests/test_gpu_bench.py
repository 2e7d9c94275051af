"""bench.py end to end on the GPU: a short run of the default workload and of the server round prints
one JSON line with the fields the bench contract names (metric, value, roofline, config, ...)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-3000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("args,workload,kernel,dense", [
    ((), "llama2-7B-bf16-ema", "compress", "refresh"),
    (("--workload", "bert-base-110M-fp32"), "bert-base-110M-fp32", "compress", "warmup"),
    (("--workload", "server-2^28-W8"), "server-2^28-W8", "server_apply", None),
])
def test_bench_prints_one_json_line(args, workload, kernel, dense):
    d = _bench(*args, "--steps", "3", "--warmup", "1", "--no-cpu")
    assert KEYS <= set(d)
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["config"]["workload"] == workload
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["kernel"] == kernel and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert d["cpu_baseline"] is None
    if dense is not None:
        # the timed steps are compressed steps; the schedule's dense steps are timed on their own
        assert d["timed_step_kinds"] == {"dense": 0, "compressed": 3}
        assert d["dense_step"]["kind"].startswith(dense) and d["dense_step"]["avg_ms"] > 0

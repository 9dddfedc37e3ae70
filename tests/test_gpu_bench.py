"""bench.py end to end on the GPU, on the small workload: one JSON line with
the fields the measurement contract names (metric, value, roofline with its
traffic slot, the CPU oracle baseline), in eager and HIP-graph launch."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [l for l in p.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, p.stdout[-2000:]
    return json.loads(lines[0])


@pytest.mark.parametrize("graph", [False, True])
def test_bench_line_contract(graph):
    args = ["--workload", "tiny_T32_d512_f256_E16", "--steps", "3", "--warmup", "1",
            "--cpu-seconds", "1"]
    rec = _bench(*args, *(["--graph"] if graph else []))
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0 and rec["unit"] == "tokens/s"
    assert rec["config"]["workload"] == "tiny_T32_d512_f256_E16"
    assert rec["config"]["launch"] == ("hip graph replay" if graph else "eager")
    # tokens per second and the step time describe the same run
    assert abs(rec["value"] - 32 / (rec["ms_per_step"] / 1e3)) <= 1e-3 * rec["value"] + 1.0
    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] in ("hbm", "mfma") and roof["frac"] > 0
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-2, abs=1e-4)
    cpu = rec["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert rec["route_table_sha256"] and len(rec["route_table_sha256"]) == 64

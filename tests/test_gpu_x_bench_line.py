"""bench.py end to end on the GPU: one short run of the OPT-13B-class batch (a few steps, a short
CPU-baseline budget, the cache-evicting reps) must print exactly one JSON line with every field of
the bench contract, finite and consistent."""
import json
import math
import subprocess
import sys
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parent.parent


def test_bench_line_has_the_contract_fields():
    cmd = [sys.executable, "-u", str(ROOT / "bench.py"), "--config", "2", "--steps", "3", "--warmup", "1",
           "--reps", "3", "--flush", "--cpu-budget-s", "1"]
    print("bench contract run:", " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=str(ROOT))
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] == "opt13b_mha"
    assert math.isfinite(d["value"]) and d["value"] > 0 and d["ms_per_step"] > 0
    # value = algorithmic bytes per step / step time: it and ms_per_step describe the same steps
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and roof["unit"] == "GB/s"
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-3)
    assert 0 < roof["frac"] < 1.0
    # every step reads at least what its decode kernel reads: the step cannot be faster than the kernel
    assert d["value"] <= roof["achieved"] * 1.001
    cpu = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cpu, k
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    p = d["decode_launch_us"]
    assert p["launches"] == 3 and p["min"] <= p["p10"] <= p["median"] <= p["p90"] <= p["max"]
    cold = d["decode_launch_us_cold"]
    assert cold["after_write"]["launches"] == 3 and cold["after_read"]["launches"] == 3
    assert d["env"]["arch"].startswith("gfx950")
    # the streaming-read probe's best rate, beside the data sheet's 8 TB/s
    assert 0 < d["measured_read_gbps"] < 8000.0
    assert d["read_ceiling"]["best"]["gbps"] == d["measured_read_gbps"]


def test_bench_counts_a_shared_prompt_once():
    """The swarm (20 rows sharing a 4000-token prompt): value, pct_hbm_peak and the roofline count each
    shared block once, and the logical rate, over every row's own reading, is reported beside it."""
    cmd = [sys.executable, "-u", str(ROOT / "bench.py"), "--config", "4", "--steps", "3", "--warmup", "1",
           "--reps", "2", "--no-cpu-baseline", "--no-read-ceiling"]
    print("bench swarm run:", " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=str(ROOT))
    assert r.returncode == 0, r.stderr[-3000:]
    d = json.loads([ln for ln in r.stdout.splitlines() if ln.strip()][0])
    roof = d["roofline"]
    # 19 of the 20 rows re-read the prompt's 4000 tokens: logical bytes exceed unique ones by that much
    per_token = 2 * 8 * 128 * 2
    assert roof["bytes_per_launch_logical"] - roof["bytes_per_launch"] == 19 * 4000 * per_token
    assert d["value_logical"] > d["value"]
    assert d["pct_hbm_peak"] == pytest.approx(100 * d["value"] / 8000.0, abs=0.01)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-3)

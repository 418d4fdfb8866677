"""Host-side helpers of bench.py: per-launch percentiles, the engine-clock parser and the --gpus
contract (CPU only)."""
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402


def test_percentiles_us_converts_ms_and_orders():
    p = bench.percentiles_us([0.4, 0.1, 0.3, 0.2])
    assert p["launches"] == 4
    assert p["min"] == 100.0 and p["max"] == 400.0
    assert p["median"] == 250.0
    assert p["p10"] <= p["median"] <= p["p90"]
    # numpy's linear interpolation: 10 % of the way from 100 to 200 after the first of 3 gaps
    assert p["p10"] == pytest.approx(130.0)
    assert p["p90"] == pytest.approx(370.0)


def test_parse_dpm_sclk_reads_active_and_max_levels():
    txt = "0: 500Mhz\n1: 1600Mhz *\n2: 2400Mhz\n"
    r = bench.parse_dpm_sclk(txt)
    assert r["current"] == 1600 and r["max"] == 2400
    # some kernels print a deep-sleep level first and no active marker
    r = bench.parse_dpm_sclk("S: 100Mhz\n0: 500Mhz\n1: 2400Mhz\n")
    assert r["current"] is None and r["max"] == 2400
    assert bench.parse_dpm_sclk("") is None
    assert bench.parse_dpm_sclk(None) is None
    assert bench.parse_dpm_sclk("no clocks here\n") is None


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""

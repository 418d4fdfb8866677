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


def test_duplicate_tokens_counts_shared_blocks_once():
    # a tiny swarm through the oracle's allocator: a 40-token prompt (blocks of 16: two full, one with 8),
    # three children sharing its first 32 tokens, each with a private suffix; the third child shares
    # only the first block
    from oracle.allocator import BlockAllocatorModel
    B = 16
    a = BlockAllocatorModel(64, B)
    a.alloc(9, 40)
    for c in (0, 1):
        a.fork(9, c, 32)
    a.fork(9, 2, 16)
    a.alloc(0, 5)
    a.alloc(1, 20)
    a.alloc(2, 1)
    rows = [9, 0, 1, 2]
    lens = [40, 37, 52, 17]
    tables = [a.block_table(r) for r in rows]
    # logical tokens 146; unique: the parent's 40, child 0's own 5, child 1's own 20, child 2's own 1
    assert bench.duplicate_tokens(tables, lens, B) == 146 - (40 + 5 + 20 + 1)
    # no sharing: nothing is counted twice
    assert bench.duplicate_tokens([[0, 1], [2]], [20, 9], B) == 0
    # a shared partial block counts its longest reader's valid tokens once
    assert bench.duplicate_tokens([[0, 1], [0, 1]], [24, 20], B) == 16 + 4


def test_host_replay_counts_the_swarm_prompt_once_per_extra_row():
    """The counter summaries price traffic against unique bytes: replaying the swarm's allocator
    operations on the host finds 19 extra readings of the 4000-token prompt (250 whole blocks) and
    none when every row holds its own copy."""
    import workloads as wl
    assert bench.host_duplicate_tokens(wl.build(4)) == 19 * 4000
    assert bench.host_duplicate_tokens(wl.build(4, copied_prefix=True)) == 0
    assert bench.host_duplicate_tokens(wl.build(4, block_size=32)) == 19 * 4000
    assert bench.host_duplicate_tokens(wl.build(3)) == 0


def test_roofline_reports_aux_bytes_and_flops_beside_the_algorithmic_bytes():
    """q, the output and the lengths are reported beside the algorithmic bytes, not counted in them; the
    attention's flops are the sum over rows of L * Hq * 4 * D."""
    import workloads as wl
    w = wl.build(3)
    tokens = 1_000_000
    kv = tokens * 2 * w.n_kv_heads * w.head_dim * 2
    res = {"decode_timed": (10, 10 * 0.75), "kv_bytes_unique": kv * 10, "kv_bytes": kv * 10,
           "table_bytes": 250_000 * 10, "steps": 10}
    r = bench.roofline(res, w)
    assert r["bytes_per_launch"] == kv + 250_000
    assert r["aux_bytes_per_launch"] == 256 * (2 * 64 * 128 * 2 + 4)
    assert r["flop_per_launch"] == tokens * 64 * 4 * 128
    assert r["frac"] == pytest.approx((kv + 250_000) / 750e-6 / 1e9 / 8000.0, abs=1e-4)
    assert "fp32 KV" in bench.kernel_label(wl.build(1)) and "MFMA" in bench.kernel_label(w)

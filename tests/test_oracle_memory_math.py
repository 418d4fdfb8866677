"""Pins of the oracle's memory arithmetic (O1) to the numbers the pages print.

Fixture: tests/golden/memory_math.json (each entry carries its page and section).
"""
import json
import math
import os

import pytest

from oracle import memory_math as mm

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "memory_math.json")))
KiB, MiB, GiB = 1024, 1024 ** 2, 1024 ** 3


@pytest.mark.parametrize("case", GOLDEN["kv_bytes_per_token"], ids=lambda c: f"{c['kib']}KiB")
def test_kv_bytes_per_token(case):
    b = mm.kv_bytes_per_token(case["n_layers"], case["n_kv_heads"], case["head_dim"], case["dtype_bytes"])
    assert b == case["bytes"]
    assert b == case["kib"] * KiB


def test_sequence_bytes():
    opt, l70, long70 = GOLDEN["sequence_bytes"]
    assert opt["tokens"] * opt["per_token_kib"] * KiB == opt["mib"] * MiB
    # "about 1.6 GB": 1600 MiB is 1.68 decimal GB and 1.5625 GiB; both round to 1.6
    assert round(opt["mib"] * MiB / 1e9, 1) in (1.6, 1.7) and round(opt["mib"] / 1024, 1) == 1.6
    assert l70["tokens"] * l70["per_token_kib"] * KiB == l70["mib"] * MiB
    per_tok = mm.kv_bytes_per_token(80, 8, 128, 2)
    total = long70["tokens"] * per_tok
    assert total == long70["gib"] * GiB
    assert total > long70["at_least_gb"] * 1e9


@pytest.mark.parametrize("case", GOLDEN["utilisation_contiguous"], ids=lambda c: str(c["L"]))
def test_utilisation_contiguous(case):
    u = mm.utilisation_contiguous(case["L"], case["L_max"])
    assert u == case["U"]
    assert round(100 * (1 - u)) == case["wasted_pct"]


def test_idle_slots():
    (case,) = GOLDEN["idle_slots"]
    idle = mm.idle_slots_contiguous(case["L"], case["L_max"])
    assert idle == case["idle"]
    assert round(100 * idle / case["L_max"]) == case["pct_rounded"]


def test_paged_waste_bounds():
    (case,) = GOLDEN["paged_waste"]
    B = case["B"]
    worst = max(mm.waste_paged(L, B) for L in range(1, 10 * B))
    assert worst == case["worst"] == B - 1
    assert mm.mean_waste_paged(B) == case["mean"]
    # the average over a full period of lengths is exactly (B-1)/2
    assert sum(mm.waste_paged(L, B) for L in range(1, B + 1)) / B == case["mean"]
    assert 100 * case["worst"] / case["L_for_pct"] < case["pct_below"]


def test_utilisation_paged_closed_form():
    for B in (1, 8, 16, 32):
        for L in range(1, 300):
            u = mm.utilisation_paged(L, B)
            assert u == L / (math.ceil(L / B) * B)
            assert 0 < u <= 1
            assert mm.waste_paged(L, B) <= B - 1
            assert (u == 1.0) == (L % B == 0)
    assert mm.blocks_needed(0, 16) == 0
    with pytest.raises(ValueError):
        mm.blocks_needed(-1, 16)


def test_worked_example_binary_units():
    w = GOLDEN["worked_example"]
    per_tok = w["per_token_kib"] * KiB
    contig = w["L_max"] * per_tok
    assert contig == w["contiguous_mib"] * MiB
    assert mm.blocks_needed(w["L"], w["B"]) == w["paged_blocks"]
    assert mm.slots_paged(w["L"], w["B"]) == w["paged_slots"]
    paged = mm.slots_paged(w["L"], w["B"]) * per_tok
    assert paged == w["paged_mib"] * MiB
    budget = w["free_gib"] * GiB
    n_c = mm.requests_that_fit(budget, contig)
    n_p = mm.requests_that_fit(budget, paged)
    assert (n_c, n_p) == (w["contiguous_requests"], w["paged_requests"])
    assert round(n_p / n_c) == w["ratio_about"]
    # decimal units would give 70 paged requests: the page's 71 needs binary KB/MB/GB
    assert mm.requests_that_fit(w["free_gib"] * 1e9, w["paged_mib"] * 1e6 / 1.0) == 70


def test_rx9070xt_budget():
    r = GOLDEN["rx9070xt"]
    mb = r["mb_per_token"]
    slot16 = r["reserve_16k"]["tokens"] * mb / 1000           # GB (decimal)
    assert slot16 == pytest.approx(r["reserve_16k"]["slot_gb"])
    assert round(r["agents"] * slot16, 1) == r["reserve_16k"]["total_gb"]
    assert mm.requests_that_fit(r["kv_budget_gb"], slot16) == r["reserve_16k"]["admitted"]
    slot8 = r["reserve_8k"]["tokens"] * mb / 1000
    assert slot8 == pytest.approx(r["reserve_8k"]["slot_gb"])
    reserved8 = r["agents"] * slot8
    assert round(reserved8, 1) == r["reserve_8k"]["total_gb"]
    live = r["agents"] * r["snapshot"]["avg_tokens"] * mb / 1000
    assert round(live, 1) == r["snapshot"]["live_gb"]
    waste_pct = 100 * mm.wasted_fraction(reserved8, live)
    assert waste_pct == pytest.approx(62.5)  # printed as 63 %, i.e. rounded half up
    assert math.floor(waste_pct + 0.5 + 1e-9) == r["snapshot"]["waste_pct_8k"]
    # paged: each agent commits ceil(3000/16) blocks, wasting under 1 %
    u = mm.utilisation_paged(r["snapshot"]["avg_tokens"], r["paged"]["B"])
    assert 100 * (1 - u) < r["paged"]["waste_pct_below"]
    assert round(r["kv_budget_gb"] - live, 1) == r["paged"]["free_gb_about"]
    cap = r["kv_budget_gb"] * 1000 / mb
    assert round(cap, -3) == r["paged"]["capacity_tokens_about"]

"""Results that wait in LDS: a wave keeps each finished unit's results (a partition's max, sum and
accumulator, or a one-partition row's output) in LDS and writes them after its last unit; a unit that
finds the entries full stores its results at once (GPU, through the C ABI, against the oracle).

32-token partitions over rows of several hundred tokens give every wave about nine units, more than its
entries (7 at one wave per SIMD, 2 at two), so both the parked and the direct stores run in one launch,
and rows of fewer than 32 tokens have one partition (a parked output).  Every row is compared with the
oracle, at head sizes 128 and 64 (whose entries are half as large).  The streamed and the cacheable loads
run kernels with different numbers of entries, so a unit parked under one is stored at once under the
other: the two outputs must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from harness import TOL, GpuState, log, max_abs_err_rows, oracle_all

pytestmark = pytest.mark.gpu


def _lens(seed):
    rng = np.random.default_rng(seed)
    long_rows = rng.integers(700, 900, size=48).tolist()
    short_rows = rng.integers(1, 32, size=8).tolist()
    return long_rows[:24] + short_rows + long_rows[24:]


@pytest.mark.parametrize("kv,dtype,G,D", [("native", "bf16", 8, 128), ("native", "f16", 1, 128),
                                          ("fp8", "bf16", 8, 128), ("native", "f16", 4, 64)])
def test_more_finished_units_than_lds_entries(kv, dtype, G, D):
    Hk = 8
    w = wl.custom(seed=91, lens=_lens(3), n_q_heads=G * Hk, n_kv_heads=Hk, head_dim=D, block_size=16,
                  dtype=dtype, partition_size=32)
    if kv == "fp8":
        w = wl.quantised(w, k_scale=0.01, v_scale=0.0125)
    units = int(np.ceil(np.asarray(w.seq_lens) / 32).sum()) * Hk
    assert units > 8 * 1024, units   # more units than a full grid of waves has LDS entries
    st = GpuState(w, poison=True)
    streamed = st.decode()
    cached = st.decode(shared_kv=True)
    err, row = max_abs_err_rows(streamed, oracle_all(w))
    log(f"parked results {kv} {dtype} G={G} D={D}: {units} units, all rows max abs err {err:.3e} (row {row})")
    assert err <= TOL[dtype], (err, row)
    assert torch.equal(streamed.view(torch.int16), cached.view(torch.int16))

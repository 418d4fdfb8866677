"""The online softmax's rescale under running maxima that rise on every tile, never after the first, or
differently for the query heads of one KV head (GPU, through the C ABI, against the oracle).

Each row's keys are a_t * u (plus small noise) with a_t growing along the row for one KV head and
shrinking for the other, and its query heads point along +u or -u in turn.  So within one KV head some
heads' scores rise with every tile (each tile raises their running max and rescales the accumulators)
while others peak at the first token (their max never rises again), and the two kinds sit in the lanes
of one wave.  Scores reach about 13 in natural-log units, so a rescale applied to the wrong lanes or
skipped when needed moves the result far beyond the tolerance.  Partitions of 256 tokens add the
merge of several running maxima per row.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_53_amd as pkv
import workloads as wl
from harness import TOL, GpuState, log
from oracle import attention as O
from oracle import fp8 as F

pytestmark = pytest.mark.gpu


def _monotone_rows(w, rng):
    """Logical K, V [L, Hk, D] (float32) per row and q [S, Hq, D] (float32)."""
    Hk, D, G = w.n_kv_heads, w.head_dim, w.n_q_heads // w.n_kv_heads
    u = rng.standard_normal((Hk, D)).astype(np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    rows = []
    for L in w.seq_lens.tolist():
        ramp = 150.0 * np.arange(L, dtype=np.float32) / max(L - 1, 1)
        a = np.stack([ramp if kv % 2 == 0 else 150.0 - ramp for kv in range(Hk)], axis=1)   # [L, Hk]
        K = a[:, :, None] * u[None] + 0.05 * rng.standard_normal((L, Hk, D)).astype(np.float32)
        V = rng.standard_normal((L, Hk, D)).astype(np.float32)
        rows.append((K, V))
    sign = np.array([1.0 if h % 2 == 0 else -1.0 for h in range(w.n_q_heads)], dtype=np.float32)
    q = sign[None, :, None] * u[np.arange(w.n_q_heads) // G][None] \
        + 0.05 * rng.standard_normal((w.num_seqs, w.n_q_heads, D)).astype(np.float32)
    return rows, q


@pytest.mark.parametrize("kv,dtype,G", [("native", "bf16", 8), ("native", "f16", 1), ("fp8", "bf16", 8)])
def test_rising_and_falling_maxima(kv, dtype, G):
    Hk = 2
    w = wl.custom(seed=77, lens=[700, 333, 1500, 17], n_q_heads=G * Hk, n_kv_heads=Hk, head_dim=128,
                  block_size=16, dtype=dtype, partition_size=256)
    if kv == "fp8":
        w = wl.quantised(w, k_scale=0.5, v_scale=0.0125)
    st = GpuState(w, poison=True)
    rng = np.random.default_rng(5)
    rows, q32 = _monotone_rows(w, rng)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    B = w.block_size
    for r, (K, V) in enumerate(rows):
        L = K.shape[0]
        t = np.arange(L)
        slots = st.tables_host[r, t // B].astype(np.int64) * B + t % B
        pkv.reshape_and_cache(torch.from_numpy(K).to(tdt).cuda(), torch.from_numpy(V).to(tdt).cuda(),
                              torch.from_numpy(slots).cuda(), st.k_pool, st.v_pool, **st.scales)
    q = torch.from_numpy(q32).to(tdt).cuda()
    out = st.decode(out_dtype=torch.float32, q=q)
    # the oracle: the stored values (rounded to the cache's type, or its FP8 codes) in fp64
    q64 = q.float().cpu().numpy().astype(np.float64)
    err = 0.0
    for r, (K, V) in enumerate(rows):
        K16 = torch.from_numpy(K).to(tdt).float().numpy()
        V16 = torch.from_numpy(V).to(tdt).float().numpy()
        if kv == "fp8":
            K64 = F.dequantize(F.quantize(K16, w.k_scale), w.k_scale)
            V64 = F.dequantize(F.quantize(V16, w.v_scale), w.v_scale)
        else:
            K64, V64 = K16.astype(np.float64), V16.astype(np.float64)
        ref = O.attention_logical(q64[r], K64, V64, w.scale)
        err = max(err, float(np.abs(out[r].cpu().numpy() - ref).max()))
    log(f"monotone maxima {kv} {dtype} G={G}: max abs err {err:.3e}")
    assert err <= TOL[dtype], err

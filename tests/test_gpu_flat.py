"""GPU parity of flat spans (pkv_span_pool + pkv_paged_attention_decode_flat).

Flat-span decode computes block ids from each row's span instead of reading a block table; the tiles,
the arithmetic and its order are those of the paged kernel, so over the same tokens its output must be
bit-identical to paged decode (random block placement) and within the 16-bit tolerance of the fp64
oracle.  Span memory is read back and compared with the oracle's scatter at the flat slots, bit for bit.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_53_amd as pkv
import workloads as wl
from harness import TOL, FlatState, GpuState, device_view, log, max_abs_err, oracle_rows

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


@pytest.mark.parametrize("cid,B", [(3, 16), (5, 8), (5, 16), (5, 32), (2, 16)])
def test_flat_decode_is_bit_identical_to_paged(cid, B):
    w = wl.build(cid, small=True, block_size=B)
    log(f"flat vs paged config {cid} small B={B}: {w.describe()}")
    paged = GpuState(w).decode(out_dtype=torch.float32)
    fs = FlatState(w)
    flat = fs.decode(out_dtype=torch.float32)
    assert torch.equal(_bits(flat), _bits(paged))
    ref = oracle_rows(w, range(w.num_seqs))
    err = max_abs_err(flat, ref, rows=range(w.num_seqs))
    log(f"  bit-identical; err vs oracle {err:.3e}")
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("dtype,G,D", [("bf16", 8, 128), ("f16", 1, 64), ("f16", 16, 128), ("bf16", 3, 64)])
def test_flat_heads_dims_sweep(dtype, G, D):
    Hk = 2
    lens = [1, 15, 16, 17, 33, 100, 511, 513, 1000]
    w = wl.custom(seed=500 + G + D, lens=lens, n_q_heads=G * Hk, n_kv_heads=Hk, head_dim=D, block_size=16,
                  dtype=dtype, partition_size=128)
    flat = FlatState(w).decode(out_dtype=torch.float32)
    paged = GpuState(w).decode(out_dtype=torch.float32)
    assert torch.equal(_bits(flat), _bits(paged))
    ref = oracle_rows(w, range(w.num_seqs))
    assert max_abs_err(flat, ref, rows=range(w.num_seqs)) <= TOL[dtype]


@pytest.mark.parametrize("chunk", [4096, 65536, 2 << 20])
def test_span_memory_matches_the_oracle_scatter(chunk):
    from oracle import scatter as SC
    w = wl.custom(seed=77, lens=[5, 40, 300, 129], n_q_heads=8, n_kv_heads=2, head_dim=64, block_size=16,
                  dtype="bf16")
    fs = FlatState(w, chunk_bytes=chunk)
    pool = fs.cache.pool
    info = pool.info()
    block_bytes = w.n_kv_heads * w.head_dim * w.block_size * 2
    # mapped memory: each span rounded up to whole chunks, in both pools
    want = sum(-(-(-(-int(L) // 16) * block_bytes) // chunk) * chunk for L in w.seq_lens) * 2
    assert info["mapped_bytes"] == want, (info, want)
    N, bps = pool.num_blocks, pool.blocks_per_span
    kv = device_view(pool.k_base, (N, w.n_kv_heads, w.head_dim // 8, 16, 8), torch.int16)
    vv = device_view(pool.v_base, (N, w.n_kv_heads, w.head_dim, 16), torch.int16)
    for r in range(w.num_seqs):
        L = int(w.seq_lens[r])
        table = SC.flat_span_table(fs.cache.span(r), bps, L, 16)
        ids = torch.tensor(table, dtype=torch.long, device="cuda")          # mapped blocks only
        kp = kv[ids].cpu().numpy().view(np.uint16)
        vp = vv[ids].cpu().numpy().view(np.uint16)
        K, V = SC.gather_logical(kp, vp, list(range(len(table))), L)
        Kw, Vw = wl.logical_kv(w, r)
        assert np.array_equal(K, wl.storage_to_numpy(Kw)) and np.array_equal(V, wl.storage_to_numpy(Vw))
    log(f"chunk {chunk}: span memory bit-exact, mapped {info['mapped_bytes']} B")


def test_span_release_reuse_and_trim():
    w = wl.custom(seed=78, lens=[300, 90], n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16, dtype="f16")
    fs = FlatState(w, chunk_bytes=65536)
    c = fs.cache
    before = c.pool.info()["mapped_bytes"]
    c.free(0)                                    # span 0 unmapped, its chunks kept
    inf = c.pool.info()
    assert inf["mapped_bytes"] < before and inf["spare_bytes"] == before - inf["mapped_bytes"]
    # a new sequence takes the released span, with other data, on reused chunks
    w2 = wl.custom(seed=79, lens=[250], n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16, dtype="f16")
    K, V = wl.logical_kv(w2, 0, device="cuda")
    c.append(10, K, V)
    assert c.span(10) == 1 or c.span(10) == 0
    span = c.span(10)
    out = torch.full((1, 8, 128), float("nan"), dtype=torch.float32, device="cuda")
    q = wl.q_values(w2, device="cuda").contiguous()
    pkv.paged_attention_decode_flat(out, q, c.pool, torch.tensor([span], dtype=torch.int32, device="cuda"),
                                    torch.tensor([250], dtype=torch.int32, device="cuda"), w2.scale, 250, 512)
    torch.cuda.synchronize()
    ref = oracle_rows(w2, [0])
    assert max_abs_err(out, ref, rows=[0]) <= TOL["f16"]
    with pytest.raises(pkv.PKVError):
        c.pool.reserve(span, 10 ** 6)            # beyond the span: rejected, nothing mapped
    c.pool.trim()
    assert c.pool.info()["spare_bytes"] == 0


def test_flat_decode_batch_steps_match_the_oracle():
    """FlatDecodeBatch: every step backs the new token (crossing chunk boundaries), scatters it and
    decodes; each step's output against the oracle on the growing histories."""
    from oracle import attention as O
    from paged_kv_cache_53_amd.runtime import FlatDecodeBatch, FlatKVCache
    rng = np.random.default_rng(3)
    Hk, G, D, B = 2, 4, 64, 16
    cache = FlatKVCache(3, 200, B, Hk, D, torch.bfloat16, chunk_bytes=4096)   # 4 KiB = one block per chunk
    hist = {}
    for s, L in enumerate((16, 31, 1)):
        k = torch.randn(L, Hk, D).to(torch.bfloat16)
        v = torch.randn(L, Hk, D).to(torch.bfloat16)
        cache.append(s, k.cuda(), v.cuda())
        hist[s] = (k, v)
    batch = FlatDecodeBatch(cache, [0, 1, 2], Hk * G, 200, partition_size=32)
    for step in range(20):
        q = torch.randn(3, Hk * G, D).to(torch.bfloat16)
        kn = torch.randn(3, Hk, D).to(torch.bfloat16)
        vn = torch.randn(3, Hk, D).to(torch.bfloat16)
        out = torch.empty(3, Hk * G, D, dtype=torch.float32, device="cuda")
        batch.step(q.cuda(), kn.cuda(), vn.cuda(), out)
        torch.cuda.synchronize()
        for i in range(3):
            hk, hv = hist[i]
            hist[i] = (torch.cat([hk, kn[i:i + 1]]), torch.cat([hv, vn[i:i + 1]]))
            ref = O.attention_logical(q[i].double().numpy(), hist[i][0].double().numpy(),
                                      hist[i][1].double().numpy(), batch.scale)
            err = float(np.max(np.abs(out[i].double().cpu().numpy() - ref)))
            assert err <= TOL["bf16"], (step, i, err)
    assert batch.seq_lens.cpu().tolist() == [36, 51, 21]


def test_flat_full_size_long_context():
    w = wl.build(5)
    log(f"flat full long_context: {w.describe()}")
    fs = FlatState(w)
    out = fs.decode()
    assert torch.isfinite(out).all()
    rows = [0, 5]
    ref = oracle_rows(w, rows)
    err = max_abs_err(out, ref, rows=rows)
    log(f"  rows {rows}: err {err:.3e}")
    assert err <= TOL["bf16"]

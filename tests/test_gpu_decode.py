"""GPU parity of paged decode attention against the fp64 oracle.

Bar: max |gpu - oracle| <= 1e-5 for fp32 KV and <= 2e-2 for fp16/bf16 KV (fp32 accumulation),
element by element over every output of the small configs (several tiles, partitions and a
ragged tail each) and over every row (all heads) at the full sizes, in the launch configuration
bench.py times (each workload's own partition size: 512 tokens for the OPT-13B-class batch, 3072
for the Llama-70B-class one, 768 for the shared-prefix swarm and 2048 for the long contexts) and,
for the long contexts, also in the 512-token partitions the workload states (128 per row).
Invariances (placement, shared vs copied prompt, load policy) are bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import paged_kv_cache_53_amd as pkv
import workloads as wl
from harness import (TOL, TORCH_DTYPE, GpuState, log, max_abs_err, max_abs_err_rows, oracle_all,
                     oracle_paged, oracle_rows)

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


# ------------------------------------------------------------------------- small configs, all rows
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_small_configs_full_oracle_pipeline(cid):
    w = wl.build(cid, small=True) if cid != 1 else wl.build(1)
    log(f"config {cid} small: {w.describe()}")
    st = GpuState(w)
    ref, model, tables = oracle_paged(w)
    for r in range(w.num_seqs):
        nb = tables.shape[1]
        t = model.block_table(int(w.batch[r]))
        assert st.tables_host[r, :len(t)].tolist() == t
    for odt in (TORCH_DTYPE[w.dtype], torch.float32):
        out = st.decode(out_dtype=odt)
        err = max_abs_err(out, ref)
        log(f"  out {odt}: max abs err {err:.3e}")
        assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("B", [8, 16, 32])
def test_long_context_block_sizes_and_placement(B):
    outs = {}
    for placement in ("random", "identity"):
        w = wl.build(5, small=True, block_size=B, placement=placement)
        st = GpuState(w)
        outs[placement] = st.decode(out_dtype=torch.float32)
    ref = oracle_rows(w, range(w.num_seqs))
    err = max_abs_err(outs["random"], ref, rows=range(w.num_seqs))
    log(f"config 5 small B={B}: err {err:.3e}")
    assert err <= TOL[w.dtype]
    # the summation order depends only on logical positions: placement changes no bit
    assert torch.equal(_bits(outs["random"]), _bits(outs["identity"]))


def test_shared_prefix_equals_copied_prefix_bitwise():
    shared, copied = wl.build(4, small=True), wl.build(4, small=True, copied_prefix=True)
    a, b = GpuState(shared), GpuState(copied)
    assert a.alloc.stats()["shared_blocks"] == 400 // 16
    oa, ob = a.decode(), b.decode()
    assert torch.equal(_bits(oa), _bits(ob))
    # the load policy (every tile cacheable, or only the shared prompt's, at various prefix lengths)
    # changes no bit of the result
    assert torch.equal(_bits(a.decode(shared_kv=True)), _bits(oa))
    for n in (400, 16, 417, 100000):
        assert torch.equal(_bits(a.decode(shared_prefix_tokens=n)), _bits(oa)), n
    ref = oracle_rows(copied, range(copied.num_seqs))
    assert max_abs_err(oa, ref, rows=range(copied.num_seqs)) <= TOL["f16"]


@pytest.mark.parametrize("P", [32, 64, 96, 512, 0])
def test_partition_sizes(P):
    w = wl.build(3, small=True)
    st = GpuState(w)
    ref = oracle_rows(w, range(w.num_seqs))
    out = st.decode(out_dtype=torch.float32, partition_size=P)
    err = max_abs_err(out, ref, rows=range(w.num_seqs))
    log(f"partition {P}: err {err:.3e}")
    assert err <= TOL["bf16"]


def test_split_and_unsplit_agree_and_calls_are_deterministic():
    w = wl.build(3, small=True)
    st = GpuState(w)
    a = st.decode(out_dtype=torch.float32, partition_size=64)
    b = st.decode(out_dtype=torch.float32, partition_size=0)
    assert float((a - b).abs().max()) <= TOL["bf16"]
    c = st.decode(out_dtype=torch.float32, partition_size=64)
    assert torch.equal(_bits(a), _bits(c))


# ------------------------------------------------------------------------- shapes and paths
SWEEP = []
for dtype in ("f16", "bf16"):
    for G in (1, 2, 3, 4, 5, 8, 16):
        for D in (64, 128):
            SWEEP.append((dtype, G, D, 16 if G % 2 else 8 if D == 64 else 32))
for G in (1, 2, 3, 4):
    SWEEP.append(("f32", G, 64 if G % 2 else 128, 16 if G < 3 else 8))


@pytest.mark.parametrize("dtype,G,D,B", SWEEP)
def test_heads_dims_blocks_sweep(dtype, G, D, B):
    Hk = 2
    lens = [1, 15, 16, 17, 31, 32, 33, 100, 511, 512, 513, 1000]
    w = wl.custom(seed=100 + G * 7 + D, lens=lens, n_q_heads=G * Hk, n_kv_heads=Hk, head_dim=D,
                  block_size=B, dtype=dtype, partition_size=128)
    st = GpuState(w)
    ref = oracle_rows(w, range(w.num_seqs))
    out = st.decode(out_dtype=torch.float32)
    err = max_abs_err(out, ref, rows=range(w.num_seqs))
    log(f"{dtype} G={G} D={D} B={B}: err {err:.3e}")
    assert err <= TOL[dtype], err
    # length 1: softmax weight exactly 1, output exactly the single value row
    K, V = wl.logical_kv(w, 0)
    v0 = V[0].float()                                    # [Hk, D]
    exp = v0.repeat_interleave(G, dim=0)
    assert torch.equal(out[0].cpu(), exp)


@pytest.mark.parametrize("dtype,D,B", [("f16", 128, 16), ("bf16", 128, 8), ("f16", 64, 32), ("bf16", 64, 16)])
def test_vector_path_for_one_head_per_kv_head(dtype, D, B):
    """16-bit KV with G = 1 on the per-token vector path (fp32 dot products, cross-lane reductions)
    instead of MFMA with the head padded to 16: within the tolerance of the oracle, streamed and
    cacheable, and only for G = 1."""
    lens = [1, 15, 16, 17, 33, 100, 511, 513, 1000]
    w = wl.custom(seed=300 + D + B, lens=lens, n_q_heads=4, n_kv_heads=4, head_dim=D, block_size=B, dtype=dtype,
                  partition_size=128)
    st = GpuState(w)
    ref = oracle_all(w)
    for shared in (False, True):
        out = st.decode(out_dtype=torch.float32, vector=True, shared_kv=shared)
        err, row = max_abs_err_rows(out, ref)
        log(f"vector path {dtype} D={D} B={B} shared={shared}: max abs err {err:.3e} (row {row})")
        assert err <= TOL[dtype], err
    K, V = wl.logical_kv(w, 0)                       # length 1: exactly the value row
    assert torch.equal(out[0].cpu(), V[0].float())
    w8 = wl.custom(seed=5, lens=[40], n_q_heads=8, n_kv_heads=4, head_dim=D, block_size=B, dtype=dtype)
    st8 = GpuState(w8)
    with pytest.raises(pkv.PKVError):
        st8.decode(vector=True)                      # G = 2: MFMA only


def test_empty_rows_are_zero():
    w = wl.custom(seed=5, lens=[40, 1, 70], n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16, dtype="bf16")
    st = GpuState(w)
    st.seq_lens[1] = 0
    out = st.decode(out_dtype=torch.float32)
    assert torch.all(out[1] == 0)
    ref = oracle_rows(w, [0, 2])
    assert max_abs_err(out, ref, rows=[0, 2]) <= TOL["bf16"]


def test_constant_values_give_the_constant():
    w = wl.build(3, small=True)
    st = GpuState(w)
    c = 1.375
    st.v_pool.fill_(c)
    out = st.decode(out_dtype=torch.float32)
    assert float((out - c).abs().max()) <= 1e-6


def test_nan_in_unused_slots_and_tables_never_leaks():
    w = wl.custom(seed=9, lens=[3, 17, 49, 300, 513], n_q_heads=16, n_kv_heads=2, head_dim=128, block_size=16,
                  dtype="f16", partition_size=64)
    st = GpuState(w, poison=True)
    # point every table entry past ceil(L/B) at a block full of NaN
    free_block = st.alloc.free_list()[0]
    st.k_pool[free_block].fill_(float("nan"))
    st.v_pool[free_block].fill_(float("nan"))
    for r in range(w.num_seqs):
        nb = -(-int(w.seq_lens[r]) // w.block_size)
        st.tables[r, nb:] = free_block
    out = st.decode(out_dtype=torch.float32)
    assert torch.isfinite(out).all()
    ref = oracle_rows(w, range(w.num_seqs))
    assert max_abs_err(out, ref, rows=range(w.num_seqs)) <= TOL["f16"]


@pytest.mark.parametrize("cid", [2, 3])
def test_large_q_is_stable(cid):
    w = wl.build(cid, small=True)
    st = GpuState(w)
    q_big = (st.q.float() * 1000).to(st.q.dtype)
    out = st.decode(out_dtype=torch.float32, q=q_big)
    assert torch.isfinite(out).all()
    ref = oracle_rows(w, range(w.num_seqs), q_np=wl.storage_to_numpy(q_big))
    err = max_abs_err(out, ref, rows=range(w.num_seqs))
    log(f"q x1000 config {cid}: err {err:.3e}")
    assert err <= TOL[w.dtype]


def test_lengths_above_max_seq_len_are_clamped():
    w = wl.custom(seed=21, lens=[100, 300, 250], n_q_heads=8, n_kv_heads=1, head_dim=128, block_size=16,
                  dtype="bf16")
    st = GpuState(w)
    out = st.decode(out_dtype=torch.float32, max_seq_len=200)
    from oracle import attention as O
    q = wl.storage_to_numpy(wl.q_values(w))
    for r, L in enumerate([100, 200, 200]):
        K, V = wl.logical_kv(w, r)
        ref = O.attention_logical(O.to_f64(q[r], "bf16"), O.to_f64(wl.storage_to_numpy(K[:L]), "bf16"),
                                  O.to_f64(wl.storage_to_numpy(V[:L]), "bf16"), w.scale)
        assert float(np.max(np.abs(out[r].double().cpu().numpy() - ref))) <= TOL["bf16"]


# ------------------------------------------------------------------------- more than 64 partitions a row
@pytest.mark.parametrize("dtype,D,G", [("bf16", 128, 8), ("f16", 64, 1), ("f32", 64, 2)])
def test_merge_past_64_partitions(dtype, D, G):
    """Rows of 65, 66 and 128 partitions of 32 tokens (and a 1-token row): the merge reads the
    partitions' maxima 64 lanes at a time, so these rows take its second and later passes."""
    lens = [32 * 128, 32 * 65 + 5, 32 * 66, 1, 33]
    w = wl.custom(seed=77 + D + G, lens=lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=D, block_size=16,
                  dtype=dtype, partition_size=32)
    st = GpuState(w)
    ref = oracle_all(w)
    for odt in (TORCH_DTYPE[dtype], torch.float32):
        out = st.decode(out_dtype=odt)
        err, row = max_abs_err_rows(out, ref)
        log(f"{dtype} D={D} G={G} P=32 (up to 128 partitions), out {odt}: max abs err {err:.3e} (row {row})")
        assert err <= TOL[dtype], err


# ------------------------------------------------------------------------- full sizes, every row
@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_full_size_all_rows(cid):
    """The bench's launch (KV-dtype output, the workload's own partition size) over the whole batch,
    every element of every row against the oracle."""
    w = wl.build(cid)
    log(f"full config {cid}: {w.describe()}")
    st = GpuState(w, poison=True)
    out = st.decode()
    del st
    torch.cuda.empty_cache()
    err, row = max_abs_err_rows(out, oracle_all(w))
    log(f"  all {w.num_seqs} rows: max abs err {err:.3e} (row {row}, L={int(w.seq_lens[row])})")
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("B", [8, 16, 32])
def test_full_size_long_context_512_token_partitions(B):
    """8 x 65,536 tokens in 512-token partitions (128 per row), random and identity placement:
    every row against the oracle, and the two placements bit-identical (any free block serves any
    sequence; the summation order depends only on logical positions).  The 2048-token partitions
    the bench uses are checked against the oracle as well."""
    outs = {}
    for placement in ("random", "identity"):
        w = wl.build(5, block_size=B, placement=placement)
        st = GpuState(w, poison=True)
        outs[placement] = st.decode(partition_size=512)
        if placement == "random":
            outs["P2048"] = st.decode(partition_size=2048)
        del st
        torch.cuda.empty_cache()
    ref = oracle_all(w)
    for k, o in outs.items():
        err, row = max_abs_err_rows(o, ref)
        log(f"config 5 B={B} {k}: max abs err over all rows {err:.3e} (row {row})")
        assert err <= TOL["bf16"], (k, err)
    assert torch.equal(_bits(outs["random"]), _bits(outs["identity"]))


def test_full_size_shared_prefix_equals_copied_prefix_bitwise():
    """The swarm at full size: 20 rows sharing the 250 physical blocks of a 4000-token prompt decode
    to the same bits as 20 private copies of it, with either load policy; every row against the
    copied-prefix oracle."""
    shared, copied = wl.build(4), wl.build(4, copied_prefix=True)
    a = GpuState(shared, poison=True)
    assert a.alloc.stats()["shared_blocks"] == 250
    oa, oa_cached = a.decode(), a.decode(shared_kv=True)
    oa_prefix = a.decode(shared_prefix_tokens=4000)
    del a
    torch.cuda.empty_cache()
    b = GpuState(copied, poison=True)
    assert b.alloc.stats()["shared_blocks"] == 0
    ob = b.decode()
    assert torch.equal(_bits(oa_prefix), _bits(oa))
    del b
    torch.cuda.empty_cache()
    assert torch.equal(_bits(oa), _bits(ob))
    assert torch.equal(_bits(oa_cached), _bits(oa))
    err, row = max_abs_err_rows(ob, oracle_all(copied))
    log(f"config 4 full, shared == copied bitwise; all rows: max abs err {err:.3e} (row {row})")
    assert err <= TOL["f16"], err


def test_out_of_pool_table_entries_are_reported():
    """A row whose table names a block outside the pool: the device check and the host check report it
    (count and first row), the runtime's debug mode refuses to decode, and the decode itself, which
    clamps such ids, still completes without a fault."""
    w = wl.custom(seed=41, lens=[40, 300, 17, 513], n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                  dtype="bf16")
    st = GpuState(w)
    r = pkv.check_block_tables(st.tables, st.seq_lens, w.block_size, w.num_blocks, w.max_seq_len)
    torch.cuda.synchronize()
    assert r.cpu().tolist() == [0, 2 ** 31 - 1]
    st.tables[1, 5] = w.num_blocks + 7
    st.tables[3, 0] = -3
    st.tables[2, 3] = w.num_blocks       # past row 2's two blocks: never read, never reported
    r = pkv.check_block_tables(st.tables, st.seq_lens, w.block_size, w.num_blocks, w.max_seq_len)
    torch.cuda.synchronize()
    log(f"device table check: {r.cpu().tolist()}")
    assert r.cpu().tolist() == [2, 1]
    assert pkv.validate_block_tables(st.tables.cpu().numpy(), st.seq_lens.cpu().numpy(), w.block_size,
                                     w.num_blocks, w.max_seq_len) == (2, 1)
    out = st.decode(out_dtype=torch.float32)
    assert torch.isfinite(out[[0, 2]]).all()
    # the runtime's debug mode stops before decoding such tables
    from paged_kv_cache_53_amd.runtime import DecodeBatch, PagedKVCache
    cache = PagedKVCache(64, 16, 2, 128, torch.bfloat16, fill="nan")
    cache.append(0, torch.randn(40, 2, 128).to(torch.bfloat16).cuda(), torch.randn(40, 2, 128).to(torch.bfloat16).cuda())
    batch = DecodeBatch(cache, [0], 8, 128, partition_size=64)
    batch.check_tables = True
    q = torch.randn(1, 8, 128).to(torch.bfloat16).cuda()
    o = torch.empty(1, 8, 128, dtype=torch.bfloat16, device="cuda")
    batch.decode_only(q, o)                                   # a good table decodes
    batch.tables[0, 1] = 64
    with pytest.raises(pkv.PKVError, match="out-of-pool"):
        batch.decode_only(q, o)

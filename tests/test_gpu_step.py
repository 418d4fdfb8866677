"""GPU parity of the fused decode step (pkv_decode_step) against the separate calls and the oracle.

The step must leave exactly what pkv_append_slots + pkv_reshape_and_cache(_fp8) +
pkv_paged_attention_decode(_ex/_fp8) leave: the same bits in the pools, the block tables, the
lengths and the output (compared bit for bit), and the output is within the decode's tolerance of
the fp64 oracle's whole pipeline (allocator, scatter, decode).  The slot mapping is read from pinned
host memory (the runtime's staging buffer) or from device memory.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_53_amd as pkv
import workloads as wl
from harness import TOL, TORCH_DTYPE, GpuState, log, max_abs_err, oracle_paged

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32).cpu()
    if t.element_size() == 1:
        return t.view(torch.uint8).cpu()
    return t.view(torch.int16).cpu()


def _two_states(w):
    """The same pre-step cache twice: one for the fused step, one for the separate calls."""
    a = GpuState(w, step=False)
    b = GpuState(w, step=False)
    assert np.array_equal(a.step_slots, b.step_slots)
    return a, b


def _run_fused(st, slots, out, partition_size=None, shared_kv=False):
    w = st.w
    pkv.decode_step(out, st.q, st.kn, st.vn, slots, st.k_pool, st.v_pool, st.tables, st.seq_lens, w.scale,
                    w.max_seq_len, w.partition_size if partition_size is None else partition_size,
                    shared_kv=shared_kv, **st.scales)


def _run_separate(st, slots_dev, out, partition_size=None, shared_kv=False):
    w = st.w
    pkv.append_slots(slots_dev, st.tables, st.seq_lens, w.block_size)
    pkv.reshape_and_cache(st.kn, st.vn, slots_dev, st.k_pool, st.v_pool, **st.scales)
    pkv.paged_attention_decode(out, st.q, st.k_pool, st.v_pool, st.tables, st.seq_lens, w.scale, w.max_seq_len,
                               w.partition_size if partition_size is None else partition_size,
                               shared_kv=shared_kv, **st.scales)


def _assert_same_state(a, b, out_a, out_b):
    assert torch.equal(_bits(out_a), _bits(out_b)), "outputs differ"
    assert torch.equal(_bits(a.k_pool), _bits(b.k_pool)), "key pools differ"
    assert torch.equal(_bits(a.v_pool), _bits(b.v_pool)), "value pools differ"
    assert torch.equal(a.tables.cpu(), b.tables.cpu()), "block tables differ"
    assert torch.equal(a.seq_lens.cpu(), b.seq_lens.cpu()), "lengths differ"


CASES = [(1, "native"), (2, "native"), (3, "native"), (4, "native"), (5, "native"),
         (2, "fp8"), (3, "fp8"), (4, "fp8"), (5, "fp8")]


@pytest.mark.parametrize("cid,kv", CASES)
def test_step_equals_separate_calls_and_matches_oracle(cid, kv):
    w = wl.build(cid, small=True) if cid != 1 else wl.build(1)
    if kv == "fp8":
        w = wl.quantised(w)
    log(f"config {cid} small, {kv} cache: {w.describe()}")
    a, b = _two_states(w)
    slots_host = torch.from_numpy(a.step_slots).pin_memory()
    slots_dev = torch.from_numpy(b.step_slots).to("cuda")
    shape = (w.num_seqs, w.n_q_heads, w.head_dim)
    out_a = torch.full(shape, float("nan"), dtype=TORCH_DTYPE[w.dtype], device="cuda")
    out_b = torch.full(shape, float("nan"), dtype=TORCH_DTYPE[w.dtype], device="cuda")
    _run_fused(a, slots_host, out_a)
    _run_separate(b, slots_dev, out_b)
    torch.cuda.synchronize()
    _assert_same_state(a, b, out_a, out_b)
    assert np.array_equal(a.seq_lens.cpu().numpy(), w.seq_lens)
    ref, _, _ = oracle_paged(w)
    err = max_abs_err(out_a, ref)
    log(f"  fused step vs oracle: max abs err {err:.3e}")
    assert err <= TOL[w.dtype], err


@pytest.mark.parametrize("where", ["device", "pinned"])
@pytest.mark.parametrize("dtype,G,D,B,P", [("bf16", 8, 128, 16, 64), ("f16", 1, 64, 8, 32),
                                           ("f32", 4, 64, 32, 96), ("bf16", 16, 64, 32, 0)])
def test_step_shapes_and_slot_memory(where, dtype, G, D, B, P):
    rng = np.random.default_rng(11)
    lens = rng.integers(1, 400, size=37)
    lens[:4] = [1, B, B + 1, 2 * B]     # a first token, and tokens that open a new block
    w = wl.custom(seed=11, lens=lens, n_q_heads=2 * G, n_kv_heads=2, head_dim=D, block_size=B, dtype=dtype,
                  partition_size=P)
    a, b = _two_states(w)
    slots = torch.from_numpy(a.step_slots)
    slots = slots.pin_memory() if where == "pinned" else slots.to("cuda")
    out_a = torch.empty(w.num_seqs, w.n_q_heads, D, dtype=TORCH_DTYPE[dtype], device="cuda")
    out_b = torch.empty_like(out_a)
    _run_fused(a, slots, out_a)
    _run_separate(b, torch.from_numpy(b.step_slots).to("cuda"), out_b)
    torch.cuda.synchronize()
    _assert_same_state(a, b, out_a, out_b)
    ref, _, _ = oracle_paged(w)
    assert max_abs_err(out_a, ref) <= TOL[dtype]


def test_step_skips_rows_with_negative_slots():
    """A negative slot leaves its row's pools, table and length alone in both forms; the rows then
    attend over the tokens they hold."""
    w = wl.custom(seed=5, lens=[17, 33, 1, 64, 200, 5], n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                  dtype="bf16", partition_size=64)
    a, b = _two_states(w)
    slots = a.step_slots.copy()
    slots[[1, 4]] = -1
    lens_before = a.seq_lens.cpu().clone()
    out_a = torch.empty(w.num_seqs, w.n_q_heads, w.head_dim, dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)
    _run_fused(a, torch.from_numpy(slots).pin_memory(), out_a)
    _run_separate(b, torch.from_numpy(slots).to("cuda"), out_b)
    torch.cuda.synchronize()
    _assert_same_state(a, b, out_a, out_b)
    after = a.seq_lens.cpu()
    assert after[1] == lens_before[1] and after[4] == lens_before[4]
    assert after[0] == lens_before[0] + 1


def test_step_on_an_empty_batch_is_a_no_op():
    st = GpuState(wl.custom(seed=1, lens=[3], n_q_heads=4, n_kv_heads=4, head_dim=64, block_size=16,
                            dtype="f16"), step=False)
    e = torch.empty(0, 4, 64, dtype=torch.float16, device="cuda")
    kv = torch.empty(0, 4, 64, dtype=torch.float16, device="cuda")
    pkv.decode_step(e, e, kv, kv, torch.empty(0, dtype=torch.int64, device="cuda"), st.k_pool, st.v_pool,
                    st.tables[:0], st.seq_lens[:0], 0.125, 16, 512)
    torch.cuda.synchronize()


def test_step_rejects_pageable_host_slots():
    w = wl.custom(seed=2, lens=[9, 20], n_q_heads=4, n_kv_heads=2, head_dim=64, block_size=16, dtype="f16")
    st = GpuState(w, step=False)
    out = torch.empty(2, 4, 64, dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        _run_fused(st, torch.from_numpy(st.step_slots), out)     # not pinned: the binding refuses
    # the library itself refuses pageable memory before any launch (no state changes)
    host = np.ascontiguousarray(st.step_slots)
    lens_before = st.seq_lens.cpu().clone()
    wsb = pkv.workspace_size(2, 4, 64, w.max_seq_len, 512)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    args = pkv._lib.pkv_decode_step_args(
        k=st.kn.data_ptr(), v=st.vn.data_ptr(), slot_mapping=host.ctypes.data, k_pool=st.k_pool.data_ptr(),
        v_pool=st.v_pool.data_ptr(), num_blocks=w.num_blocks, block_tables=st.tables.data_ptr(),
        seq_lens=st.seq_lens.data_ptr(), block_table_stride=st.tables.stride(0), num_seqs=2, n_q_heads=4,
        n_kv_heads=2, head_dim=64, block_size=16, out=out.data_ptr(), out_dtype=pkv.PKV_F16, dtype=pkv.PKV_F16,
        q=st.q.data_ptr(), scale=0.125, max_seq_len=w.max_seq_len, partition_size=512, workspace=ws.data_ptr(),
        workspace_bytes=wsb)
    assert pkv.lib().pkv_decode_step(args, None) == pkv.PKV_ERR_INVALID
    torch.cuda.synchronize()
    assert torch.equal(st.seq_lens.cpu(), lens_before)


@pytest.mark.parametrize("kv", ["native", "fp8"])
def test_runtime_steps_fused_equal_unfused_with_forks(kv):
    """Twenty runtime steps over forked rows (copy-on-write on the first append into a shared,
    partly filled block): the fused and the separate-call steps give the same bits every step, and
    so does the fused step with the load policy forced to streamed loads (the runtime picks cacheable
    loads for a batch with shared blocks).  Twenty steps cycle the batch's ring of slot stages more
    than twice, so stages are rewritten after the step that read them has finished."""
    from paged_kv_cache_53_amd.runtime import DecodeBatch, PagedKVCache
    Hk, D, B, G = 2, 128, 16, 4
    outs, pools = {}, {}
    for fused, policy in ((True, "auto"), (False, "auto"), (True, "streamed")):
        kw = dict(k_scale=0.02, v_scale=0.03) if kv == "fp8" else {}
        dt = torch.float8_e4m3fn if kv == "fp8" else torch.bfloat16
        cache = PagedKVCache(256, B, Hk, D, dt, device="cuda", fill="zero", **kw)
        g = torch.Generator(device="cpu").manual_seed(3)
        prompt = torch.randn(45, Hk, D, generator=g).to(torch.bfloat16).cuda()
        cache.append(0, prompt, prompt * 0.5)
        for child in (1, 2):
            cache.fork(0, child)
        cache.append(3, prompt[:20], prompt[:20] * 2)
        batch = DecodeBatch(cache, [0, 1, 2, 3], G * Hk, 128, partition_size=32)
        batch.load_policy = policy
        # rows 0-2 share the 45-token prompt's three blocks: read cacheable, the rest streamed
        assert batch._load_args() == ({"shared_prefix_tokens": 45} if policy == "auto" else {})
        seq = []
        for i in range(20):
            q = torch.randn(4, G * Hk, D, generator=g).to(torch.bfloat16).cuda()
            kn = torch.randn(4, Hk, D, generator=g).to(torch.bfloat16).cuda()
            vn = torch.randn(4, Hk, D, generator=g).to(torch.bfloat16).cuda()
            out = torch.empty(4, G * Hk, D, dtype=torch.bfloat16, device="cuda")
            batch.step(q, kn, vn, out, fused=fused)
            seq.append(out.clone())
        torch.cuda.synchronize()
        outs[(fused, policy)] = seq
        pools[(fused, policy)] = (cache.k_pool.clone(), cache.v_pool.clone(), batch.tables.clone(),
                                  batch.seq_lens.clone())
    ref = (True, "auto")
    for other in ((False, "auto"), (True, "streamed")):
        for x, y in zip(outs[ref], outs[other]):
            assert torch.equal(_bits(x), _bits(y)), other
        for x, y in zip(pools[ref], pools[other]):
            assert torch.equal(_bits(x), _bits(y)), other
    assert torch.isfinite(outs[ref][-1].float()).all()


@pytest.mark.parametrize("kv", ["native", "fp8"])
def test_step_full_size_llama70b_batch(kv):
    """The bench's workload and launch (256 rows, 1.2 M tokens, partitions of 3072): the fused step
    leaves the same bits as the separate calls, and every row matches the oracle."""
    w = wl.build(3)
    if kv == "fp8":
        w = wl.quantised(w)
    log(f"full config 3, {kv} cache: {w.describe()}")
    a, b = _two_states(w)
    out_a = torch.empty(w.num_seqs, w.n_q_heads, w.head_dim, dtype=TORCH_DTYPE[w.dtype], device="cuda")
    out_b = torch.empty_like(out_a)
    _run_fused(a, torch.from_numpy(a.step_slots).pin_memory(), out_a)
    _run_separate(b, torch.from_numpy(b.step_slots).to("cuda"), out_b)
    torch.cuda.synchronize()
    _assert_same_state(a, b, out_a, out_b)
    del b
    torch.cuda.empty_cache()
    del a
    torch.cuda.empty_cache()
    from harness import max_abs_err_rows, oracle_all
    err, row = max_abs_err_rows(out_a, oracle_all(w))
    log(f"  all {w.num_seqs} rows: max abs err {err:.3e} (row {row}, L={int(w.seq_lens[row])})")
    assert err <= TOL[w.dtype], err

"""GPU parity of the quantised cache (FP8 E4M3 pools with per-tensor scales) against the oracle.

The scatter's codes are compared bit for bit with the oracle's quantisation (oracle.fp8: the fp32
quotient, nearest code, ties even, saturation, NaN), over every byte of both pools.  Decode is
compared with the fp64 oracle on the dequantised values (k_scale * value(code), v_scale *
value(code)), within the tolerance of 16-bit KV: max |gpu - oracle| <= 2e-2 (the codes widen to
q's type exactly; the error is that of the 16-bit MFMA path).  Scale invariances are bit-exact.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_53_amd as pkv
import workloads as wl
from harness import (TOL, TORCH_DTYPE, GpuState, log, max_abs_err, max_abs_err_rows, oracle_all,
                     oracle_paged, oracle_rows)

pytestmark = pytest.mark.gpu

FP8 = torch.float8_e4m3fn


def _codes(t):
    return t.view(torch.uint8).cpu().numpy()


def _edge_rows(rng, T, Hk, D, scale):
    """Rows whose quotients x / scale hit the encoder's cases: midpoints between codes (ties), values
    just off them, the subnormal range, saturation, infinities, NaN, signed zeros, plus N(0, 1)."""
    from oracle import fp8 as F
    mids = [(F.decode_code(c) + F.decode_code(c + 1)) / 2 for c in range(0x7E)]
    special = mids + [-m for m in mids] + [448.0, 449.0, 464.0, 480.0, 1e4, -1e4, 2.0 ** -10, 3 * 2.0 ** -10,
                                           2.0 ** -12, -2.0 ** -10, 0.0, -0.0, np.inf, -np.inf, np.nan]
    x = rng.standard_normal((T, Hk, D)).astype(np.float32) * 2
    flat = x.reshape(-1)
    vals = np.array(special, dtype=np.float64) * scale
    flat[:len(vals)] = vals.astype(np.float32)
    return x


@pytest.mark.parametrize("src", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("B", [8, 16, 32])
def test_fp8_scatter_codes_bit_exact_vs_oracle(src, B):
    from oracle import attention as O
    from oracle import scatter as SC
    rng = np.random.default_rng(11 + B)
    N, Hk, D, T = 40, 2, 128, 96
    ks, vs = 0.0125, 2.0 ** -3
    k32 = _edge_rows(rng, T, Hk, D, ks)
    v32 = _edge_rows(rng, T, Hk, D, vs)
    dt = TORCH_DTYPE[src]
    k = torch.from_numpy(k32).to(dt)          # rows as the library receives them
    v = torch.from_numpy(v32).to(dt)
    slots = rng.permutation(N * B)[:T].astype(np.int64)
    slots[3], slots[7] = -1, N * B + 5        # padding token and an out-of-pool slot: skipped
    kp = torch.full(pkv.key_pool_shape(N, Hk, D, B, FP8), 0xA5, dtype=torch.uint8, device="cuda").view(FP8)
    vp = torch.full(pkv.value_pool_shape(N, Hk, D, B), 0xA5, dtype=torch.uint8, device="cuda").view(FP8)
    pkv.reshape_and_cache(k.cuda(), v.cuda(), torch.from_numpy(slots).cuda(), kp, vp, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    okp, ovp = SC.empty_pools(N, Hk, D, B, np.uint8, 0xA5)
    kx = O.to_f64(pkv_storage(k), src).astype(np.float32)     # the exact values of the rows sent
    vx = O.to_f64(pkv_storage(v), src).astype(np.float32)
    SC.reshape_and_cache_fp8(kx, vx, slots, okp, ovp, ks, vs)
    assert np.array_equal(_codes(kp), okp)
    assert np.array_equal(_codes(vp), ovp)
    log(f"fp8 scatter {src} B={B}: {T} tokens, codes bit-exact")


def pkv_storage(t):
    return wl.storage_to_numpy(t)


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_fp8_small_configs_full_oracle_pipeline(cid):
    w = wl.quantised(wl.build(cid, small=True))
    log(f"config {cid} small fp8: {w.describe()}")
    st = GpuState(w)
    ref, model, tables, okp, ovp = oracle_paged(w, with_pools=True)
    for odt in (TORCH_DTYPE[w.dtype], torch.float32):
        out = st.decode(out_dtype=odt)
        err = max_abs_err(out, ref)
        log(f"  out {odt}: max abs err {err:.3e}")
        assert err <= TOL[w.dtype], err
    # the pools the library built hold exactly the oracle's codes wherever a table points
    for r in range(w.num_seqs):
        L = int(w.seq_lens[r])
        nb = -(-L // w.block_size)
        ids = st.tables_host[r, :nb]
        assert np.array_equal(_codes(st.k_pool[torch.from_numpy(ids).long().cuda()]), okp[ids])
        assert np.array_equal(_codes(st.v_pool[torch.from_numpy(ids).long().cuda()]), ovp[ids])


SWEEP = []
for dtype in ("bf16", "f16"):
    for G in (1, 3, 8, 16):
        for D in (64, 128):
            SWEEP.append((dtype, G, D, (8, 16, 32)[(G + D // 64) % 3]))


@pytest.mark.parametrize("dtype,G,D,B", SWEEP)
def test_fp8_heads_dims_blocks_sweep(dtype, G, D, B):
    Hk = 2
    lens = [1, 15, 16, 17, 33, 100, 511, 513, 1000]
    w = wl.quantised(wl.custom(seed=300 + G * 7 + D, lens=lens, n_q_heads=G * Hk, n_kv_heads=Hk, head_dim=D,
                               block_size=B, dtype=dtype, partition_size=128))
    st = GpuState(w)
    ref = oracle_rows(w, range(w.num_seqs))
    out = st.decode(out_dtype=torch.float32)
    err = max_abs_err(out, ref, rows=range(w.num_seqs))
    log(f"fp8 {dtype} G={G} D={D} B={B}: err {err:.3e}")
    assert err <= TOL[dtype], err
    # length 1: weight exactly 1, so the output is v_scale * value(code) rounded once to fp32
    from oracle import fp8 as F
    vcode = _codes(st.v_pool[int(st.tables_host[0, 0])])[:, :, 0]          # [Hk, D]: token 0 of the block
    exp = torch.from_numpy(np.float32(w.v_scale) * F.decode(vcode).astype(np.float32)).repeat_interleave(G, dim=0)
    assert torch.equal(out[0].cpu(), exp)


def test_fp8_scales_are_exact_power_of_two_factors():
    # doubling k_scale is doubling the score scale (one fp32 product on the host either way), and
    # doubling v_scale doubles every output exactly
    w = wl.quantised(wl.build(3, small=True))
    st = GpuState(w)
    base = st.decode(out_dtype=torch.float32)
    a = st.decode(out_dtype=torch.float32, scales={"k_scale": 2 * w.k_scale, "v_scale": w.v_scale})
    b_out = torch.full_like(base, float("nan"))
    pkv.paged_attention_decode(b_out, st.q, st.k_pool, st.v_pool, st.tables, st.seq_lens, 2 * w.scale,
                               w.max_seq_len, w.partition_size, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    assert torch.equal(a, b_out)
    c = st.decode(out_dtype=torch.float32, scales={"k_scale": w.k_scale, "v_scale": 2 * w.v_scale})
    assert torch.equal(c, 2 * base)


def test_fp8_saturated_cache_matches_oracle():
    # scales small enough that the tails of the N(0, 1) rows saturate at +-448 codes
    w = wl.quantised(wl.build(2, small=True), k_scale=2.0 ** -8, v_scale=0.005)
    st = GpuState(w)
    assert int((_codes(st.k_pool) & 0x7F == 0x7E).sum()) > 0         # some keys saturated
    ref = oracle_rows(w, range(w.num_seqs))
    out = st.decode(out_dtype=torch.float32)
    err = max_abs_err(out, ref, rows=range(w.num_seqs))
    log(f"fp8 saturated: err {err:.3e}")
    assert err <= TOL[w.dtype]


def test_fp8_nan_codes_in_unused_slots_and_tables_never_leak():
    w = wl.quantised(wl.custom(seed=9, lens=[3, 17, 49, 300, 513], n_q_heads=16, n_kv_heads=2, head_dim=128,
                               block_size=16, dtype="bf16", partition_size=64))
    st = GpuState(w, poison=True)                 # every unwritten slot holds the NaN code
    free_block = st.alloc.free_list()[0]
    for r in range(w.num_seqs):
        nb = -(-int(w.seq_lens[r]) // w.block_size)
        st.tables[r, nb:] = free_block
    out = st.decode(out_dtype=torch.float32)
    assert torch.isfinite(out).all()
    ref = oracle_rows(w, range(w.num_seqs))
    assert max_abs_err(out, ref, rows=range(w.num_seqs)) <= TOL["bf16"]


def test_fp8_shared_prefix_cache_policy_changes_no_bit():
    w = wl.quantised(wl.build(4, small=True))
    st = GpuState(w)
    a = st.decode()
    b = st.decode(shared_kv=True)
    assert torch.equal(a.view(torch.int16).cpu(), b.view(torch.int16).cpu())
    for n in (400, 32, 100000):
        c = st.decode(shared_prefix_tokens=n)
        assert torch.equal(a.view(torch.int16).cpu(), c.view(torch.int16).cpu()), n
    ref = oracle_rows(w, range(w.num_seqs))
    assert max_abs_err(a, ref, rows=range(w.num_seqs)) <= TOL[w.dtype]


def test_fp8_runtime_decode_step_with_copy_on_write():
    """The runtime on an FP8 cache: prompt, forks, decode steps (appends into shared blocks get
    private copies of the codes); each step's output against the oracle on the quantised history."""
    from oracle import attention as O
    from oracle import fp8 as F
    from paged_kv_cache_53_amd.runtime import DecodeBatch, PagedKVCache
    rng = np.random.default_rng(17)
    N, B, Hk, G, D = 64, 16, 2, 4, 64
    Hq = Hk * G
    ks, vs = 0.02, 0.015
    cache = PagedKVCache(N, B, Hk, D, FP8, free_order=rng.permutation(N).tolist(), fill="nan",
                         k_scale=ks, v_scale=vs)
    hist = {}
    pk = torch.randn(21, Hk, D).to(torch.bfloat16)
    pv = torch.randn(21, Hk, D).to(torch.bfloat16)
    cache.append(0, pk.cuda(), pv.cuda())
    hist[0] = (pk, pv)
    for c in (1, 2):
        cache.fork(0, c)
        hist[c] = (pk.clone(), pv.clone())
    seqs = [0, 1, 2]
    batch = DecodeBatch(cache, seqs, Hq, 64, partition_size=32)
    for step in range(3):
        q = torch.randn(3, Hq, D).to(torch.bfloat16)
        kn = torch.randn(3, Hk, D).to(torch.bfloat16)
        vn = torch.randn(3, Hk, D).to(torch.bfloat16)
        out = torch.empty(3, Hq, D, dtype=torch.float32, device="cuda")
        batch.step(q.cuda(), kn.cuda(), vn.cuda(), out)
        torch.cuda.synchronize()
        for i, s in enumerate(seqs):
            hk, hv = hist[s]
            hist[s] = (torch.cat([hk, kn[i:i + 1]]), torch.cat([hv, vn[i:i + 1]]))
            K = F.dequantize(F.quantize(hist[s][0].float().numpy(), ks), ks)
            V = F.dequantize(F.quantize(hist[s][1].float().numpy(), vs), vs)
            ref = O.attention_logical(q[i].double().numpy(), K, V, batch.scale)
            err = float(np.max(np.abs(out[i].double().cpu().numpy() - ref)))
            assert err <= TOL["bf16"], (step, s, err)
    assert cache.allocator.stats()["shared_blocks"] == 1     # the prompt's first full block


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_fp8_full_size_all_rows(cid):
    """The bench's FP8 launch (q-dtype output, the workload's own partition size) over the whole
    batch, every element of every row against the oracle on the dequantised codes."""
    w = wl.quantised(wl.build(cid))
    log(f"full config {cid} fp8: {w.describe()}")
    st = GpuState(w, poison=True)
    out = st.decode()
    del st
    torch.cuda.empty_cache()
    err, row = max_abs_err_rows(out, oracle_all(w))
    log(f"  all {w.num_seqs} rows: max abs err {err:.3e} (row {row}, L={int(w.seq_lens[row])})")
    assert err <= TOL[w.dtype], err


def test_fp8_full_size_shared_prefix_equals_copied_prefix_bitwise():
    """The swarm on an FP8 cache at full size: shared prompt blocks and private copies of them decode
    to the same bits, with either load policy; every row against the copied-prefix oracle."""
    shared, copied = wl.quantised(wl.build(4)), wl.quantised(wl.build(4, copied_prefix=True))
    a = GpuState(shared, poison=True)
    assert a.alloc.stats()["shared_blocks"] == 250
    oa, oa_cached = a.decode(), a.decode(shared_kv=True)
    assert torch.equal(a.decode(shared_prefix_tokens=4000).view(torch.int16).cpu(), oa.view(torch.int16).cpu())
    del a
    torch.cuda.empty_cache()
    b = GpuState(copied, poison=True)
    ob = b.decode()
    del b
    torch.cuda.empty_cache()
    assert torch.equal(oa.view(torch.int16).cpu(), ob.view(torch.int16).cpu())
    assert torch.equal(oa_cached.view(torch.int16).cpu(), oa.view(torch.int16).cpu())
    err, row = max_abs_err_rows(ob, oracle_all(copied))
    log(f"config 4 full fp8, shared == copied bitwise; all rows: max abs err {err:.3e} (row {row})")
    assert err <= TOL[copied.dtype], err

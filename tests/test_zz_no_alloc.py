"""The decode entry point that allocates nothing (pkv_paged_attention_decode_noalloc), called through the
C ABI: the same bits as pkv_paged_attention_decode_ex with a caller workspace, over two calls in a row on
one GPU (the second smaller, so it runs over what the first left in the static scratch), and within
the oracle's tolerance."""
import pytest
import torch

import paged_kv_cache_53_amd as pkv
import workloads as wl
from harness import TOL, GpuState, log, max_abs_err_rows, oracle_all

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


def _noalloc(st, out, P, shared_kv=False):
    w = st.w
    return pkv.lib().pkv_paged_attention_decode_noalloc(
        out.data_ptr(), pkv.dtype_code(out), st.q.data_ptr(), st.k_pool.data_ptr(), st.v_pool.data_ptr(),
        st.tables.data_ptr(), st.tables.stride(0), st.seq_lens.data_ptr(), w.num_seqs, w.n_q_heads,
        w.n_kv_heads, w.head_dim, w.block_size, w.num_blocks, w.scale, w.max_seq_len, P,
        pkv.dtype_code(st.k_pool), pkv.PKV_DECODE_SHARED_KV if shared_kv else 0,
        torch.cuda.current_stream().cuda_stream)


def test_noalloc_equals_workspace_decode_on_two_calls_in_a_row():
    cases = [(wl.build(3), 3072, torch.bfloat16),              # 256 rows, up to 11 partitions a row
             (wl.build(3, small=True), 64, torch.float32)]     # then a smaller call over the same scratch
    for w, P, odt in cases:
        need = pkv.workspace_size(w.num_seqs, w.n_q_heads, w.head_dim, w.max_seq_len, P)
        log(f"noalloc {w.name} ({w.variant}), P={P}: workspace {need} B of {pkv.PKV_STATIC_SCRATCH_BYTES}")
        assert 0 < need <= pkv.PKV_STATIC_SCRATCH_BYTES
        st = GpuState(w, poison=True)
        ref = st.decode(out_dtype=odt, partition_size=P)          # pkv_paged_attention_decode_ex, workspace
        out = torch.full_like(ref, float("nan"))
        assert _noalloc(st, out, P) == pkv.PKV_OK
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref))
        err, row = max_abs_err_rows(out, oracle_all(w))
        log(f"  noalloc == workspace decode bitwise; all rows: max abs err {err:.3e} (row {row})")
        assert err <= TOL[w.dtype], err
        del st
        torch.cuda.empty_cache()


def test_noalloc_shared_prefix_and_fp32():
    # the cacheable-load variant and the vector path take the same scratch
    for w, kw in ((wl.build(4, small=True), {"shared_kv": True}), (wl.build(1), {})):
        st = GpuState(w)
        ref = st.decode(out_dtype=torch.float32, partition_size=32, **kw)
        out = torch.full_like(ref, float("nan"))
        assert _noalloc(st, out, 32, **kw) == pkv.PKV_OK
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), w.name

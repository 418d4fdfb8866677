"""The C++ host allocator (libpagedkv) against the allocator model (oracle O2), bit for bit.

Compared after every operation: slots, copy pairs, block tables, lengths, reference counts,
the free list in order, and which error each side reports.  Runs on the CPU (host code only).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import paged_kv_cache_53_amd as pkv
import workloads as wl
from oracle.allocator import BlockAllocatorModel, OutOfBlocks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def same_state(model: BlockAllocatorModel, lib: pkv.Allocator):
    assert lib.free_list() == model.free
    assert [lib.ref_count(b) for b in range(model.num_blocks)] == model.ref
    for seq, t in model.tables.items():
        assert lib.block_table(seq) == t
        assert lib.seq_len(seq) == model.lens[seq]
    st_l, st_m = lib.stats(), model.stats()
    for k in ("free_blocks", "allocated_blocks", "shared_blocks", "num_seqs", "live_tokens", "allocated_slots"):
        assert st_l[k] == st_m[k], k


def apply_both(model, lib, kind, x, y, n):
    """Run one op on both; return the exception class each raised (None if fine)."""
    err_m = err_l = None
    res_m = res_l = None
    try:
        if kind == "alloc":
            res_m = model.alloc(x, n)
        elif kind == "fork":
            model.fork(x, y, n)
        else:
            model.free_seq(x)
    except OutOfBlocks:
        err_m = "oom"
    except KeyError:
        err_m = "missing"
    except ValueError:
        err_m = "invalid"
    try:
        if kind == "alloc":
            res_l = lib.alloc(x, n)
        elif kind == "fork":
            lib.fork(x, y, n)
        else:
            lib.free(x)
    except pkv.PKVError as e:
        err_l = {pkv.PKV_ERR_OOM: "oom", pkv.PKV_ERR_NOT_FOUND: "missing", pkv.PKV_ERR_INVALID: "invalid"}[e.status]
    assert err_m == err_l, (kind, x, y, n, err_m, err_l)
    if kind == "alloc" and err_m is None:
        assert res_l[0] == res_m[0] and res_l[1] == res_m[1]


ops = st.lists(st.tuples(st.sampled_from(["alloc", "alloc", "alloc", "fork", "free"]),
                         st.integers(0, 6), st.integers(0, 6), st.integers(-1, 45)), max_size=80)


@settings(max_examples=300, deadline=None)
@given(ops=ops, B=st.sampled_from([1, 2, 4, 8, 16]), N=st.integers(1, 30), seed=st.integers(0, 10 ** 6))
def test_matches_model_under_random_ops(ops, B, N, seed):
    order = np.random.default_rng(seed).permutation(N).tolist()
    model, lib = BlockAllocatorModel(N, B, order), pkv.Allocator(N, B, order)
    for kind, x, y, n in ops:
        if kind == "alloc":
            n = max(n, 0)
        apply_both(model, lib, kind, x, y, n)
        same_state(model, lib)


def apply_swap_ops(model, lib, kind, x, y, n):
    """The swap operations on both sides (plus the others); compares pairs and errors."""
    if kind not in ("swap_out", "swap_in"):
        return apply_both(model, lib, kind, x, y, n)
    err_m = err_l = None
    res_m = res_l = None
    try:
        res_m = model.swap_out(x) if kind == "swap_out" else model.swap_in(x)
    except OutOfBlocks:
        err_m = "oom"
    except KeyError:
        err_m = "missing"
    try:
        res_l = lib.swap_out(x) if kind == "swap_out" else lib.swap_in(x)
    except pkv.PKVError as e:
        err_l = {pkv.PKV_ERR_OOM: "oom", pkv.PKV_ERR_NOT_FOUND: "missing", pkv.PKV_ERR_INVALID: "invalid"}[e.status]
    assert err_m == err_l, (kind, x, err_m, err_l)
    if err_m is None:
        assert [tuple(p) for p in res_l] == [tuple(p) for p in res_m]


def same_swap_state(model, lib):
    same_state(model, lib)
    st = lib.swap_stats()
    assert st["host_free"] == len(model.host_free) and st["swapped_seqs"] == len(model.swapped)


swap_ops = st.lists(st.tuples(st.sampled_from(["alloc", "alloc", "alloc", "fork", "free", "swap_out", "swap_in",
                                               "swap_in"]),
                              st.integers(0, 6), st.integers(0, 6), st.integers(-1, 45)), max_size=80)


@settings(max_examples=300, deadline=None)
@given(ops=swap_ops, B=st.sampled_from([1, 4, 16]), N=st.integers(1, 30), H=st.integers(0, 20),
       seed=st.integers(0, 10 ** 6))
def test_swaps_match_model_under_random_ops(ops, B, N, H, seed):
    order = np.random.default_rng(seed).permutation(N).tolist()
    model, lib = BlockAllocatorModel(N, B, order), pkv.Allocator(N, B, order)
    model.set_swap_space(H)
    lib.set_swap_space(H)
    for kind, x, y, n in ops:
        if kind == "alloc":
            n = max(n, 0)
        apply_swap_ops(model, lib, kind, x, y, n)
        same_swap_state(model, lib)


def test_swap_requires_swap_space_and_reports_the_block_count():
    import ctypes as C
    lib = pkv.Allocator(8, 4)
    lib.alloc(0, 10)
    with pytest.raises(pkv.PKVError):
        lib.swap_out(0)                              # no swap space yet
    lib.set_swap_space(4)
    with pytest.raises(pkv.PKVError):
        lib.set_swap_space(4)                        # set once
    table = lib.block_table(0)
    n = C.c_int32(0)
    small = (C.c_int32 * 2)()
    assert pkv.lib().pkv_swap_out(lib._h, 0, small, 1, C.byref(n)) == pkv.PKV_ERR_INVALID
    assert n.value == 3 and lib.block_table(0) == table   # too small: nothing changed, count reported
    assert lib.swap_out(0) == [(b, h) for h, b in enumerate(table)]
    assert lib.free_list()[-3:] == table
    with pytest.raises(pkv.PKVError):
        lib.alloc(0, 1)                              # swapped out: cannot append
    with pytest.raises(pkv.PKVError):
        lib.block_table(0)                           # and has no table


@pytest.mark.parametrize("cid,copied", [(1, False), (2, False), (3, False), (4, False), (4, True), (5, False)])
def test_workload_scripts_give_identical_tables(cid, copied):
    w = wl.build(cid, small=True, copied_prefix=copied) if cid == 4 else wl.build(cid, small=True)
    model = BlockAllocatorModel(w.num_blocks, w.block_size, w.free_order)
    lib = pkv.Allocator(w.num_blocks, w.block_size, w.free_order)
    for op in w.prompt_ops:
        k = op["op"]
        if k == "alloc":
            apply_both(model, lib, "alloc", op["seq"], None, op["n"])
        elif k == "fork":
            apply_both(model, lib, "fork", op["parent"], op["child"], op["n"])
        else:
            apply_both(model, lib, "free", op["seq"], None, None)
    slots_m = []
    for seq in w.batch.tolist():
        slots_m += model.alloc(seq, 1)[0]
    slots_l, pairs = lib.alloc_batch(w.batch.tolist(), 1)
    assert slots_l.tolist() == slots_m and pairs == []
    same_state(model, lib)
    stride = max(len(model.block_table(int(s))) for s in w.batch) + 3
    tables, lens = lib.fill_block_tables(w.batch.tolist(), stride, pad=-1)
    for r, seq in enumerate(w.batch.tolist()):
        t = model.block_table(seq)
        assert tables[r, :len(t)].tolist() == t and (tables[r, len(t):] == -1).all()
        assert lens[r] == w.seq_lens[r]


def test_full_size_llama70b_tables_match():
    w = wl.build(3)
    model = BlockAllocatorModel(w.num_blocks, w.block_size, w.free_order)
    lib = pkv.Allocator(w.num_blocks, w.block_size, w.free_order)
    for op in w.prompt_ops:
        model.alloc(op["seq"], op["n"])
        lib.alloc(op["seq"], op["n"])
    for seq in w.batch.tolist():
        model.alloc(seq, 1)
    lib.alloc_batch(w.batch.tolist(), 1)
    stride = int(-(-w.max_seq_len // w.block_size))
    tables, lens = lib.fill_block_tables(w.batch.tolist(), stride, pad=-1)
    for r, seq in enumerate(w.batch.tolist()):
        t = model.block_table(seq)
        assert tables[r, :len(t)].tolist() == t
    assert lib.free_list() == model.free


def test_batch_alloc_is_atomic_and_rejects_repeats():
    lib = pkv.Allocator(4, 4)
    lib.alloc(0, 3)
    lib.alloc(1, 4)
    before = (lib.free_list(), lib.block_table(0), lib.block_table(1))
    with pytest.raises(pkv.OutOfBlocks):
        lib.alloc_batch([0, 1, 2], 6)        # needs 1 + 2 + 2 blocks, 2 free
    assert (lib.free_list(), lib.block_table(0), lib.block_table(1)) == before
    with pytest.raises(pkv.PKVError) as e:
        lib.alloc_batch([0, 0], 1)
    assert e.value.status == pkv.PKV_ERR_INVALID
    with pytest.raises(pkv.PKVError):
        lib.block_table(2)                   # the failed batch did not create sequence 2


def test_copy_on_write_pairs_in_batch():
    lib = pkv.Allocator(16, 4)
    model = BlockAllocatorModel(16, 4)
    for a in (lib, model):
        a.alloc(10, 6)
    lib.fork(10, 11, 6)
    model.fork(10, 11, 6)
    slots, pairs = lib.alloc_batch([11, 10], 1)
    s11, p11 = model.alloc(11, 1)
    s10, p10 = model.alloc(10, 1)
    assert pairs == p11 + p10 == [(1, 2)]
    assert slots.tolist() == s11 + s10
    same_state(model, lib)


def test_create_rejects_bad_orders():
    for args in [(0, 16, None), (4, 0, None), (4, 4, [0, 1, 2, 2]), (3, 4, [0, 1, 5])]:
        with pytest.raises(pkv.PKVError):
            pkv.Allocator(*args)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_asan_ubsan_session(tmp_path):
    exe = tmp_path / "alloc_asan"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           f"-I{ROOT}/include", f"{ROOT}/paged_kv_cache_53_amd/csrc/allocator.cpp",
           f"{ROOT}/tests/native/alloc_asan.cpp", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    r = subprocess.run([str(exe), "150"], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1",
                            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"

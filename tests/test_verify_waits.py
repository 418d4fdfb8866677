"""The static check of explicitly waited loads (paged_kv_cache_53_amd.verify_waits).

Small hand-written gfx9 assembly bodies exercise each rule: an in-flight destination register
must not be read, copied or overwritten before a covering s_waitcnt; vmcnt retires in order;
joins keep the most recent load; flag-guarded structurizer paths are followed only where the flag
value allows; scalars materialised from in-flight registers may not be used.  The library's own
kernel assembly, as compiled from the sources, must pass.
"""
import os

import pytest

from paged_kv_cache_53_amd import verify_waits as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _check(text):
    return V.check_kernel([l for l in text.strip("\n").splitlines()])


def _asm(line):
    return f";;#ASMSTART\n\t{line}\n;;#ASMEND"


def test_read_before_wait_is_reported():
    body = f"""
{_asm("global_load_dwordx4 v[4:7], v[0:1], off")}
\tv_mov_b32_e32 v8, v4
\ts_endpgm
"""
    assert len(_check(body)) == 1


def test_covering_wait_makes_read_safe():
    body = f"""
{_asm("global_load_dwordx4 v[4:7], v[0:1], off")}
{_asm("global_load_dwordx4 v[8:11], v[0:1], off")}
{_asm("s_waitcnt vmcnt(1)")}
\tv_mov_b32_e32 v20, v4
\ts_endpgm
"""
    assert _check(body) == []


def test_too_permissive_wait_is_reported():
    # vmcnt(2) leaves both loads possibly outstanding: the first one is not covered
    body = f"""
{_asm("global_load_dwordx4 v[4:7], v[0:1], off")}
{_asm("global_load_dwordx4 v[8:11], v[0:1], off")}
{_asm("s_waitcnt vmcnt(2)")}
\tv_add_f32_e32 v20, v4, v5
\ts_endpgm
"""
    assert len(_check(body)) == 1


def test_overwriting_an_in_flight_register_is_reported():
    body = f"""
{_asm("global_load_dwordx2 v[4:5], v[0:1], off")}
\tv_mov_b32_e32 v5, 0
\ts_endpgm
"""
    assert len(_check(body)) == 1


def test_compiler_loads_count_towards_the_wait():
    # a compiler-visible load issued after the asm load retires after it: vmcnt(1) covers the asm one
    body = f"""
{_asm("global_load_dwordx4 v[4:7], v[0:1], off")}
\tglobal_load_dword v12, v[0:1], off
\ts_waitcnt vmcnt(1)
\tv_mov_b32_e32 v20, v4
\ts_endpgm
"""
    assert _check(body) == []


def test_join_keeps_the_most_recent_load():
    # one branch waits, the other does not: the read after the join is unsafe
    body = f"""
{_asm("global_load_dwordx4 v[4:7], v[0:1], off")}
\ts_cbranch_scc1 .LBB0_2
{_asm("s_waitcnt vmcnt(0)")}
.LBB0_2:
\tv_mov_b32_e32 v20, v4
\ts_endpgm
"""
    assert len(_check(body)) == 1


def test_loop_carried_load_needs_a_wait_on_the_back_edge():
    body = f"""
.LBB0_1:
\tv_add_f32_e32 v20, v4, v20
{_asm("global_load_dwordx4 v[4:7], v[0:1], off")}
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
"""
    assert len(_check(body)) == 1
    fixed = body.replace("\tv_add_f32_e32", _asm("s_waitcnt vmcnt(0)") + "\n\tv_add_f32_e32")
    assert _check(fixed) == []


def test_flag_guarded_infeasible_path_is_not_followed():
    # the block that skips the wait always sets s[8:9] = -1, which sends the flow block to the exit
    body = f"""
{_asm("global_load_dwordx4 v[4:7], v[0:1], off")}
\ts_cbranch_scc1 .LBB0_3
{_asm("s_waitcnt vmcnt(0)")}
\ts_mov_b64 s[8:9], 0
\ts_branch .LBB0_4
.LBB0_3:
\ts_mov_b64 s[8:9], -1
.LBB0_4:
\ts_and_b64 vcc, exec, s[8:9]
\ts_cbranch_vccnz .LBB0_5
\tv_mov_b32_e32 v20, v4
.LBB0_5:
\ts_endpgm
"""
    assert _check(body) == []
    # without the flag the same read is reachable without a wait
    assert len(_check(body.replace("\ts_mov_b64 s[8:9], -1\n", ""))) == 1


def test_scalar_read_from_in_flight_register_must_stay_unused():
    body = f"""
{_asm("global_atomic_add v4, v[0:1], v2, off sc0")}
\tv_readfirstlane_b32 s6, v4
\ts_mov_b32 s7, s6
\ts_endpgm
"""
    assert _check(body) == []
    used = body.replace("\ts_endpgm", "\ts_cmp_ge_i32 s7, 3\n\ts_endpgm")
    assert len(_check(used)) == 1


def test_carry_out_of_a_vop3b_instruction_is_a_definition():
    # v_mad_i64_i32 writes its second operand (the carry-out): a poisoned scalar there is overwritten,
    # not used; its scalar sources are still uses
    body = f"""
{_asm("global_atomic_add v4, v[0:1], v2, off sc0")}
\tv_readfirstlane_b32 s6, v4
\tv_mad_i64_i32 v[10:11], s[6:7], v1, s8, v[12:13]
\ts_cmp_ge_i32 s6, 3
\ts_endpgm
"""
    assert _check(body) == []
    as_source = body.replace("v_mad_i64_i32 v[10:11], s[6:7], v1, s8,", "v_mad_i64_i32 v[10:11], s[2:3], v1, s6,")
    assert len(_check(as_source)) == 2      # the mad and the compare both read s6


def test_load_into_lds_has_no_register_destination():
    # global_load_lds_dwordx4 reads its address registers and writes LDS only: reusing the address
    # registers afterwards is not a use of in-flight data, but it still counts towards vmcnt
    body = f"""
{_asm("global_load_dwordx4 v[4:7], v[0:1], off")}
{_asm("s_mov_b32 m0, s2")}
{_asm("global_load_lds_dwordx4 v[8:9], off")}
\tv_mov_b32_e32 v8, 0
{_asm("s_waitcnt vmcnt(1)")}
\tv_mov_b32_e32 v20, v4
\ts_endpgm
"""
    assert _check(body) == []
    too_early = body.replace("vmcnt(1)", "vmcnt(2)")
    assert len(_check(too_early)) == 1


def test_accumulation_registers_are_tracked():
    body = f"""
{_asm("global_atomic_add a4, v[0:1], v2, off sc0")}
\tv_accvgpr_read_b32 v8, a4
\ts_endpgm
"""
    assert len(_check(body)) == 1
    waited = body.replace("\tv_accvgpr_read_b32", _asm("s_waitcnt vmcnt(0)") + "\n\tv_accvgpr_read_b32")
    assert _check(waited) == []
    # a4 and v4 are different registers
    assert _check(body.replace("v_accvgpr_read_b32 v8, a4", "v_mov_b32_e32 v8, v4")) == []


def test_branches_inside_inline_assembly_are_followed():
    # one asm statement choosing between two load forms: both paths load v[4:7], one instruction each
    two_paths = """
;;#ASMSTART
\ts_cmp_eq_u32 s6, 0
\ts_cbranch_scc1 1f
\tglobal_load_dwordx4 v[4:7], v[0:1], off
\ts_branch 2f
1:
\tglobal_load_dwordx4 v[4:7], v[0:1], off nt
2:
;;#ASMEND
{wait}
\tv_mov_b32_e32 v20, v4
\ts_endpgm
"""
    assert _check(two_paths.format(wait=_asm("s_waitcnt vmcnt(0)"))) == []
    assert len(_check(two_paths.format(wait=""))) == 1
    # a path that loads nothing more: the wait count that suffices on the other path is then too loose
    uneven = """
{load}
;;#ASMSTART
\ts_cmp_eq_u32 s6, 0
\ts_cbranch_scc1 1f
\tglobal_load_dwordx4 v[8:11], v[0:1], off
1:
;;#ASMEND
{wait}
\tv_mov_b32_e32 v20, v4
\ts_endpgm
""".format(load=_asm("global_load_dwordx4 v[4:7], v[0:1], off"), wait=_asm("s_waitcnt vmcnt(1)"))
    assert len(_check(uneven)) == 1


def test_built_decode_kernels_pass():
    path = os.path.join(ROOT, "paged_kv_cache_53_amd", "_build", "decode.s")
    if not os.path.exists(path):
        pytest.skip("library not built here")
    res = V.check_file(path)
    assert res, "no decode kernels found in the assembly"
    assert {k: v for k, v in res.items() if v} == {}

"""The hand-placed waits after inline-assembly loads, checked on the AMD GPU
assembly of this repository's own build (the checked_build fixture: the
library's device flags; tests/asm_waits.py explains the model), and the
kernels that issue such loads use no scratch memory."""
import os
from concurrent.futures import ProcessPoolExecutor

import pytest

from tests import asm_waits as A

FAMILIES = ("decode_mfma", "decode_mfma_coop", "dense_mfma", "dense_bwd_dq", "dense_bwd_dkdv")


@pytest.fixture(scope="module")
def functions(checked_build):
    _, asm = checked_build
    with open(asm) as f:
        funcs = A.parse(f.read())
    return A.asm_load_functions(funcs)


def _check(f):
    return f.name, A.check_function(f, max_states=4096)


def test_every_family_is_checked(functions):
    names = [f.name for f in functions]
    for fam in FAMILIES:
        tag = f"{len(fam)}{fam}I"  # Itanium-mangled name of the template
        assert any(tag in n for n in names), fam
    assert len(functions) >= 100


def test_no_register_of_an_inline_asm_load_is_touched_before_its_wait(functions):
    with ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_check, functions, chunksize=4))
    bad = [(n, v) for n, v in results if v]
    assert not bad, "\n".join(f"{n}:\n  " + "\n  ".join(v[:3]) for n, v in bad[:5])


def test_kernels_with_inline_asm_loads_use_no_scratch(functions):
    bad = [f.name for f in functions if f.scratch != 0]
    assert not bad, bad[:5]


def test_checker_catches_a_read_before_the_wait():
    # planted mistakes in a hand-written function: a copy of the Q registers
    # before any wait, and a read of a transposed-read result before an
    # lgkmcnt wait covers it (one younger LDS read, lgkmcnt(2) waited: both may
    # still be outstanding; lgkmcnt(1) would cover it)
    text = """
kern:
	;;#ASMSTART
	global_load_dwordx4 v[2:5], v1, s[4:5] offset:0
	;;#ASMEND
	v_mov_b32_e32 v10, v3
	s_waitcnt vmcnt(0)
	;;#ASMSTART
	ds_read_b64_tr_b16 v[20:21], v30
	;;#ASMEND
	ds_read_b128 v[40:43], v31
	s_waitcnt lgkmcnt(2)
	v_mov_b32_e32 v11, v20
	s_endpgm
.Lfunc_end0:
; ScratchSize: 0
"""
    (f,) = A.parse(text)
    v = A.check_function(f)
    assert len(v) == 2 and "v3" in v[0] and "v20" in v[1], v
    good = text.replace("\tv_mov_b32_e32 v10, v3\n", "").replace("lgkmcnt(2)", "lgkmcnt(1)")
    (f,) = A.parse(good)
    assert A.check_function(f) == []


def test_checker_follows_flag_routed_branches():
    # the wait is chosen through a flag register: the path that skips it is
    # taken only when the flag says the other wait ran
    text = """
kern:
	;;#ASMSTART
	global_load_dwordx4 v[2:5], v1, s[4:5] offset:0
	;;#ASMEND
	s_cmp_lt_i32 s10, 2
	s_mov_b64 s[16:17], -1
	s_cbranch_scc0 .LBB0_2
	s_waitcnt vmcnt(4)
	s_mov_b64 s[16:17], 0
.LBB0_2:
	s_andn2_b64 vcc, exec, s[16:17]
	s_cbranch_vccnz .LBB0_4
	s_waitcnt vmcnt(0)
.LBB0_4:
	v_mov_b32_e32 v10, v3
	s_endpgm
.Lfunc_end0:
; ScratchSize: 0
"""
    (f,) = A.parse(text)
    assert A.check_function(f) == []
    # without the second wait, the s10 >= 2 path reaches the read unwaited
    (f,) = A.parse(text.replace("\ts_waitcnt vmcnt(0)\n", ""))
    assert A.check_function(f)

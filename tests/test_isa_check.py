"""The build's scans of the asm-MFMA kernels: accesses inside an MFMA's
latency window (a CDNA XDL op of N passes needs N + 3 wait states before a
VALU or memory access of its result registers), uses of M0, and accesses of
the registers of a load still in flight."""
import importlib.util
import os

import pytest

_HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location(
    "isa_check", os.path.join(_HERE, "..", "implicit_gemm_conv_nhwc_amd", "isa_check.py"))
isa_check = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(isa_check)


def _kernel(body):
    return "k:\n" + "\n".join("\t" + l for l in body) + "\n.Lfunc_end0:\n"


MFMA = "v_mfma_f32_32x32x16_f16 v[0:15], a[0:3], v[20:23], v[0:15]"


def test_copy_right_after_mfma_is_found():
    bad = isa_check.scan(_kernel([MFMA, "v_mov_b64_e32 v[40:41], v[14:15]"]))
    assert len(bad) == 1 and "v_mov_b64" in bad[0][2]


def test_padding_clears_it():
    assert isa_check.scan(_kernel([MFMA, "s_nop 7", "s_nop 7", "v_mov_b64_e32 v[40:41], v[14:15]"])) == []


def test_eleven_wait_states_are_not_enough_here():
    # 8 passes + 3 + the one extra the scan keeps
    assert len(isa_check.scan(_kernel([MFMA, "s_nop 7", "s_nop 2", "v_mov_b32_e32 v40, v3"]))) == 1
    assert isa_check.scan(_kernel([MFMA, "s_nop 7", "s_nop 3", "v_mov_b32_e32 v40, v3"])) == []


def test_dependent_accumulation_is_exempt_but_b_operand_is_not():
    nxt_c = "v_mfma_f32_32x32x16_f16 v[0:15], a[4:7], v[24:27], v[0:15]"
    assert isa_check.scan(_kernel([MFMA, nxt_c])) == []
    nxt_b = "v_mfma_f32_32x32x16_f16 v[32:47], a[4:7], v[12:15], v[32:47]"
    assert len(isa_check.scan(_kernel([MFMA, nxt_b]))) == 1


def test_overwriting_srcc_or_result_in_flight_is_found():
    assert len(isa_check.scan(_kernel([MFMA, "v_mov_b32_e32 v5, 0"]))) == 1
    # a store reads its data: a result register as store data is a read
    assert len(isa_check.scan(_kernel([MFMA, "buffer_store_dwordx4 v[0:3], v30, s[4:7], 0 offen"]))) == 1
    # unrelated registers are fine
    assert isa_check.scan(_kernel([MFMA, "v_mov_b32_e32 v50, v51", "ds_read_b128 v[60:63], v52"])) == []


@pytest.mark.parametrize("op,passes", [("v_mfma_f32_32x32x16_f16", 8), ("v_mfma_f32_16x16x32_f16", 4)])
def test_window_follows_the_pass_count(op, passes):
    mf = "%s v[0:15], a[0:3], v[20:23], v[0:15]" % op
    pad = ["s_nop 0"] * (passes + 3)
    assert len(isa_check.scan(_kernel([mf] + pad + ["v_mov_b32_e32 v40, v0"]))) == 1
    assert isa_check.scan(_kernel([mf] + pad + ["s_nop 0", "v_mov_b32_e32 v40, v0"])) == []


def test_m0_rule():
    ok = _kernel(["s_mov_b32 m0, s4", "s_nop 0", "buffer_load_dwordx4 v1, s[8:11], s6 offen lds", "s_mov_b32 s5, m0"])
    assert isa_check.scan_m0(ok) == []
    assert len(isa_check.scan_m0(_kernel(["v_readlane_b32 s0, v1, m0"]))) == 1
    assert len(isa_check.scan_m0(_kernel(["s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)"]))) == 1
    assert len(isa_check.scan_m0(_kernel(["s_movrels_b32 s0, s1"]))) == 1


LOAD = "buffer_load_dwordx4 v[2:5], v14, s[28:31], 0 offen"


def test_copy_of_a_load_in_flight_is_found():
    """The compiler takes an asm load's registers for written at issue: a
    copy placed before the kernel's own wait reads data not yet landed."""
    bad = _kernel([LOAD, "buffer_load_dwordx4 v[6:9], v14, s[28:31], 0 offen", "v_mov_b64_e32 v[40:41], v[4:5]",
                   "s_waitcnt vmcnt(0)"])
    f = isa_check.scan_vmem(bad)
    assert len(f) == 1 and f[0][1] == LOAD


def test_wait_retires_all_but_the_last_n():
    later = "buffer_load_dwordx4 v[6:9], v14, s[28:31], 0 offen"
    # vmcnt(1): the first load has landed, the second may not have
    ok = _kernel([LOAD, later, "s_waitcnt vmcnt(1)", "v_mov_b64_e32 v[40:41], v[4:5]"])
    assert isa_check.scan_vmem(ok) == []
    bad = _kernel([LOAD, later, "s_waitcnt vmcnt(1)", "v_mov_b64_e32 v[40:41], v[8:9]"])
    assert len(isa_check.scan_vmem(bad)) == 1
    # stores and loads into LDS count in vmcnt but write no registers
    ok2 = _kernel([LOAD, "buffer_store_dwordx4 v[10:13], v14, s[28:31], 0 offen",
                   "buffer_load_dwordx4 v1, s[8:11], s6 offen lds", "s_waitcnt vmcnt(2)", "v_add_f32_e32 v40, v2, v3"])
    assert isa_check.scan_vmem(ok2) == []
    # a second load into the same registers before the first has landed
    assert len(isa_check.scan_vmem(_kernel([LOAD, LOAD]))) == 1


def test_a_label_starts_afresh():
    """Code reached by a branch has its own waits on every path."""
    ok = _kernel([LOAD, "s_cbranch_execz .LBB0_2", ".LBB0_2:", "v_mov_b32_e32 v2, 0"])
    assert isa_check.scan_vmem(ok) == []

"""The build's assembly check for vector writes ahead of an exec-mask restore (CPU only): it must
flag the miscompilation the SIC super-block kernel once carried and leave the ordinary lowerings
of if, if/else and loops alone."""
from rate_allocated_weight_amd import build

BAD = """
_Zkernel:
	v_cmp_lt_i32_e32 vcc, 0, v249
	s_and_b64 s[8:9], s[2:3], vcc
	s_and_saveexec_b64 s[2:3], s[8:9]
	s_cbranch_execz .LBB16_72
	global_load_dwordx2 v[20:21], v[20:21], off
	s_waitcnt vmcnt(0)
.LBB16_72:
	v_accvgpr_write_b32 a3, v100
	v_mov_b32_e32 v133, 0x26424
	s_or_b64 exec, exec, s[2:3]
	ds_read_b32 v48, v133
	s_endpgm
"""

GOOD_IF = """
_Zkernel:
	s_and_saveexec_b64 s[2:3], s[8:9]
	s_cbranch_execz .LBB0_2
	v_mov_b32_e32 v1, 0
	ds_write_b32 v0, v1
.LBB0_2:
	s_or_b64 exec, exec, s[2:3]
	v_mov_b32_e32 v133, 0x26424
	s_endpgm
"""

GOOD_IF_ELSE = """
_Zkernel:
	s_and_saveexec_b64 s[2:3], vcc
	s_xor_b64 s[2:3], exec, s[2:3]
	s_cbranch_execz .LBB0_2
	v_mov_b32_e32 v1, 1
.LBB0_2:
	s_andn2_saveexec_b64 s[2:3], s[2:3]
	v_mov_b32_e32 v1, 2
	s_or_b64 exec, exec, s[2:3]
	s_endpgm
"""


def test_flags_writes_before_exec_restore():
    bad = build.exec_join_writes(BAD)
    assert len(bad) == 1
    func, line, label, writes = bad[0]
    assert func == "_Zkernel" and label == ".LBB16_72"
    assert writes == ["v_accvgpr_write_b32 a3, v100", "v_mov_b32_e32 v133, 0x26424"]


def test_ordinary_lowerings_pass():
    assert build.exec_join_writes(GOOD_IF) == []
    assert build.exec_join_writes(GOOD_IF_ELSE) == []

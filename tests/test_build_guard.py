"""The build's check that compiler-generated device code never uses m0 (CPU).

The tile-copy helper writes m0 inside inline assembly; the build scans the
device assembly of every source and fails if an instruction outside the
inline-assembly blocks names m0 (exact_tiled_attention_12_amd/build.py).
"""

from exact_tiled_attention_12_amd.build import compiler_m0_uses

CLEAN = """
	v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
	; ;;#ASMSTART
	s_mov_b32 m0, s4
	s_nop 0
	buffer_load_dwordx4 v1, s[8:11], 0 offen lds
	; ;;#ASMEND
	s_waitcnt vmcnt(3)   ; m0 mentioned only in a comment
"""


def test_clean_assembly_passes():
    assert compiler_m0_uses(CLEAN) == []


def test_compiler_m0_use_is_caught():
    dirty = CLEAN + "\ts_mov_b32 m0, -1\n\tds_read_b32 v0, v1\n"
    bad = compiler_m0_uses(dirty)
    assert len(bad) == 1 and "s_mov_b32 m0, -1" in bad[0][1]
    # also inside an instruction's operand list, and after an unterminated block closes
    assert compiler_m0_uses("\tv_movrels_b32 v0, v1 ; uses m0\n\ts_add_u32 m0, m0, 1\n") == [(2, "s_add_u32 m0, m0, 1")]

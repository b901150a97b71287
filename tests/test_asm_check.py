"""The build-time check of inline-assembly MFMAs (exact_io_aware_10_amd/asm_check.py)
flags a result read inside the MFMA's write window and accepts fenced code."""
from exact_io_aware_10_amd import asm_check

MFMA = """;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]
;;#ASMEND
"""


def test_early_valu_read_is_flagged():
    assert len(asm_check.check(MFMA + "\tv_add_f32_e32 v30, v1, v2\n")) == 1


def test_early_copy_of_agpr_result_is_flagged():
    text = MFMA.replace("v[0:15]", "a[0:15]") + "\tv_accvgpr_mov_b32 a200, a15\n"
    assert len(asm_check.check(text)) == 1


def test_fenced_read_is_accepted():
    assert asm_check.check(MFMA + "\ts_nop 15\n\tv_add_f32_e32 v30, v1, v2\n") == []


def test_unrelated_registers_and_chains_are_accepted():
    text = MFMA + MFMA + "\tv_add_f32_e32 v30, v40, v41\n"
    assert asm_check.check(text) == []


def test_compiler_mfma_is_not_checked():
    text = "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]\n\tv_add_f32_e32 v30, v1, v2\n"
    assert asm_check.check(text) == []


MFMA_C = """;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[40:55]
;;#ASMEND
"""


def test_early_write_of_srcc_is_flagged():
    # A VALU write or an LDS load into the accumulator input while it is read.
    assert len(asm_check.check(MFMA_C + "\tv_xor_b32_e32 v52, 64, v60\n")) == 1
    assert len(asm_check.check(MFMA_C + "\tds_read_b128 v[40:43], v60\n")) == 1


def test_reads_of_srcc_and_fenced_writes_are_accepted():
    assert asm_check.check(MFMA_C + "\tv_add_f32_e32 v60, v40, v41\n") == []
    assert asm_check.check(MFMA_C + "\ts_nop 15\n\tds_read_b128 v[40:43], v60\n") == []
    # An LDS-direct load names a VGPR as its address, not as a destination.
    assert asm_check.check(MFMA_C + "\tbuffer_load_dwordx4 v40, s[0:3], 0 offen lds\n") == []


def test_inline_asm_load_into_registers_is_flagged():
    # The compiler cannot wait for a load it does not know about (it copied
    # such a destination into AGPRs before the data arrived once).
    text = ";;#ASMSTART\n\tbuffer_load_dwordx4 v[4:7], v1, s[0:3], 0 offen\n;;#ASMEND\n"
    assert len(asm_check.check(text)) == 1
    # The same load emitted by the compiler, and an inline-asm LDS-direct load, pass.
    assert asm_check.check("\tbuffer_load_dwordx4 v[4:7], v1, s[0:3], 0 offen\n") == []
    assert asm_check.check(";;#ASMSTART\n\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds\n;;#ASMEND\n") == []

"""The device code has no wide buffer store whose data registers a VALU write
overtakes (gpt_pretraining_step_bf16_amd.isa_check): first the scanner on
hand-written assembly, then every csrc/*.hip file compiled for gfx950 with
the library's flags (CPU only: hipcc cross-compiles)."""
import os
import shutil

import pytest

from gpt_pretraining_step_bf16_amd import build, isa_check

HAZARD = """
kern:
\tbuffer_store_dwordx4 v[96:99], v206, s[8:11], s14 offen
\tv_cvt_f16_f32_e32 v96, v96
"""


def test_scanner_flags_a_valu_write_right_behind_a_wide_store():
    hits = isa_check.scan_asm(HAZARD)
    assert len(hits) == 1 and hits[0][0] == "kern"


@pytest.mark.parametrize("text", [
    # two wait states written out
    HAZARD.replace("offen\n", "offen\n\ts_nop 1\n"),
    # constant soffset: the compiler's own hazard handling applies
    HAZARD.replace("s14 offen", "0 offen"),
    # an 8-byte store reads its data in time
    HAZARD.replace("buffer_store_dwordx4 v[96:99]", "buffer_store_dwordx2 v[96:97]"),
    # the VALU writes another register
    HAZARD.replace("v_cvt_f16_f32_e32 v96, v96", "v_cvt_f16_f32_e32 v100, v96"),
    # two other instructions in between
    HAZARD.replace("offen\n", "offen\n\ts_mul_i32 s3, s46, 40\n\tv_mov_b32 v1, v2\n"),
])
def test_scanner_accepts_safe_sequences(text):
    assert isa_check.scan_asm(text) == []


def test_scanner_sees_every_data_register():
    text = HAZARD.replace("v_cvt_f16_f32_e32 v96, v96", "v_mul_f32_e32 v99, s3, v0")
    assert len(isa_check.scan_asm(text)) == 1


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
@pytest.mark.timeout(900)
def test_library_device_code_has_no_unguarded_wide_store():
    res = isa_check.check_sources()
    assert res, "no sources compiled"
    bad = {name: hits[:3] for name, hits in res.items() if hits}
    assert not bad, bad

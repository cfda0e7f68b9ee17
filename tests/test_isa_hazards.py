"""The device assembly of every kernel source has no MFMA result read before
the wait states that the compiler itself pads such reads with in straight-line
code (mamba_ssd_selective_amd.isa_check).  The checker is first pinned on
small hand-written fragments: a store at the head of a block that a branch
reaches straight from the MFMA is caught; padding, a rewrite of the register
and an intervening MFMA's passes clear it."""
import os
import shutil

import pytest

from mamba_ssd_selective_amd import _build, isa_check


def _fn(body):
    return "_ZN3ssd4testEv:\n" + "\n".join("\t" + l if not l.endswith(":") else l
                                          for l in body) + "\n.Lfunc_end0:\n"


MFMA = "v_mfma_f32_16x16x4_f32 v[6:9], v31, v13, v[6:9]"


def test_flags_store_reached_by_branch():
    asm = _fn([MFMA, "s_cbranch_vccnz .LBB0_2", "s_nop 7", "s_nop 7", ".LBB0_2:",
               "global_store_dwordx4 v1, v[6:9], s[2:3]", "s_endpgm"])
    found = isa_check.check_asm(asm)
    assert len(found) == 1 and "1 wait states" in found[0]


def test_flags_straight_line_read_too_close():
    asm = _fn([MFMA, "v_add_f32_e32 v40, v8, v41", "s_endpgm"])
    assert len(isa_check.check_asm(asm)) == 1


def test_padding_clears_it():
    # 10 wait states clear the fp32 MFMA; 9 do not
    asm = _fn([MFMA, "s_nop 7", "s_nop 1", "global_store_dwordx4 v1, v[6:9], s[2:3]", "s_endpgm"])
    assert isa_check.check_asm(asm) == []
    asm = _fn([MFMA, "s_nop 7", "s_nop 0", "global_store_dwordx4 v1, v[6:9], s[2:3]", "s_endpgm"])
    assert len(isa_check.check_asm(asm)) == 1


def test_rewrite_clears_it():
    asm = _fn([MFMA, "v_mov_b32_e32 v8, 0", "v_mov_b32_e32 v9, 0", "v_mov_b32_e32 v6, 0",
               "v_mov_b32_e32 v7, 0", "global_store_dwordx4 v1, v[6:9], s[2:3]", "s_endpgm"])
    assert isa_check.check_asm(asm) == []


def test_intervening_mfma_passes_count():
    bf = "v_mfma_f32_16x16x32_bf16 v[2:5], v[10:13], v[14:17], v[2:5]"
    other = "v_mfma_f32_16x16x32_bf16 v[20:23], v[10:13], v[14:17], v[20:23]"
    # two later MFMAs of 4 passes each: 8 wait states, what the bf16 MFMA needs
    assert isa_check.check_asm(_fn([bf, other, other, "v_mul_f32_e32 v2, v40, v2", "s_endpgm"])) == []
    assert len(isa_check.check_asm(_fn([bf, other, "v_mul_f32_e32 v2, v40, v2", "s_endpgm"]))) == 1


def test_dependent_mfma_chain_is_not_a_finding():
    asm = _fn([MFMA, "v_mfma_f32_16x16x4_f32 v[6:9], v32, v14, v[6:9]", "s_nop 7", "s_nop 1",
               "global_store_dwordx4 v1, v[6:9], s[2:3]", "s_endpgm"])
    assert isa_check.check_asm(asm) == []


def test_unknown_mfma_is_reported():
    asm = _fn(["v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], 0", "s_endpgm"])
    assert len(isa_check.check_asm(asm)) == 1


@pytest.mark.skipif(not (os.path.exists(_build.HIPCC) or shutil.which(_build.HIPCC)),
                    reason="hipcc not available")
def test_library_device_assembly(tmp_path):
    found = []
    for path in isa_check.device_asm(str(tmp_path)):
        with open(path) as f:
            found += ["%s: %s" % (os.path.basename(path), l) for l in isa_check.check_asm(f.read())]
    assert found == [], "\n".join(found)

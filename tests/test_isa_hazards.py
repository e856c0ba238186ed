"""Wait states after the dK/dV kernel's inline-assembly MFMAs (CPU only): the
checker that every build runs, pinned on small hand-written sequences, and
run on the assembly generated from the current sources."""
import os

import pytest

from document_masked_attention_amd import build, isa_check

SYM = "_ZN7docmask11dkdv_kernelILi128EEEvNS_9BwdParamsE"


def _fn(body):
    return f"\n{SYM}:\n" + "\n".join("\t" + line for line in body) + "\n.Lfunc_end0:\n"


MFMA = "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]"


def test_read_inside_the_window_is_reported():
    n, v = isa_check.check(_fn([MFMA, "s_nop 3", "v_add_f32_e32 v20, v1, v2", "s_endpgm"]), SYM)
    assert n == 1 and len(v) == 1 and "after 4 wait states" in v[0]


def test_twelve_wait_states_are_enough():
    n, v = isa_check.check(_fn([MFMA, "s_nop 7", "s_nop 3", "v_add_f32_e32 v20, v1, v2", "s_endpgm"]), SYM)
    assert n == 1 and v == []
    # 11 are not; a write counts like a read
    n, v = isa_check.check(_fn([MFMA, "s_nop 7", "s_nop 2", "v_mov_b32_e32 v15, 0", "s_endpgm"]), SYM)
    assert len(v) == 1


def test_every_branch_path_is_followed():
    asm = _fn([MFMA, "s_cbranch_scc1 .LBB0_2", "s_nop 7", "s_nop 7", ".LBB0_2:", "v_add_f32_e32 v20, v3, v2",
               "s_endpgm"])
    n, v = isa_check.check(asm, SYM)
    assert len(v) == 1 and "after 1 wait states" in v[0]


def test_accumulating_chain_and_agpr_destinations():
    # the next MFMA accumulating into the same tile continues the chain
    n, v = isa_check.check(_fn([MFMA, MFMA, "s_nop 7", "s_nop 3", "v_add_f32_e32 v20, v0, v1", "s_endpgm"]), SYM)
    assert n == 2 and v == []
    # ... one reading the tile as a multiplicand does not
    n, v = isa_check.check(_fn([MFMA, "v_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], a[0:3], v[32:47]", "s_endpgm"]),
                           SYM)
    assert len(v) == 1
    # MFMAs writing AGPRs are the compiler's own and are not checked
    n, v = isa_check.check(_fn(["v_mfma_f32_32x32x16_bf16 a[0:15], v[16:19], v[20:23], a[0:15]",
                                "v_add_f32_e32 v20, v1, v2", "s_endpgm"]), SYM)
    assert n == 0 and v == []


def test_generated_dkdv_kernels_respect_the_window():
    n = build.check_inline_mfma_wait_states()
    assert n >= 100          # every S / dP MFMA of both head sizes was found and checked

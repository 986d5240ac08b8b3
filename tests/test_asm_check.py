"""The checks of the library's machine code (dense_tiled_gemm_04_amd/asm_check.py): planted wait-state hazards
in small assembly texts are found, their fixed forms pass, the built library has none, and every kernel of the
built library uses the instructions its design names."""
import os

import pytest

from dense_tiled_gemm_04_amd import asm_check

HEAD = "_ZN2gk4testEv:\n"


def rules(text):
    return [h["rule"] for h in asm_check.hazards(HEAD + text)]


def test_valu_sgpr_write_then_copy_is_flagged():
    # the copy's scalar base written by readfirstlane one wait state before the load
    asm = """
        v_readfirstlane_b32 s38, v114
        v_readfirstlane_b32 s39, v115
        s_mov_b32 m0, s30
        s_nop 0
        global_load_lds_dwordx4 v106, s[38:39]
        s_endpgm
    """
    assert rules(asm) == ["sgpr->vmem"]
    assert asm_check.hazards(HEAD + asm)[0]["wait_states"] == 2  # s_mov + s_nop 0 after the s39 write


def test_five_wait_states_or_a_salu_writer_pass():
    ok_nops = """
        v_readfirstlane_b32 s38, v114
        v_readfirstlane_b32 s39, v115
        s_nop 4
        global_load_lds_dwordx4 v106, s[38:39]
        s_endpgm
    """
    ok_salu = """
        v_readfirstlane_b32 s8, v114
        v_readfirstlane_b32 s9, v115
        s_add_u32 s38, s8, s36
        s_addc_u32 s39, s9, s37
        global_load_lds_dwordx4 v106, s[38:39]
        s_endpgm
    """
    buffer = """
        v_readfirstlane_b32 s40, v1
        s_nop 0
        buffer_load_dwordx4 v2, s[40:43], 0 offen lds
        s_endpgm
    """
    assert rules(ok_nops) == []
    # s_add reads s8/s9, but the load reads s38/s39, last written by SALU
    assert rules(ok_salu) == []
    assert rules(buffer) == ["sgpr->vmem"]


def test_hazard_across_a_loop_back_edge():
    # the load at the loop head reads what the previous iteration's tail wrote
    asm = """
    .LBB0_1:
        global_load_lds_dwordx4 v106, s[38:39]
        s_add_u32 s2, s2, 1
        s_cmp_lg_u32 s2, 8
        v_readfirstlane_b32 s38, v7
        s_cbranch_scc1 .LBB0_1
        s_endpgm
    """
    assert rules(asm) == ["sgpr->vmem"]
    # the fall-through predecessor alone would have shown nothing: the label has no instruction above it
    asm_objdump = asm.replace(".LBB0_1:", "<L0>:").replace("s_cbranch_scc1 .LBB0_1", "s_cbranch_scc1 L0")
    assert rules(asm_objdump) == ["sgpr->vmem"]


def test_valu_write_then_mfma_source():
    bad = """
        v_mov_b32_e32 v12, v40
        v_mfma_f32_16x16x32_f16 a[0:3], v[10:13], v[14:17], a[0:3]
        s_endpgm
    """
    good = """
        v_mov_b32_e32 v12, v40
        s_nop 1
        v_mfma_f32_16x16x32_f16 a[0:3], v[10:13], v[14:17], a[0:3]
        s_endpgm
    """
    acc = """
        v_accvgpr_write_b32 a2, 0
        v_mfma_f32_16x16x32_f16 a[0:3], v[10:13], v[14:17], a[0:3]
        s_endpgm
    """
    chained = """
        v_mfma_f32_16x16x32_f16 a[0:3], v[10:13], v[14:17], a[0:3]
        v_mfma_f32_16x16x32_f16 a[0:3], v[18:21], v[14:17], a[0:3]
        s_endpgm
    """
    assert rules(bad) == ["valu->mfma"]
    assert rules(good) == []
    assert rules(acc) == ["valu->mfma"]
    assert rules(chained) == []


def test_built_library_has_no_hazard():
    from dense_tiled_gemm_04_amd import build

    if not os.path.exists(build.LIB_PATH):
        pytest.skip("library not built")
    try:
        n = asm_check.check_library(build.LIB_PATH)
    except FileNotFoundError as e:
        pytest.skip("LLVM tools missing: %s" % e)
    assert n > 1000


def test_disassembly_covers_every_unit():
    # the library links one offload bundle per translation unit; the check must read all of them, not the first
    from dense_tiled_gemm_04_amd import build

    if not os.path.exists(build.LIB_PATH):
        pytest.skip("library not built")
    try:
        text = asm_check.disassemble_library(build.LIB_PATH)
    except FileNotFoundError as e:
        pytest.skip("LLVM tools missing: %s" % e)
    names = [n for n, _ in asm_check._functions(text)]
    for unit_kernel in ("gemm_tile_pipe_kernel", "gemm_skinny_kernel", "flash_attn_fwd_pipe_kernel",
                        "softmax_reg_kernel", "vector_add_f32_kernel"):
        assert any(unit_kernel in n for n in names), unit_kernel


def test_kernels_use_the_intended_instructions():
    # The pages read the generated code for tensor-core operations, asynchronous copies and barriers.  Here every
    # kernel of the built library is checked for the gfx950 instructions of its design, decoded from its
    # template arguments: the MFMA shape, the copy form of its loader (LDS-DMA from global or buffer
    # addresses, or register staging written with ds_write_b128), LDS transpose reads exactly when B is
    # row-major, a barrier, and exponentials exactly in the GELU instantiations.
    from dense_tiled_gemm_04_amd import build

    if not os.path.exists(build.LIB_PATH):
        pytest.skip("library not built")
    try:
        text = asm_check.disassemble_library(build.LIB_PATH)
    except FileNotFoundError as e:
        pytest.skip("LLVM tools missing: %s" % e)
    seen = dict.fromkeys(("tile", "skinny", "attention", "softmax"), 0)
    for name, m in asm_check.instruction_markers(text).items():
        a = asm_check.template_ints(name)
        if "gemm_tile_pipe_kernel" in name:
            # BM BN BK WM WN STAGES GROUP_M EPI BSLOT DSTRIDE LOADER CSLOT WPE MF SPREAD BT
            seen["tile"] += 1
            epi, loader, mf, bt = a[7], a[10], a[13], a[15]
            assert m["v_mfma_f32_%s_f16" % ("16x16x32" if mf == 16 else "32x32x16")] > 0, name
            copy = {0: "global_load_lds_dwordx4", 1: "ds_write_b128", 2: "buffer_load_lds"}[loader]
            assert m[copy] > 0, name
            if loader != 1:
                assert m["ds_write_b128"] == 0, name          # the LDS-DMA loaders stage nothing through VGPRs
            assert (m["ds_read_b64_tr_b16"] > 0) == (bt == 0), name
            assert m["s_barrier"] > 0, name
            assert (m["v_exp_f32"] > 0) == (epi == 2), name
        elif "gemm_skinny_kernel" in name:
            # MB STAGES EPI BT KROT A16
            seen["skinny"] += 1
            epi, bt = a[2], a[3]
            assert m["v_mfma_f32_16x16x32_f16"] > 0 and m["buffer_load_lds"] > 0, name
            assert (m["ds_read_b64_tr_b16"] > 0) == (bt == 0), name
            assert (m["v_exp_f32"] > 0) == (epi == 2), name
        elif "flash_attn_fwd" in name:
            seen["attention"] += 1
            assert m["v_mfma_f32_32x32x16_f16"] > 0 and m["buffer_load_lds"] > 0, name
            assert m["ds_read_b64_tr_b16"] > 0 and m["v_exp_f32"] > 0 and m["s_barrier"] > 0, name
        elif "softmax" in name:
            seen["softmax"] += 1
            assert m["v_mfma_f32_16x16x32_f16"] == m["v_mfma_f32_32x32x16_f16"] == 0, name
            assert m["v_exp_f32"] > 0, name
    assert all(seen.values()), seen

"""The C ABI without a GPU: the library loads, exports every function that
include/rankmixer.h declares, and rejects bad arguments on the host before
anything is launched.  No call here reaches a kernel launch."""
import ctypes as C
import os
import re

import pytest

from rankmixer_token_mixing_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rankmixer.h")


@pytest.fixture(scope="module")
def lib():
    from rankmixer_token_mixing_amd.build import build, library_is_fresh
    if not library_is_fresh(bd.lib_path()):
        build()
    bd.check_fresh()
    return bd.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_six_calls():
    names = declared_functions()
    for n in ("rm_tokenize_padsplit", "rm_token_mix", "rm_pffn_fwd", "rm_block_fwd", "rm_moe_relu_fwd",
              "rm_model_fwd"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and the binding wraps the same set
    for name in declared_functions():
        assert name in bd._SIGNATURES, name


def test_status_strings_and_version(lib):
    assert lib.rm_status_string(0) == b"ok"
    assert lib.rm_status_string(3) == b"workspace too small"
    assert lib.rm_status_string(99) == b"unknown status"
    assert b"gfx950" in lib.rm_version()


A16 = 0x10000  # a 16-byte aligned stand-in address; never dereferenced


def err(lib):
    return lib.rm_last_error().decode()


def test_token_mix_argument_errors(lib):
    assert lib.rm_token_mix(None, A16, 4, 2, 8, bd.RM_BF16, None) == bd.RM_ERR_INVALID
    assert "NULL" in err(lib)
    assert lib.rm_token_mix(A16, A16 + 4096, 4, 3, 8, bd.RM_BF16, None) == bd.RM_ERR_UNSUPPORTED
    assert "divisible" in err(lib)
    assert lib.rm_token_mix(A16 + 2, A16 + 4096, 4, 2, 8, bd.RM_BF16, None) == bd.RM_ERR_INVALID
    assert "aligned" in err(lib)
    assert lib.rm_token_mix(A16, A16, 4, 2, 8, bd.RM_BF16, None) == bd.RM_ERR_INVALID
    assert "alias" in err(lib)
    assert lib.rm_token_mix(A16, A16 + 4096, -3, 2, 8, bd.RM_BF16, None) == bd.RM_ERR_INVALID
    assert lib.rm_token_mix(A16, A16 + 4096, 4, 2, 8, 7, None) == bd.RM_ERR_UNSUPPORTED


def test_tokenizer_argument_errors(lib):
    assert lib.rm_tokenize_padsplit(A16, 4, 5121, 16, 320, bd.RM_BF16, A16 * 2, None) == bd.RM_ERR_UNSUPPORTED
    assert "fit" in err(lib)
    assert lib.rm_tokenize_padsplit(None, 4, 5000, 16, 320, bd.RM_BF16, A16, None) == bd.RM_ERR_INVALID


def _pffn():
    return bd.PffnParams(A16, A16, A16, A16)


def test_pffn_workspace_and_shape_errors(lib):
    need = lib.rm_pffn_workspace_bytes(64, 4, 64, 128, bd.RM_F32)
    assert need >= 64 * 4 * 128 * 4
    p = _pffn()
    s, v, ws = A16 * 2, A16 * 3, A16 * 4
    assert lib.rm_pffn_fwd(s, C.byref(p), v, 64, 4, 64, 128, bd.RM_F32, ws, need - 1, None) == bd.RM_ERR_WORKSPACE
    assert "workspace" in err(lib)
    assert lib.rm_pffn_fwd(s, C.byref(p), v, 64, 4, 68, 128, bd.RM_F32, ws, need, None) == bd.RM_ERR_UNSUPPORTED
    assert lib.rm_pffn_fwd(s, C.byref(p), v, 64, 4, 64, 100, bd.RM_F32, ws, need, None) == bd.RM_ERR_UNSUPPORTED
    assert lib.rm_pffn_fwd(s, None, v, 64, 4, 64, 128, bd.RM_F32, ws, need, None) == bd.RM_ERR_INVALID
    p.b2 = None
    assert lib.rm_pffn_fwd(s, C.byref(p), v, 64, 4, 64, 128, bd.RM_F32, ws, need, None) == bd.RM_ERR_INVALID
    assert "b2" in err(lib)
    assert lib.rm_pffn_fwd(s, C.byref(_pffn()), s, 64, 4, 64, 128, bd.RM_F32, ws, need, None) == bd.RM_ERR_INVALID


def test_moe_shape_errors(lib):
    p = bd.MoeParams(A16, A16, A16, A16, A16, A16)
    need = lib.rm_moe_workspace_bytes(64, 4, 64, 8, 128, bd.RM_BF16)
    assert need > 0
    args = (A16 * 2, C.byref(p), A16 * 3, None, 64, 4, 64)
    assert lib.rm_moe_relu_fwd(*args, 0, 128, bd.RM_BF16, A16 * 4, need, None) == bd.RM_ERR_UNSUPPORTED
    assert lib.rm_moe_relu_fwd(*args, 33, 128, bd.RM_BF16, A16 * 4, need, None) == bd.RM_ERR_UNSUPPORTED
    assert lib.rm_moe_relu_fwd(*args, 8, 128, bd.RM_BF16, A16 * 4, 16, None) == bd.RM_ERR_WORKSPACE
    assert lib.rm_moe_relu_fwd(A16 * 2, C.byref(p), A16 * 3, A16 + 4, 64, 4, 64, 8, 128, bd.RM_BF16, A16 * 4, need,
                               None) == bd.RM_ERR_INVALID  # misaligned gates


def test_block_and_model_errors(lib):
    bp = bd.BlockParams()
    bp.kind = 5
    bp.ln1_g = bp.ln1_b = bp.ln2_g = bp.ln2_b = A16
    assert lib.rm_block_fwd(A16, C.byref(bp), A16 * 2, 8, 4, 64, 128, 0, bd.RM_BF16, A16 * 3, 1 << 30,
                            None) == bd.RM_ERR_UNSUPPORTED
    bp.kind = bd.RM_BLOCK_DENSE
    bp.pffn = _pffn()
    need = lib.rm_block_workspace_bytes(0, 8, 4, 64, 128, 0, bd.RM_BF16)
    assert lib.rm_block_fwd(A16, C.byref(bp), A16 * 2, 8, 4, 64, 128, 0, bd.RM_BF16, A16 * 3, need - 1,
                            None) == bd.RM_ERR_WORKSPACE
    bp.hidden = 128
    arr = (bd.BlockParams * 1)(bp)
    m = bd.ModelDesc(4, 64, bd.RM_BF16, 1, arr, 0, None, 0.0)
    need = lib.rm_model_workspace_bytes(C.byref(m), 8)
    assert need >= lib.rm_block_workspace_bytes(0, 8, 4, 64, 128, 0, bd.RM_BF16)
    assert lib.rm_model_fwd(C.byref(m), A16, None, None, A16 * 2, 8, A16 * 3, need, None) == bd.RM_ERR_INVALID
    assert "head_w" in err(lib)
    m.F = 300
    assert lib.rm_model_fwd(C.byref(m), A16, None, None, None, 8, A16 * 3, need, None) == bd.RM_ERR_UNSUPPORTED


def test_workspace_sizes_scale_with_the_problem(lib):
    small = lib.rm_block_workspace_bytes(0, 1024, 32, 1536, 6144, 0, bd.RM_BF16)
    # S, H and the W2 product rows, all bf16
    assert small >= 1024 * 32 * (1536 * 2 + 6144 * 2 + 1536 * 2)
    assert lib.rm_block_workspace_bytes(1, 2048, 16, 768, 1536, 8, bd.RM_BF16) > \
        lib.rm_block_workspace_bytes(1, 1024, 16, 768, 1536, 8, bd.RM_BF16)


def test_empty_batch_is_a_no_op(lib):
    # B = 0: arguments other than the data pointers are still checked
    assert lib.rm_token_mix(None, None, 0, 4, 64, bd.RM_BF16, None) == bd.RM_OK
    assert lib.rm_token_mix(None, None, 0, 3, 64, bd.RM_BF16, None) == bd.RM_ERR_UNSUPPORTED
    assert lib.rm_token_mix(None, None, -1, 4, 64, bd.RM_BF16, None) == bd.RM_ERR_INVALID
    assert lib.rm_tokenize_padsplit(None, 0, 5000, 16, 320, bd.RM_BF16, None, None) == bd.RM_OK
    assert lib.rm_pffn_fwd(None, None, None, 0, 4, 64, 128, bd.RM_BF16, None, 0, None) == bd.RM_OK
    assert lib.rm_moe_relu_fwd(None, None, None, None, 0, 4, 64, 8, 128, bd.RM_BF16, None, 0, None) == bd.RM_OK
    bp = bd.BlockParams()
    bp.kind = bd.RM_BLOCK_DENSE
    bp.ln1_g = bp.ln1_b = bp.ln2_g = bp.ln2_b = A16
    bp.pffn = _pffn()
    assert lib.rm_block_fwd(None, C.byref(bp), None, 0, 4, 64, 128, 0, bd.RM_BF16, None, 0, None) == bd.RM_OK
    bp.hidden = 128
    arr = (bd.BlockParams * 1)(bp)
    m = bd.ModelDesc(4, 64, bd.RM_BF16, 1, arr, 0, None, 0.0)
    assert lib.rm_model_fwd(C.byref(m), None, None, None, None, 0, None, 0, None) == bd.RM_OK


def test_width_limits(lib):
    # one [D] row per wavefront: 8192 wide with heads of 8*k is the limit
    need = lib.rm_block_workspace_bytes(0, 1, 16, 8192, 64, 0, bd.RM_BF16)
    bp = bd.BlockParams()
    bp.kind = bd.RM_BLOCK_DENSE
    bp.ln1_g = bp.ln1_b = bp.ln2_g = bp.ln2_b = A16
    bp.pffn = _pffn()
    assert lib.rm_block_fwd(A16, C.byref(bp), A16 * 2, 1, 16, 8200, 64, 0, bd.RM_BF16, A16 * 3, 1 << 40,
                            None) == bd.RM_ERR_UNSUPPORTED  # 8200 % 16 != 0
    assert lib.rm_block_fwd(A16, C.byref(bp), A16 * 2, 1, 16, 8192 * 2, 64, 0, bd.RM_BF16, A16 * 3, 1 << 40,
                            None) == bd.RM_ERR_UNSUPPORTED  # too wide
    assert "wider" in err(lib)
    p = bd.MoeParams(A16, A16, A16, A16, A16, A16)
    assert lib.rm_moe_relu_fwd(A16, C.byref(p), A16 * 2, None, 4, 256, 64, 32, 64, bd.RM_BF16, A16 * 3, 1 << 40,
                               None) == bd.RM_ERR_UNSUPPORTED  # T*E = 8192 lists
    # blocks with an MoE keep the 4096 limit of the MoE row kernels
    bp.kind = bd.RM_BLOCK_MOE
    bp.moe = p
    assert lib.rm_block_fwd(A16, C.byref(bp), A16 * 2, 1, 16, 8192, 64, 4, bd.RM_BF16, A16 * 3, 1 << 40,
                            None) == bd.RM_ERR_UNSUPPORTED
    assert "MoE" in err(lib)
    assert need > 0


def test_projection_tokenizer_errors(lib):
    p = bd.ProjParams(A16, A16)
    # bf16 with F % 4 == 0 reads the embedding in place: no workspace
    assert lib.rm_tokenize_project_workspace_bytes(64, 5000, 16, 320, bd.RM_BF16) == 0
    assert lib.rm_tokenize_project_workspace_bytes(64, 4999, 16, 320, bd.RM_BF16) >= 64 * 16 * 320 * 2
    need = lib.rm_tokenize_project_workspace_bytes(64, 5000, 16, 320, bd.RM_F32)
    assert need >= 64 * 16 * 320 * 4
    args = (A16 * 2, C.byref(p), 64)
    f32 = (A16 * 3, A16 * 4, need, None)
    assert lib.rm_tokenize_project(*args, 5121, 16, 320, 320, bd.RM_F32, *f32) == bd.RM_ERR_UNSUPPORTED
    assert "fit" in err(lib)
    assert lib.rm_tokenize_project(*args, 5000, 16, 316, 320, bd.RM_F32, *f32) == bd.RM_ERR_UNSUPPORTED
    assert lib.rm_tokenize_project(*args, 5000, 16, 320, 324, bd.RM_F32, *f32) == bd.RM_ERR_UNSUPPORTED
    assert lib.rm_tokenize_project(*args, 5000, 16, 320, 320, bd.RM_F32, A16 * 3, A16 * 4, need - 1, None) \
        == bd.RM_ERR_WORKSPACE
    assert lib.rm_tokenize_project(*args, 5000, 16, 320, 320, bd.RM_F32, A16 * 3, None, need, None) \
        == bd.RM_ERR_INVALID
    assert lib.rm_tokenize_project(A16 * 2, None, 64, 5000, 16, 320, 320, bd.RM_F32, *f32) == bd.RM_ERR_INVALID
    p.b = None
    assert lib.rm_tokenize_project(*args, 5000, 16, 320, 320, bd.RM_F32, *f32) == bd.RM_ERR_INVALID
    assert "b is NULL" in err(lib)
    assert lib.rm_tokenize_project(None, None, 0, 5000, 16, 320, 320, bd.RM_BF16, None, None, 0, None) == bd.RM_OK


def _dense_bp():
    bp = bd.BlockParams()
    bp.kind = bd.RM_BLOCK_DENSE
    bp.ln1_g = bp.ln1_b = bp.ln2_g = bp.ln2_b = A16
    bp.pffn = _pffn()
    return bp


def test_training_entry_points_check_their_arguments(lib):
    bp = _dense_bp()
    sv = lib.rm_block_saved_bytes(64, 4, 64, 128, bd.RM_BF16)
    assert sv >= 64 * 4 * (64 + 128 + 64) * 2
    wsf = lib.rm_block_workspace_bytes(0, 64, 4, 64, 128, 0, bd.RM_BF16)
    wsb = lib.rm_block_bwd_workspace_bytes(64, 4, 64, 128, bd.RM_BF16)
    assert wsb > wsf
    fwd = lambda *a: lib.rm_block_fwd_train(A16, C.byref(bp), A16 * 2, A16 * 3, *a)
    assert fwd(sv - 1, 64, 4, 64, 128, bd.RM_BF16, A16 * 4, wsf, None) == bd.RM_ERR_WORKSPACE
    assert "saved" in err(lib)
    assert fwd(sv, 64, 4, 64, 128, bd.RM_BF16, A16 * 4, wsf - 1, None) == bd.RM_ERR_WORKSPACE
    assert fwd(sv, 64, 4, 8192, 128, bd.RM_BF16, A16 * 4, 1 << 40, None) == bd.RM_ERR_UNSUPPORTED  # D > 4096
    moe = bd.BlockParams()
    moe.kind = bd.RM_BLOCK_MOE
    moe.ln1_g = moe.ln1_b = moe.ln2_g = moe.ln2_b = A16
    moe.moe = bd.MoeParams(A16, A16, A16, A16, A16, A16)
    assert lib.rm_block_fwd_train(A16, C.byref(moe), A16 * 2, A16 * 3, sv, 64, 4, 64, 128, bd.RM_BF16, A16 * 4, wsf,
                                  None) == bd.RM_ERR_UNSUPPORTED
    assert "dense" in err(lib)
    g = bd.BlockGrads(*([A16 * 5] * 8))
    bwd = lambda dx, gg, ws_bytes: lib.rm_block_bwd(A16, C.byref(bp), A16 * 3, sv, A16 * 6, dx, gg, 64, 4, 64, 128,
                                                    bd.RM_BF16, A16 * 4, ws_bytes, None)
    assert bwd(A16 * 7, C.byref(g), wsb - 1) == bd.RM_ERR_WORKSPACE
    assert bwd(A16, C.byref(g), wsb) == bd.RM_ERR_INVALID  # dx aliases x
    assert "alias" in err(lib)
    assert bwd(A16 * 7, None, wsb) == bd.RM_ERR_INVALID
    g.b2 = None
    assert bwd(A16 * 7, C.byref(g), wsb) == bd.RM_ERR_INVALID
    assert "grads.b2" in err(lib)


def test_block_flags_and_variant_kinds(lib):
    bp = _dense_bp()
    bp.flags = 2  # not a known flag
    assert lib.rm_block_fwd(A16, C.byref(bp), A16 * 2, 8, 4, 64, 128, 0, bd.RM_BF16, A16 * 3, 1 << 30,
                            None) == bd.RM_ERR_UNSUPPORTED
    assert "flags" in err(lib)
    # the SwiGLU block needs room for the gate | up product as well
    assert lib.rm_block_workspace_bytes(bd.RM_BLOCK_SWIGLU, 64, 4, 64, 128, 0, bd.RM_BF16) > \
        lib.rm_block_workspace_bytes(bd.RM_BLOCK_DENSE, 64, 4, 64, 128, 0, bd.RM_BF16)
    # training covers the plain dense block only
    sv = lib.rm_block_saved_bytes(64, 4, 64, 128, bd.RM_BF16)
    for kind, flags in ((bd.RM_BLOCK_SWIGLU, 0), (bd.RM_BLOCK_DENSE, bd.RM_BLOCK_NO_MIX_NORM)):
        bp.kind, bp.flags = kind, flags
        assert lib.rm_block_fwd_train(A16, C.byref(bp), A16 * 2, A16 * 3, sv, 64, 4, 64, 128, bd.RM_BF16, A16 * 4,
                                      1 << 30, None) == bd.RM_ERR_UNSUPPORTED


def test_moe_training_entry_points_check_their_arguments(lib):
    # nothing here reaches a launch: every call fails its host-side checks
    moe = bd.BlockParams()
    moe.kind = bd.RM_BLOCK_MOE
    moe.ln1_g = moe.ln1_b = moe.ln2_g = moe.ln2_b = A16
    moe.moe = bd.MoeParams(A16, A16, A16, A16, A16, A16)
    B, T, D, He, E = 64, 4, 64, 64, 4
    sv = lib.rm_moe_saved_bytes(B, T, D, He, E, bd.RM_BF16)
    # S, U, Y, both gate sets (fp32), Z
    assert sv >= B * T * D * 2 + B * T * E * He * 2 + B * T * E * D * 2 + 2 * B * T * E * 4 + B * T * D * 2
    ws = lib.rm_moe_train_workspace_bytes(B, T, D, He, E, bd.RM_BF16)
    fwd = lambda p, l_reg, sb, wb, t=T, e=E: lib.rm_moe_block_fwd_train(
        A16, C.byref(p), A16 * 2, A16 * 3, A16 * 4, l_reg, A16 * 5, sb, B, t, D, He, e, bd.RM_BF16, A16 * 6, wb, None)
    assert fwd(moe, A16 * 7, sv - 1, ws) == bd.RM_ERR_WORKSPACE
    assert "saved" in err(lib)
    assert fwd(moe, A16 * 7, sv, ws - 1) == bd.RM_ERR_WORKSPACE
    assert fwd(moe, None, sv, ws) == bd.RM_ERR_INVALID
    assert "l_reg" in err(lib)
    assert fwd(moe, A16 * 7, 1 << 40, 1 << 40, t=2, e=3) == bd.RM_ERR_UNSUPPORTED  # T*E = 6
    assert "multiple of 8" in err(lib)
    dense = _dense_bp()
    assert fwd(dense, A16 * 7, sv, ws) == bd.RM_ERR_UNSUPPORTED
    moe.flags = bd.RM_BLOCK_NO_MIX_NORM
    assert fwd(moe, A16 * 7, sv, ws) == bd.RM_ERR_UNSUPPORTED
    moe.flags = 0
    assert lib.rm_moe_block_fwd_train(A16, C.byref(moe), None, A16 * 3, A16 * 4, A16 * 7, A16 * 5, sv, B, T, D, He,
                                      E, bd.RM_BF16, A16 * 6, ws, None) == bd.RM_ERR_INVALID
    assert "wr_train" in err(lib)
    g = bd.MoeGrads(*([A16 * 8] * 12))
    bwd = lambda dx, gg, wb: lib.rm_moe_block_bwd(A16, C.byref(moe), A16 * 3, A16 * 4, 0.5, A16 * 5, sv, A16 * 9, dx,
                                                  gg, B, T, D, He, E, bd.RM_BF16, A16 * 6, wb, None)
    assert bwd(A16 * 10, C.byref(g), ws - 1) == bd.RM_ERR_WORKSPACE
    assert bwd(A16 * 9, C.byref(g), ws) == bd.RM_ERR_INVALID  # dx aliases d_out
    assert "alias" in err(lib)
    assert bwd(A16 * 10, None, ws) == bd.RM_ERR_INVALID
    g.wr_infer = None
    assert bwd(A16 * 10, C.byref(g), ws) == bd.RM_ERR_INVALID
    assert "grads.wr_infer" in err(lib)


def test_epilogue_overlap_mode(lib):
    assert lib.rm_get_epilogue_overlap() == 0  # the default
    assert lib.rm_set_epilogue_overlap(2) == bd.RM_ERR_INVALID
    assert "0 or 1" in err(lib)
    try:
        assert lib.rm_set_epilogue_overlap(1) == 0
        assert lib.rm_get_epilogue_overlap() == 1
    finally:
        lib.rm_set_epilogue_overlap(0)
    assert lib.rm_get_epilogue_overlap() == 0


def test_generated_kstep_bodies_are_current():
    # the committed inline-asm k-steps are what their generator writes
    import importlib.util
    path = os.path.join(ROOT, "rankmixer_token_mixing_amd", "csrc", "gemm_defer_gen.py")
    spec = importlib.util.spec_from_file_location("gemm_defer_gen", path)
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    with open(os.path.join(ROOT, "rankmixer_token_mixing_amd", "csrc", "gemm_defer_kstep.inc")) as f:
        assert f.read() == gen.render()


def test_noalloc_route_refuses_more_than_its_scratch(lib):
    # the size check runs on the host before the device is touched
    assert lib.rm_moe_route_noalloc_max_scratch_bytes() == 16 << 20
    B, T, E = 40000, 16, 8  # 5.1 M (sample, token, expert) entries
    assert lib.rm_moe_route_noalloc_scratch_bytes(B, T, E) > lib.rm_moe_route_noalloc_max_scratch_bytes()
    assert lib.rm_moe_route_noalloc_scratch_bytes(2048, 16, 8) < 3 << 20
    st = lib.rm_moe_route_noalloc(A16, A16, A16, A16, A16, A16, B, T, 64, E, bd.RM_BF16, None)
    assert st == bd.RM_ERR_UNSUPPORTED
    assert "scratch" in err(lib)
    # and it checks its arguments like rm_moe_route
    assert lib.rm_moe_route_noalloc(None, A16, A16, A16, A16, A16, 4, 2, 64, 4, bd.RM_BF16, None) == bd.RM_ERR_INVALID
    assert lib.rm_moe_route_noalloc(A16, A16, A16, A16, A16, A16, 4, 2, 64, 33, bd.RM_BF16, None) == \
        bd.RM_ERR_UNSUPPORTED


def test_probe_entry_points_check_their_arguments(lib):
    RM_ERR_INVALID = 1
    assert lib.rm_probe_mfma_frag_bytes() == 64 * 16 * 64 * 16
    assert lib.rm_probe_kstep_slab_bytes() == 65536
    # flop counts follow the launch shapes: 32768 flop per MFMA, 64 MFMAs per
    # round and wave (MFMA loop), 32 per round and wave (k-step, 8 waves per block)
    waves = lib.rm_probe_mfma_out_floats() // 64
    assert lib.rm_probe_mfma_flop(10) == waves * 10 * 64 * 32768.0
    blocks = lib.rm_probe_kstep_out_floats() // 512
    assert lib.rm_probe_kstep_flop(10) == blocks * 8 * 10 * 32 * 32768.0
    assert lib.rm_probe_mfma_bf16(None, C.c_void_p(A16), 1, None) == RM_ERR_INVALID
    assert lib.rm_probe_kstep_bf16(None, C.c_void_p(A16), 1, None) == RM_ERR_INVALID
    assert "slab" in err(lib)
    assert lib.rm_probe_kstep_bf16(C.c_void_p(A16), C.c_void_p(A16), 0, None) == RM_ERR_INVALID
    assert "iters" in err(lib)
    assert lib.rm_probe_copy(C.c_void_p(A16), C.c_void_p(2 * A16), 24, None) == RM_ERR_INVALID
    assert lib.rm_probe_copy(C.c_void_p(A16), C.c_void_p(A16 + 16), 64, None) == RM_ERR_INVALID
    assert "overlap" in err(lib)

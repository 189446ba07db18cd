"""Host-side bounds audit of every launch, without a GPU.

The C entry points see only pointers, so a block sized with the wrong hidden
width or expert count reads past the end of its weights.  With the library's
audit switched on (rm_audit_enable), an entry point checks its arguments and
enqueues nothing; it records, for every launch it would make, each
caller-owned buffer that launch reads and how far.  These tests build real
host tensors, run the entry points in audit mode and check that every record
lies inside the tensor it starts in (or inside the workspace), and that each
parameter tensor is read by some launch.

The stacks include the one a randomized parity sweep faulted on, a SwiGLU
block, an MoE block with E = 4 (no Add & Norm after its mix) and an MoE block
with E = 8, each sized from its own descriptor."""
import ctypes as C
import os

import pytest
import torch

from rankmixer_token_mixing_amd import binding as bd

WS_BASE = 1 << 46  # stand-in workspace address; never dereferenced in audit mode


@pytest.fixture(scope="module")
def lib():
    from rankmixer_token_mixing_amd.build import build, library_is_fresh
    if not library_is_fresh(bd.lib_path()):
        build()
    bd.check_fresh()
    return bd.load()


def _block(kind, T, D, H, dtype, E=0, no_mix_norm=False, seed=0):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g, dtype=torch.float32)  # noqa: E731
    if kind == "moe":
        p = {"w1": r(T, E, H, D).to(dtype), "b1": r(T, E, H), "w2": r(T, E, D, H).to(dtype), "b2": r(T, E, D),
             "wr": r(T, E, D).to(dtype), "br": r(T, E)}
    else:
        n1 = 2 * H if kind == "swiglu" else H
        p = {"w1": r(T, n1, D).to(dtype), "b1": r(T, n1), "w2": r(T, D, H).to(dtype), "b2": r(T, D)}
    p.update({k: r(D) for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b")})
    if kind == "swiglu":
        p["swiglu"] = True
    if no_mix_norm:
        p["no_mix_norm"] = True
    return p


def _tensors(*dicts):
    out = []
    for d in dicts:
        out += [v for v in d.values() if isinstance(v, torch.Tensor)]
    return out


def _records(lib):
    out = []
    name = C.create_string_buffer(128)
    base, nbytes = C.c_uint64(), C.c_uint64()
    for i in range(lib.rm_audit_count()):
        assert lib.rm_audit_read(i, name, 128, C.byref(base), C.byref(nbytes)) == bd.RM_OK
        out.append((name.value.decode(), base.value, nbytes.value))
    return out


def _audited(lib, call):
    lib.rm_audit_enable(1)
    try:
        st = call()
        recs = _records(lib)
    finally:
        lib.rm_audit_enable(0)
    assert st == bd.RM_OK, lib.rm_last_error().decode()
    return recs


def _check_inside(recs, tensors, ws_bytes, must_read=()):
    """Every record inside the tensor its base falls in, or inside the
    workspace; every tensor of must_read read at least once."""
    spans = [(t.data_ptr(), t.data_ptr() + t.numel() * t.element_size(), t) for t in tensors]
    read = set()
    for name, base, nbytes in recs:
        hit = [s for s in spans if s[0] <= base < s[1]]
        if hit:
            lo, hi, t = hit[0]
            assert base + nbytes <= hi, f"{name} reads {base + nbytes - hi} bytes past the end of its buffer"
            read.add(id(t))
        else:
            assert WS_BASE <= base and base + nbytes <= WS_BASE + ws_bytes, f"{name} reads outside any buffer"
    for t in must_read:
        assert id(t) in read, "a parameter tensor is never read"


def _model_call(lib, model, x, B, ws):
    return lambda: lib.rm_model_fwd(C.byref(model.desc), x.data_ptr(), None, None, None, B, WS_BASE, ws, None)


def test_heterogeneous_moe_stack_reads_stay_inside_every_buffer(lib):
    # fp32, B=329, T=32, D=608 (heads of 19), hidden 24: SwiGLU, MoE E=4
    # without the Add & Norm after its mix, MoE E=8
    B, T, D, H = 329, 32, 608, 24
    blocks = [_block("swiglu", T, D, H, torch.float32, seed=1),
              _block("moe", T, D, H, torch.float32, E=4, no_mix_norm=True, seed=2),
              _block("moe", T, D, H, torch.float32, E=8, seed=3)]
    model = bd.Model(blocks, T, D, torch.float32)
    assert [(b.hidden, b.E) for b in model._arr] == [(24, 0), (24, 4), (24, 8)]
    x = torch.randn(B, T, D, dtype=torch.float32)
    ws = model.workspace_bytes(B)
    recs = _audited(lib, _model_call(lib, model, x, B, ws))
    params = _tensors(*blocks)
    _check_inside(recs, params + [x], ws, must_read=[t for t in params if t.dim() > 1] + [x])
    # the E = 4 block's router and experts are read as four experts per token
    wr4 = blocks[1]["wr"]
    ext = [n for name, base, n in recs if base == wr4.data_ptr()]
    assert ext and max(ext) == wr4.numel() * 4


def test_the_audit_catches_a_block_sized_with_another_blocks_expert_count(lib):
    # the descriptor of the E = 4 block claims E = 8 (what a model-wide expert
    # count taken from the last MoE block gives): the audit shows reads past
    # the end of its router and expert weights
    B, T, D, H = 64, 8, 64, 16
    blocks = [_block("moe", T, D, H, torch.bfloat16, E=4, seed=4), _block("moe", T, D, H, torch.bfloat16, E=8, seed=5)]
    model = bd.Model(blocks, T, D, torch.bfloat16)
    model._arr[0].E = 8
    x = torch.randn(B, T, D, dtype=torch.float32).to(torch.bfloat16)
    ws = model.workspace_bytes(B)
    recs = _audited(lib, _model_call(lib, model, x, B, ws))
    with pytest.raises(AssertionError, match="past the end"):
        _check_inside(recs, _tensors(*blocks) + [x], ws)


def test_dense_and_swiglu_blocks_of_different_widths_are_sized_per_block(lib):
    B, T, D = 100, 4, 64
    blocks = [_block("dense", T, D, 256, torch.bfloat16, seed=6), _block("swiglu", T, D, 48, torch.bfloat16, seed=7),
              _block("moe", T, D, 32, torch.bfloat16, E=3, seed=8), _block("dense", T, D, 128, torch.bfloat16, seed=9)]
    head = {"w": torch.randn(D, dtype=torch.float32), "c": 0.5}
    model = bd.Model(blocks, T, D, torch.bfloat16, head=head)
    x = torch.randn(B, T, D, dtype=torch.float32).to(torch.bfloat16)
    ws = model.workspace_bytes(B)
    recs = _audited(lib, _model_call(lib, model, x, B, ws))
    params = _tensors(*blocks)
    _check_inside(recs, params + [x, head["w"]], ws, must_read=[t for t in params if t.dim() > 1])
    # the workspace holds the largest block (the 256-wide dense one), not a
    # stack-wide maximum of every width
    one = lib.rm_block_workspace_bytes(bd.RM_BLOCK_DENSE, B, T, D, 256, 0, bd.RM_BF16)
    assert ws <= 2 * B * T * D * 2 + one + 2 * 256


def test_single_entry_points_read_inside_their_buffers(lib):
    B, T, D, H, E = 70, 4, 64, 96, 5
    dense = _block("dense", T, D, H, torch.bfloat16, seed=10)
    moe = _block("moe", T, D, H, torch.bfloat16, E=E, seed=11)
    x = torch.randn(B, T, D, dtype=torch.float32).to(torch.bfloat16)
    y = torch.empty_like(x)
    bf = bd.RM_BF16
    # rm_block_fwd, dense and MoE
    for blk, hid, e in ((dense, H, 0), (moe, H, E)):
        bp = bd._block_struct(blk)
        ws = lib.rm_block_workspace_bytes(bp.kind, B, T, D, hid, e, bf)
        recs = _audited(lib, lambda: lib.rm_block_fwd(x.data_ptr(), C.byref(bp), y.data_ptr(), B, T, D, hid, e, bf,
                                                      WS_BASE, ws, None))
        _check_inside(recs, _tensors(blk) + [x], ws, must_read=[x] + [t for t in _tensors(blk) if t.dim() > 1])
    # rm_pffn_fwd and rm_moe_relu_fwd
    ps = bd._pffn_struct(dense)
    ws = lib.rm_pffn_workspace_bytes(B, T, D, H, bf)
    recs = _audited(lib, lambda: lib.rm_pffn_fwd(x.data_ptr(), C.byref(ps), y.data_ptr(), B, T, D, H, bf, WS_BASE, ws,
                                                 None))
    _check_inside(recs, _tensors(dense) + [x], ws, must_read=[x, dense["w1"], dense["w2"], dense["b1"], dense["b2"]])
    ms = bd._moe_struct(moe)
    ws = lib.rm_moe_workspace_bytes(B, T, D, E, H, bf)
    recs = _audited(lib, lambda: lib.rm_moe_relu_fwd(x.data_ptr(), C.byref(ms), y.data_ptr(), None, B, T, D, E, H, bf,
                                                     WS_BASE, ws, None))
    _check_inside(recs, _tensors(moe) + [x], ws, must_read=[x, moe["w1"], moe["w2"], moe["wr"], moe["br"]])
    # the dense block's training forward and backward
    bp = bd._block_struct(dense)
    saved_n = lib.rm_block_saved_bytes(B, T, D, H, bf)
    ws = lib.rm_block_bwd_workspace_bytes(B, T, D, H, bf)
    grads = [torch.empty(1 << 20, dtype=torch.float32) for _ in range(8)]
    gs = bd.BlockGrads(*[g.data_ptr() for g in grads])
    d_out = torch.randn(B, T, D, dtype=torch.float32).to(torch.bfloat16)
    recs = _audited(lib, lambda: lib.rm_block_bwd(x.data_ptr(), C.byref(bp), WS_BASE, saved_n, d_out.data_ptr(),
                                                  y.data_ptr(), C.byref(gs), B, T, D, H, bf, WS_BASE, ws, None))
    _check_inside(recs, _tensors(dense) + [x, d_out], max(ws, saved_n), must_read=[x, d_out, dense["w1"], dense["w2"]])


def test_inconsistent_widths_are_refused_before_any_launch(lib):
    B, T, D = 16, 4, 64
    blk = _block("dense", T, D, 128, torch.bfloat16)
    x = torch.randn(B, T, D, dtype=torch.float32).to(torch.bfloat16)
    bp = bd._block_struct(blk)
    ws = lib.rm_block_workspace_bytes(0, B, T, D, 128, 0, bd.RM_BF16)
    # the descriptor says 128, the argument 256
    assert lib.rm_block_fwd(x.data_ptr(), C.byref(bp), WS_BASE + (1 << 30), B, T, D, 256, 0, bd.RM_BF16, WS_BASE,
                            1 << 40, None) == bd.RM_ERR_INVALID
    assert "hidden" in lib.rm_last_error().decode()
    # a model block without its width, an MoE block without experts, a dense
    # block with experts
    for hidden, kind, E in ((0, bd.RM_BLOCK_DENSE, 0), (128, bd.RM_BLOCK_MOE, 0), (128, bd.RM_BLOCK_DENSE, 4)):
        b = bd._block_struct(blk)
        b.hidden, b.kind, b.E = hidden, kind, E
        if kind == bd.RM_BLOCK_MOE:
            b.moe = bd.MoeParams(*([0x10000] * 6))
        arr = (bd.BlockParams * 1)(b)
        m = bd.ModelDesc(T, D, bd.RM_BF16, 1, arr, 0, None, 0.0)
        assert lib.rm_model_fwd(C.byref(m), x.data_ptr(), None, None, None, B, WS_BASE, 1 << 40,
                                None) == bd.RM_ERR_INVALID, (hidden, kind, E)
    del ws
    # the binding refuses tensors that do not match the widths they imply
    bad = dict(blk)
    bad["w2"] = torch.randn(T, D, 64).to(torch.bfloat16)
    with pytest.raises(ValueError, match="w2"):
        bd.Model([bad], T, D, torch.bfloat16)
    bad = dict(blk)
    bad["b1"] = torch.randn(T, 128).to(torch.bfloat16)
    with pytest.raises(ValueError, match="b1"):
        bd.Model([bad], T, D, torch.bfloat16)
    moe = _block("moe", T, D, 32, torch.bfloat16, E=4)
    moe["br"] = torch.randn(T, 8)
    with pytest.raises(ValueError, match="br"):
        bd.Model([blk, moe], T, D, torch.bfloat16)


def test_audit_mode_enqueues_nothing_and_is_off_by_default(lib):
    assert lib.rm_audit_count() == 0
    # with the audit off, a zero-sized batch still enqueues nothing and records nothing
    assert lib.rm_token_mix(None, None, 0, 4, 64, bd.RM_BF16, None) == bd.RM_OK
    assert lib.rm_audit_count() == 0
    name = C.create_string_buffer(16)
    a, b = C.c_uint64(), C.c_uint64()
    assert lib.rm_audit_read(0, name, 16, C.byref(a), C.byref(b)) == bd.RM_ERR_INVALID


@pytest.mark.parametrize("seed", __import__("tests.sweep_cases", fromlist=["SEEDS"]).SEEDS)
def test_sweep_cases_read_inside_their_buffers(lib, seed):
    # every stack of the GPU shape sweep, audited on host tensors first: each
    # launch it would make reads inside a caller buffer or the workspace
    from tests import sweep_cases as sc
    case = sc.draw(seed)
    dt = torch.bfloat16 if case.dtype == "bf16" else torch.float32
    blocks = bd.upload_blocks(case.blocks, device="cpu")
    head = None
    if case.head:
        head = {"w": torch.from_numpy(case.head_params["w"]), "c": case.head_params["c"]}
    model = bd.Model(blocks, case.T, case.D, dt, F=case.F, head=head)
    inp = bd.to_device(case.inp, device="cpu")
    x = torch.empty((case.B, case.T, case.D), dtype=dt)
    pooled = torch.empty((case.B, case.D), dtype=torch.float32) if case.head else None
    logit = torch.empty(case.B, dtype=torch.float32) if case.head else None
    ws = model.workspace_bytes(case.B)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    recs = _audited(lib, lambda: lib.rm_model_fwd(C.byref(model.desc), inp.data_ptr(), x.data_ptr(), ptr(pooled),
                                                  ptr(logit), case.B, WS_BASE, ws, None))
    params = _tensors(*blocks)
    outs = [t for t in (x, pooled, logit) if t is not None]
    _check_inside(recs, params + [inp] + outs + ([head["w"]] if head else []), ws,
                  must_read=[inp] + [t for t in params if t.dim() > 1])


@pytest.mark.parametrize("seed", __import__("tests.sweep_cases", fromlist=["TRAIN_SEEDS"]).TRAIN_SEEDS)
def test_training_sweep_cases_read_inside_their_buffers(lib, seed):
    # every block of the GPU training sweep, its training forward and
    # backward audited on host tensors (the saved tensors and the workspace
    # are stand-ins at WS_BASE)
    from tests import sweep_cases as sc
    case = sc.draw_train(seed)
    bf = bd.RM_BF16 if case.dtype == "bf16" else bd.RM_F32
    blk = bd.upload_blocks([case.blk], device="cpu")[0]
    x = bd.to_device(case.x, device="cpu")
    d_out = bd.to_device(case.d_out, device="cpu")
    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    B, T, D, H, E = case.B, case.T, case.D, case.H, case.E
    bp = bd._block_struct(blk)
    if case.kind == "dense":
        saved_n = lib.rm_block_saved_bytes(B, T, D, H, bf)
        ws = max(lib.rm_block_workspace_bytes(bd.RM_BLOCK_DENSE, B, T, D, H, 0, bf),
                 lib.rm_block_bwd_workspace_bytes(B, T, D, H, bf))
        shapes = [(T, H, D), (T, H), (T, D, H), (T, D), (D,), (D,), (D,), (D,)]
        grads = [torch.empty(s, dtype=torch.float32) for s in shapes]
        gs = bd.BlockGrads(*[t.data_ptr() for t in grads])
        fwd = lambda: lib.rm_block_fwd_train(x.data_ptr(), C.byref(bp), y.data_ptr(), WS_BASE, saved_n, B, T, D, H,  # noqa: E731
                                             bf, WS_BASE, ws, None)
        bwd = lambda: lib.rm_block_bwd(x.data_ptr(), C.byref(bp), WS_BASE, saved_n, d_out.data_ptr(), dx.data_ptr(),  # noqa: E731
                                       C.byref(gs), B, T, D, H, bf, WS_BASE, ws, None)
        extra = []
    else:
        saved_n = max(lib.rm_moe_saved_bytes(B, T, D, H, E, bf), 16)
        ws = lib.rm_moe_train_workspace_bytes(B, T, D, H, E, bf)
        l_reg = torch.empty(1, dtype=torch.float32)
        shapes = {"w1": (T, E, H, D), "b1": (T, E, H), "w2": (T, E, D, H), "b2": (T, E, D), "wr_train": (T, E, D),
                  "br_train": (T, E), "wr": (T, E, D), "br": (T, E), "ln1_g": (D,), "ln1_b": (D,), "ln2_g": (D,),
                  "ln2_b": (D,)}
        grads = [torch.empty(shapes[k], dtype=torch.float32) for k in bd.MOE_GRADS]
        gs = bd.MoeGrads(*[t.data_ptr() for t in grads])
        wrt, brt = blk["wr_train"], blk["br_train"]
        fwd = lambda: lib.rm_moe_block_fwd_train(x.data_ptr(), C.byref(bp), wrt.data_ptr(), brt.data_ptr(),  # noqa: E731
                                                 y.data_ptr(), l_reg.data_ptr(), WS_BASE, saved_n, B, T, D, H, E, bf,
                                                 WS_BASE, ws, None)
        bwd = lambda: lib.rm_moe_block_bwd(x.data_ptr(), C.byref(bp), wrt.data_ptr(), brt.data_ptr(), 0.37,  # noqa: E731
                                           WS_BASE, saved_n, d_out.data_ptr(), dx.data_ptr(), C.byref(gs), B, T, D, H,
                                           E, bf, WS_BASE, ws, None)
        extra = [l_reg]
    params = _tensors(blk)
    for call in (fwd, bwd):
        recs = _audited(lib, call)
        _check_inside(recs, params + [x, d_out, y, dx] + grads + extra, max(ws, saved_n))

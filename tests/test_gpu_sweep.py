"""Seeded random sweeps against the fp64 oracle.  First rm_model_fwd: stacks of
dense, SwiGLU and MoE blocks whose hidden widths and expert counts differ
from block to block, token counts from 1 to 40 (odd ones and non-powers of
two included), head widths from 1 to 64, ragged batches, gates mostly
closed, mostly open or about a quarter open, the Add & Norm after the mix
switched off now and then, and the pad-split tokenizer and the pooled logit
head on some of them (tests/sweep_cases.py draws them).

Before anything is launched, each case runs once through the library's
host-side audit with the real device buffers: every read that each launch
would make has to lie inside a caller buffer or the workspace.  Then the
training rows: one dense or MoE block's training forward and backward (below)."""
import ctypes as C

import numpy as np
import pytest
import torch

from oracle import rankmixer_oracle as orc
from tests import sweep_cases as sc
from tests.gpu_util import TOL, ensure_lib, host, note, rel_l2, rel_l2_rows

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def lib():
    return ensure_lib()


def _audit(lib, model, inp, outs, B, ws, tensors):
    from rankmixer_token_mixing_amd import binding as bd
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    lib.rm_audit_enable(1)
    try:
        st = lib.rm_model_fwd(C.byref(model.desc), inp.data_ptr(), ptr(outs["x"]), ptr(outs.get("pooled")),
                              ptr(outs.get("logit")), B, ws.data_ptr(), ws.numel(), None)
        name = C.create_string_buffer(128)
        base, nbytes = C.c_uint64(), C.c_uint64()
        recs = []
        for i in range(lib.rm_audit_count()):
            assert lib.rm_audit_read(i, name, 128, C.byref(base), C.byref(nbytes)) == bd.RM_OK
            recs.append((name.value.decode(), base.value, nbytes.value))
    finally:
        lib.rm_audit_enable(0)
    assert st == bd.RM_OK, lib.rm_last_error().decode()
    spans = [(t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()) for t in tensors + [ws]]
    for nm, b, n in recs:
        hit = [s for s in spans if s[0] <= b < s[1]]
        assert hit and b + n <= hit[0][1], f"{nm} would read outside its buffer"


@pytest.mark.parametrize("seed", sc.SEEDS)
def test_random_stack_matches_oracle(lib, seed):
    from rankmixer_token_mixing_amd import binding as bd
    case = sc.draw(seed)
    note(f"[gpu] sweep {case.describe()}")
    dt = DT[case.dtype]
    blocks = bd.upload_blocks(case.blocks)
    head = None
    if case.head:
        head = {"w": bd.to_device(case.head_params["w"]), "c": case.head_params["c"]}
    model = bd.Model(blocks, case.T, case.D, dt, F=case.F, head=head)
    inp = bd.to_device(case.inp)
    outs = {"x": torch.empty((case.B, case.T, case.D), dtype=dt, device="cuda")}
    if case.head:
        outs["pooled"] = torch.empty((case.B, case.D), dtype=torch.float32, device="cuda")
        outs["logit"] = torch.empty(case.B, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, model.workspace_bytes(case.B)), dtype=torch.uint8, device="cuda")
    tensors = [t for b in blocks for t in b.values() if isinstance(t, torch.Tensor)] + [inp] + list(outs.values())
    if head:
        tensors.append(head["w"])
    _audit(lib, model, inp, outs, case.B, ws, tensors)

    out = bd.rm_model_fwd(model, inp, want_x=True, want_pooled=case.head, out=outs)
    torch.cuda.synchronize()
    ref = orc.model_fwd(case.inp, case.blocks, case.T, case.D, case.dtype, case.F, case.head_params)
    tol = TOL[case.dtype]
    y = host(out["x"])
    assert np.isfinite(y).all()
    err = rel_l2_rows(y, ref["x"])
    assert err <= tol, f"{case.describe()}: max relative L2 {err:.3e}"
    if case.head:
        assert rel_l2_rows(host(out["pooled"]), ref["pooled"]) <= tol
        assert rel_l2(host(out["logit"]), ref["logit"]) <= tol


# ---------------------------------------------------------------------------
# training: a seeded random dense or MoE block (tests/sweep_cases.py
# draw_train), its training forward and backward against the fp64 oracle.
# Every case's launches were audited on host tensors of the same shapes
# (tests/test_model_bounds_cpu.py); weight and bias gradients are compared per
# token (per token and expert for the MoE block), the LayerNorm vectors whole.

GRADS = ("w1", "b1", "w2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")
GROUPS_DENSE = {"w1": 1, "b1": 1, "w2": 1, "b2": 1}
GROUPS_MOE = {"w1": 2, "b1": 2, "w2": 2, "b2": 2, "wr_train": 2, "wr": 2, "br_train": 1, "br": 1}
# a token's router-bias gradient is E numbers, each a sum over the batch of
# D-long dot products; such small groups vary in norm far more than groups
# of thousands of weights, and the bf16 rounding of the summands is about the
# same absolute size in every group, so they are judged with the floor at
# half the root-mean-square group norm (a wrong group still reads as an O(1)
# error).  Seen on a bf16 MoE block with T = 32, D = 768, E = 4: the whole
# br_train within 4.5e-3, its smallest token groups 2.2e-2 against the
# default quarter floor, the same case in fp32 within 1e-5 everywhere.
FLOOR = {"br_train": 0.5, "br": 0.5}
LAM = 0.37


@pytest.mark.parametrize("seed", sc.TRAIN_SEEDS)
def test_random_training_step_matches_oracle(lib, seed):
    from oracle import block_backward as bw
    from oracle import moe_training as mt
    from rankmixer_token_mixing_amd import binding as bd
    from tests.gpu_util import rel_l2_groups
    case = sc.draw_train(seed)
    note(f"[gpu] training sweep {case.describe()}")
    tol = TOL[case.dtype]
    dev = bd.upload_blocks([case.blk])[0]
    xd = bd.to_device(case.x)
    dod = bd.to_device(case.d_out)
    if case.kind == "dense":
        y, saved = bd.rm_block_fwd_train(xd, dev)
        dx, g = bd.rm_block_bwd(xd, dev, saved, dod)
        torch.cuda.synchronize()
        y_ref = orc.block_fwd(case.x, case.blk)
        ref = bw.block_bwd(case.x, case.blk, case.d_out)
        names, groups = GRADS, GROUPS_DENSE
    else:
        f = mt.dtsi_fwd_saved(case.x, case.blk)
        # both sides take the same gate decisions only away from the kink
        assert min(np.abs(f["Zt"]).min(), np.abs(f["Zi"]).min()) > 0.25
        y, l_reg, saved = bd.rm_moe_block_fwd_train(xd, dev)
        dx, g = bd.rm_moe_block_bwd(xd, dev, saved, dod, LAM)
        torch.cuda.synchronize()
        y_ref = f["out"]
        lr = float(host(l_reg)[0])
        assert abs(lr - f["l_reg"]) <= tol * max(abs(f["l_reg"]), 1e-30), (lr, f["l_reg"])
        ref = mt.dtsi_bwd(case.x, case.blk, case.d_out, LAM)
        names, groups = bd.MOE_GRADS, GROUPS_MOE
    assert rel_l2_rows(host(y), y_ref) <= tol
    e = rel_l2_rows(host(dx), ref["dX"])
    assert e <= tol, f"{case.describe()}: dX {e:.3e}"
    for k in names:
        if k in groups:
            e = rel_l2_groups(host(g[k]), ref[k], groups[k], floor=FLOOR.get(k, 0.25))
        else:
            e = rel_l2(host(g[k]), ref[k])
        assert e <= tol, f"{case.describe()}: {k} {e:.3e}"

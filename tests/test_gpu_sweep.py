"""A seeded random sweep of rm_model_fwd against the fp64 oracle: stacks of
dense, SwiGLU and MoE blocks whose hidden widths and expert counts differ
from block to block, token counts from 1 to 40 (odd ones and non-powers of
two included), head widths from 1 to 64, ragged batches, gates mostly
closed, mostly open or about a quarter open, the Add & Norm after the mix
switched off now and then, and the pad-split tokenizer and the pooled logit
head on some of them (tests/sweep_cases.py draws them).

Before anything is launched, each case runs once through the library's
host-side audit with the real device buffers: every read that each launch
would make has to lie inside a caller buffer or the workspace."""
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

"""GPU parity of the two training paths at the benchmarked sizes, in the
launch configuration the benchmark times (one call over the whole batch):
the dense block backward on block 0 of the ~1B-class workload (B=1024, T=32,
D=1536, hidden 6144) and the MoE block training step on block 0 of the MoE
workload (B=2048, T=16, D=768, 8 experts of 768 -> 1536 -> 768) with its
training router.  The oracle evaluates sampled samples: the forward output and
dX of a sample depend on that sample alone, so the sampled rows are exact.
Weight gradients sum over the whole batch; the oracle computes those of a few
sampled tokens exactly over the full batch (past the token mix, a token's
parameters see only that token's rows: LN2 normalises each row by itself),
and they are compared per token (per token and expert for the MoE block).

For dX of the MoE block, the ReLU gates decide which router terms exist; the
kernels take the decision in fp32 from bf16 S (rounding error of a router
pre-activation ~1e-3 here), the oracle in fp64, so dX is compared on sampled
samples whose pre-activations (fp64) all lie at least 0.01 from zero.  The
router gradients sum over every sample, so there the oracle takes the
decisions the kernels take (S rounded to bf16, the pre-activation in fp32),
and each decision within 1e-3 of the kink -- where the kernels' own
rounding could still flip it -- widens the bound by what flipping it
changes: |dG| |s_t| for the training router, lambda |s_t| for the
inference router."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import block_backward as bw
from oracle import moe_training as mt
from oracle import rankmixer_oracle as orc
from tests.gpu_util import TOL, ensure_lib, host, note, rel_l2_groups, rel_l2_rows

pytestmark = pytest.mark.gpu

KINK_MARGIN = 0.01
DECISION_BAND = 1e-3  # kernel-precision router pre-activations closer to zero may go either way
DENSE_TOKENS = (0, 17, 31)
MOE_TOKENS = (0, 11)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _workload(name):
    cfg = si.CONFIGS[name]
    inputs = si.make_inputs(si.scaled(cfg, L=1))
    d_out = si.make_inputs(si.scaled(cfg, L=0), seed=100 + si.SEEDS[name])["x"]
    return cfg, inputs, d_out


def test_dense_backward_full_size_sampled():
    from rankmixer_token_mixing_amd import binding as bd
    cfg, inputs, d_out_np = _workload("c3")
    blk_np = inputs["blocks"][0]
    blk = bd.upload_blocks([blk_np])[0]
    x = bd.to_device(inputs["x"])
    note(f"[gpu] rm_block_fwd_train + rm_block_bwd, {cfg.description}, block 0")
    y, saved = bd.rm_block_fwd_train(x, blk)
    dx, g = bd.rm_block_bwd(x, blk, saved, bd.to_device(d_out_np))
    torch.cuda.synchronize()
    rows = si.random_rows(cfg.B, 8)
    xr = inputs["x"][rows]
    assert rel_l2_rows(host(y)[rows], orc.block_fwd(xr, blk_np)) <= TOL["bf16"]
    ref = bw.block_bwd(xr, blk_np, d_out_np[rows])
    err = rel_l2_rows(host(dx)[rows], ref["dX"])
    assert err <= TOL["bf16"], f"dX {err:.3e}"
    # weight gradients of sampled tokens over the full batch
    for t in DENSE_TOKENS:
        rt = bw.block_bwd_token(inputs["x"], blk_np, d_out_np, t)
        for k in ("w1", "b1", "w2", "b2"):
            e = rel_l2_groups(host(g[k][t])[None], rt[k][None], 1)
            assert e <= TOL["bf16"], f"{k}[{t}] {e:.3e}"


def test_moe_training_full_size_sampled():
    from rankmixer_token_mixing_amd import binding as bd
    cfg, inputs, d_out_np = _workload("c4")
    blk_np = si.add_training_router(inputs["blocks"][0], cfg.dtype)
    blk = bd.upload_blocks([blk_np])[0]
    x = bd.to_device(inputs["x"])
    lam = 0.01
    note(f"[gpu] rm_moe_block_fwd_train + rm_moe_block_bwd, {cfg.description}, block 0")
    y, l_reg, saved = bd.rm_moe_block_fwd_train(x, blk)
    dx, g = bd.rm_moe_block_bwd(x, blk, saved, bd.to_device(d_out_np), lam)
    torch.cuda.synchronize()
    # the sparsity loss sums the inference gates over the whole batch
    S = orc.layer_norm(orc.token_mix(inputs["x"]) + orc.as_f64(inputs["x"]), blk_np["ln1_g"], blk_np["ln1_b"])  # fp64
    l_ref = orc.moe_gates(S, blk_np["wr"], blk_np["br"]).sum()
    assert abs(float(host(l_reg)[0]) - l_ref) <= 1e-3 * l_ref
    # forward output on sampled samples (a gate near zero contributes ~0 either way)
    rows = si.random_rows(cfg.B, 8)
    f = mt.dtsi_fwd_saved(inputs["x"][rows], blk_np)
    assert rel_l2_rows(host(y)[rows], f["out"]) <= TOL["bf16"]
    # dX on sampled samples clear of the ReLU kink
    cand = si.random_rows(cfg.B, 96, seed=777)
    fc = mt.dtsi_fwd_saved(inputs["x"][cand], blk_np)
    margin = np.minimum(np.abs(fc["Zt"]).min(axis=(1, 2)), np.abs(fc["Zi"]).min(axis=(1, 2)))
    clear = cand[margin > KINK_MARGIN][:8]
    assert len(clear) >= 4, f"only {len(clear)} of {len(cand)} sampled samples clear of the kink"
    ref = mt.dtsi_bwd(inputs["x"][clear], blk_np, d_out_np[clear], lam)
    err = rel_l2_rows(host(dx)[clear], ref["dX"])
    assert err <= TOL["bf16"], f"dX {err:.3e}"
    # expert and router gradients of sampled tokens over the full batch
    for t in MOE_TOKENS:
        s_t = S[:, t]
        zt = _kernel_preactivation(s_t, blk_np["wr_train"][t], blk_np["br_train"][t])
        zi = _kernel_preactivation(s_t, blk_np["wr"][t], blk_np["br"][t])
        rt = mt.dtsi_bwd_token(inputs["x"], blk_np, d_out_np, lam, t, train_on=zt > 0, infer_on=zi > 0)
        for k in ("w1", "b1", "w2", "b2"):
            e = rel_l2_groups(host(g[k][t]), rt[k], 1)
            assert e <= TOL["bf16"], f"{k}[{t}] {e:.3e}"
        s_norm = np.linalg.norm(s_t, axis=1)
        near_t = np.abs(zt) < DECISION_BAND
        near_i = np.abs(zi) < DECISION_BAND
        flip = {"wr_train": (np.abs(rt["dG"]) * near_t).T @ s_norm, "br_train": (np.abs(rt["dG"]) * near_t).sum(axis=0),
                "wr": lam * (near_i.T @ s_norm), "br": lam * near_i.sum(axis=0)}
        for k, allow in flip.items():
            got, want = host(g[k][t]), rt[k]
            num = np.linalg.norm((got - want).reshape(len(want), -1), axis=1)
            den = np.linalg.norm(want.reshape(len(want), -1), axis=1)
            den = np.maximum(den, 0.25 * np.sqrt(np.mean(den * den)))
            bound = TOL["bf16"] * den + allow
            assert (num <= bound).all(), f"{k}[{t}] {num} > {bound} ({near_t.sum()}, {near_i.sum()} near the kink)"


def _kernel_preactivation(s_t, w, b):
    """A router's pre-activations as the kernels form them: S rounded to
    bf16, the weights as stored, the product and bias in fp32."""
    sb = orc.round_to_bf16(s_t).astype(np.float32)
    wf = orc.as_f64(w).astype(np.float32)
    return (sb @ wf.T + np.asarray(b, dtype=np.float32)).astype(np.float64)

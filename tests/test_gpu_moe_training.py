"""GPU parity of the MoE block training forward and backward with the
dense-training / sparse-inference routers against the fp64 oracle
(oracle/moe_training.py), through the C ABI.

The ReLU gates decide which terms exist (dz = dG [G_train > 0], the h_infer
gradient counts [G_infer > 0]).  The oracle takes those decisions in fp64, the
kernels in fp32 from dtype inputs, so every case checks on the oracle's side
that no router pre-activation lies within the dtype's rounding of the kink:
bf16 cases use routers whose biases sit at +-3 (pre-activations ~ N(+-3, 1/4)),
fp32 cases seeds whose smallest |pre-activation| is far above fp32 rounding."""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import moe_training as mt
from oracle import rankmixer_oracle as orc
from tests.gpu_util import TOL, ensure_lib, host, note, rel_l2, rel_l2_groups, rel_l2_rows

pytestmark = pytest.mark.gpu

# leading axes that index one group of each gradient: (token, expert) for the
# experts and the router rows, token for the router biases
GROUP_AXES = {"w1": 2, "b1": 2, "w2": 2, "b2": 2, "wr_train": 2, "wr": 2, "br_train": 1, "br": 1}
LAM = 0.37
MARGIN = {"f32": 1e-4, "bf16": 0.25}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _block(T, D, E, He, dtype, seed, separated):
    rng = np.random.default_rng(seed)
    if separated:
        # each (token, expert) router bias is +3 or -3; |w . s| stays near 0.5
        sign = np.where(rng.random((2, T, E)) < 0.6, 1.0, -1.0)
        wscale, br, brt = 0.5, 3.0 * sign[0], 3.0 * sign[1]
    else:
        wscale, br, brt = 1.0, 0.3 * rng.standard_normal((T, E)), 0.4 + 0.3 * rng.standard_normal((T, E))
    p = {
        "w1": rng.standard_normal((T, E, He, D)) / math.sqrt(D),
        "b1": 0.1 * rng.standard_normal((T, E, He)),
        "w2": rng.standard_normal((T, E, D, He)) / math.sqrt(He),
        "b2": 0.1 * rng.standard_normal((T, E, D)),
        "wr": wscale * rng.standard_normal((T, E, D)) / math.sqrt(D),
        "br": br,
        "wr_train": wscale * rng.standard_normal((T, E, D)) / math.sqrt(D),
        "br_train": brt,
        "ln1_g": 1 + 0.1 * rng.standard_normal(D), "ln1_b": 0.1 * rng.standard_normal(D),
        "ln2_g": 1 + 0.1 * rng.standard_normal(D), "ln2_b": 0.1 * rng.standard_normal(D),
    }
    p = {k: v.astype(np.float32) for k, v in p.items()}
    if dtype == "bf16":
        for k in ("w1", "w2", "wr", "wr_train"):
            p[k] = si.to_bf16_bits(p[k])
    return p


def _act(shape, dtype, seed):
    a = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return si.to_bf16_bits(a) if dtype == "bf16" else a


def _run(dtype, B, T, D, E, He, seed, separated):
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(T, D, E, He, dtype, seed, separated)
    x = _act((B, T, D), dtype, seed + 1)
    d_out = _act((B, T, D), dtype, seed + 2)
    f = mt.dtsi_fwd_saved(x, blk)
    margin = min(np.abs(f["Zt"]).min(), np.abs(f["Zi"]).min())
    assert margin > MARGIN[dtype], f"inputs put a gate within {margin:.2e} of the ReLU kink"
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(x)
    y, l_reg, saved = bd.rm_moe_block_fwd_train(xd, dev)
    dx, g = bd.rm_moe_block_bwd(xd, dev, saved, bd.to_device(d_out), LAM)
    torch.cuda.synchronize()
    return blk, x, d_out, f, y, l_reg, dx, g


@pytest.mark.parametrize("dtype,B,T,D,E,He,separated", [
    ("f32", 64, 4, 64, 4, 64, False),      # small fp32 block, natural routers
    ("f32", 33, 2, 40, 4, 24, False),      # batch not a multiple of 64, heads of width 20
    ("bf16", 300, 4, 128, 4, 128, True),   # ragged batch: transposed rows padded to 320
    ("bf16", 1, 2, 16, 4, 32, True),       # one sample
    ("bf16", 1024, 8, 256, 4, 256, True),  # no transposes: GELU' in the dH epilogue, K-major dW1 / dW2
    ("bf16", 320, 2, 384, 4, 384, True),   # no transposes, ragged 256-tiles (B = 320, D = He = 384)
    ("f32", 96, 1, 64, 8, 32, False),      # T = 1: the token mix is the identity
])
def test_moe_training_matches_oracle(dtype, B, T, D, E, He, separated):
    blk, x, d_out, f, y, l_reg, dx, g = _run(dtype, B, T, D, E, He, seed=B + T + E, separated=separated)
    tol = TOL[dtype]
    e = rel_l2_rows(host(y), f["out"])
    assert e <= tol, f"x_out {e:.3e}"
    lr = float(host(l_reg)[0])
    assert abs(lr - f["l_reg"]) <= tol * max(abs(f["l_reg"]), 1e-30), (lr, f["l_reg"])
    ref = mt.dtsi_bwd(x, blk, d_out, LAM)
    e = rel_l2_rows(host(dx), ref["dX"])
    assert e <= tol, f"dX {e:.3e}"
    from rankmixer_token_mixing_amd.binding import MOE_GRADS
    for k in MOE_GRADS:
        # per (token, expert) for the experts and the router rows, per token
        # for the router biases, whole for the LayerNorm vectors
        e = rel_l2_groups(host(g[k]), ref[k], GROUP_AXES[k]) if k in GROUP_AXES else rel_l2(host(g[k]), ref[k])
        assert e <= tol, f"{k} {e:.3e}"


def test_equal_routers_give_the_inference_block():
    # h_train = h_infer: the training forward is the inference MoE block
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(4, 128, 4, 128, "bf16", 11, True)
    blk["wr_train"], blk["br_train"] = blk["wr"].copy(), blk["br"].copy()
    dev = bd.upload_blocks([blk])[0]
    x = _act((256, 4, 128), "bf16", 12)
    xd = bd.to_device(x)
    y_train, l_reg, _ = bd.rm_moe_block_fwd_train(xd, dev)
    y_inf = bd.rm_block_fwd(xd, {k: v for k, v in dev.items() if k not in ("wr_train", "br_train")})
    assert rel_l2_rows(host(y_train), host(y_inf)) <= 1e-2
    assert rel_l2_rows(host(y_train), orc.block_fwd(x, blk)) <= TOL["bf16"]


def test_lambda_scales_only_the_inference_router_gradient():
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(4, 64, 4, 64, "bf16", 13, True)
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(_act((200, 4, 64), "bf16", 14))
    do = bd.to_device(_act((200, 4, 64), "bf16", 15))
    _, _, saved = bd.rm_moe_block_fwd_train(xd, dev)
    a = bd.rm_moe_block_bwd(xd, dev, saved, do, 0.0)
    b = bd.rm_moe_block_bwd(xd, dev, saved, do, 2.0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(a[1]["wr"]).item() == 0 and torch.count_nonzero(a[1]["br"]).item() == 0
    assert torch.count_nonzero(b[1]["br"]).item() > 0
    assert torch.equal(a[0], b[0])
    from rankmixer_token_mixing_amd.binding import MOE_GRADS
    for k in MOE_GRADS:
        if k not in ("wr", "br"):
            assert torch.equal(a[1][k], b[1][k]), k


def test_moe_backward_is_deterministic():
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd.binding import MOE_GRADS
    blk = _block(4, 128, 4, 128, "bf16", 16, True)
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(_act((200, 4, 128), "bf16", 17))
    do = bd.to_device(_act((200, 4, 128), "bf16", 18))
    y1, l1, saved = bd.rm_moe_block_fwd_train(xd, dev)
    y2, l2, _ = bd.rm_moe_block_fwd_train(xd, dev)
    a = bd.rm_moe_block_bwd(xd, dev, saved, do, LAM)
    b = bd.rm_moe_block_bwd(xd, dev, saved, do, LAM)
    assert torch.equal(y1, y2) and torch.equal(l1, l2)
    assert torch.equal(a[0], b[0])
    for k in MOE_GRADS:
        assert torch.equal(a[1][k], b[1][k]), k


def test_moe_empty_batch():
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd.binding import MOE_GRADS
    blk = _block(4, 64, 4, 64, "bf16", 19, True)
    dev = bd.upload_blocks([blk])[0]
    x = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    y, l_reg, saved = bd.rm_moe_block_fwd_train(x, dev)
    dx, g = bd.rm_moe_block_bwd(x, dev, saved, x, LAM)
    torch.cuda.synchronize()
    assert y.shape == (0, 4, 64) and dx.shape == (0, 4, 64)
    assert float(l_reg.item()) == 0.0
    for k in MOE_GRADS:
        assert torch.count_nonzero(g[k]).item() == 0, k


@pytest.mark.parametrize("B,T,D,E,He,transpose_free", [(1024, 8, 256, 4, 256, True), (320, 2, 384, 4, 384, True),
                                                       (300, 4, 128, 4, 128, False)])
def test_moe_backward_path_choice(B, T, D, E, He, transpose_free):
    # bf16, a batch that is a multiple of 64 and experts at least 256 wide
    # run without transposes of dy, H, dU or W2
    from rankmixer_token_mixing_amd import binding as bd
    blk = bd.upload_blocks([_block(T, D, E, He, "bf16", 3, True)])[0]
    xd = bd.to_device(_act((B, T, D), "bf16", 4))
    y, l_reg, saved = bd.rm_moe_block_fwd_train(xd, blk)
    torch.cuda.synchronize()
    bd.profile_enable(True)
    try:
        bd.rm_moe_block_bwd(xd, blk, saved, bd.to_device(_act((B, T, D), "bf16", 5)), LAM)
        torch.cuda.synchronize()
        names = set(bd.profile_read())
    finally:
        bd.profile_enable(False)
    assert ("gelu_bwd" not in names and "tr_dy" not in names and "sums_dy" in names) == transpose_free, names
    # dS reads each token's W1 as stored where the product is at least 256 x 256
    assert ("tr_W1" not in names) == (B >= 256 and D >= 256), names

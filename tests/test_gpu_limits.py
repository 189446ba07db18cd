"""GPU parity at the edges of what the library accepts, against the fp64
oracle through the C ABI: the widest rows (1024 16-byte chunks: D = 8192 in
bf16 and 4096 in fp32 for the token mix and dense blocks; 4096 for MoE
blocks and the training calls), the most experts per token (E = 32) and the
most (token, expert) lists (T*E = 4096).  Hidden widths and batches are kept
small so the oracle stays fast; the widths are what these cases exercise."""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import block_backward as bw
from oracle import moe_training as mt
from oracle import rankmixer_oracle as orc
from tests.gpu_util import TOL, ensure_lib, host, note, rel_l2, rel_l2_groups, rel_l2_rows

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _act(shape, dtype, seed):
    a = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return si.to_bf16_bits(a) if dtype == "bf16" else a


def _ln(rng, D):
    return {"ln1_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
            "ln1_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
            "ln2_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
            "ln2_b": (0.1 * rng.standard_normal(D)).astype(np.float32)}


def _dense(T, D, Hd, dtype, seed):
    rng = np.random.default_rng(seed)
    p = {"w1": (rng.standard_normal((T, Hd, D)) / math.sqrt(D)).astype(np.float32),
         "b1": (0.1 * rng.standard_normal((T, Hd))).astype(np.float32),
         "w2": (rng.standard_normal((T, D, Hd)) / math.sqrt(Hd)).astype(np.float32),
         "b2": (0.1 * rng.standard_normal((T, D))).astype(np.float32), **_ln(rng, D)}
    if dtype == "bf16":
        for k in ("w1", "w2"):
            p[k] = si.to_bf16_bits(p[k])
    return p


def _moe(T, D, E, He, dtype, seed, bias=-0.6745):
    rng = np.random.default_rng(seed)
    p = {"w1": (rng.standard_normal((T, E, He, D)) / math.sqrt(D)).astype(np.float32),
         "b1": (0.1 * rng.standard_normal((T, E, He))).astype(np.float32),
         "w2": (rng.standard_normal((T, E, D, He)) / math.sqrt(He)).astype(np.float32),
         "b2": (0.1 * rng.standard_normal((T, E, D))).astype(np.float32),
         "wr": (rng.standard_normal((T, E, D)) / math.sqrt(D)).astype(np.float32),
         "br": np.full((T, E), bias, np.float32), **_ln(rng, D)}
    if dtype == "bf16":
        for k in ("w1", "w2", "wr"):
            p[k] = si.to_bf16_bits(p[k])
    return p


WIDEST = {"bf16": 8192, "f32": 4096}  # 1024 16-byte chunks per row


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [16, 1024])
def test_token_mix_widest_row(dtype, T):
    # the widest row: heads of D/16 (T = 16) and of 8 or 4 elements (T = 1024)
    from rankmixer_token_mixing_amd import binding as bd
    x = bd.to_device(_act((3, T, WIDEST[dtype]), dtype, T))
    y = bd.rm_token_mix(x)
    np.testing.assert_array_equal(host(y), orc.token_mix(host(x)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_block_widest_row(dtype):
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, Hd = 40, 16, WIDEST[dtype], 64
    blk = _dense(T, D, Hd, dtype, 1)
    x = _act((B, T, D), dtype, 2)
    y = bd.rm_block_fwd(bd.to_device(x), bd.upload_blocks([blk])[0])
    assert rel_l2_rows(host(y), orc.block_fwd(x, blk)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_moe_block_widest_row(dtype):
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, E, He = 50, 8, 4096, 4, 64
    blk = _moe(T, D, E, He, dtype, 3)
    x = _act((B, T, D), dtype, 4)
    y = bd.rm_block_fwd(bd.to_device(x), bd.upload_blocks([blk])[0])
    assert rel_l2_rows(host(y), orc.block_fwd(x, blk)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,B,T,D,E,He", [
    ("bf16", 300, 4, 64, 32, 32),   # the most experts per token
    ("f32", 6, 128, 128, 32, 8),    # T*E = 4096 lists, heads of width 1
])
def test_moe_block_most_experts(dtype, B, T, D, E, He):
    from rankmixer_token_mixing_amd import binding as bd
    blk = _moe(T, D, E, He, dtype, 5)
    x = _act((B, T, D), dtype, 6)
    y = bd.rm_block_fwd(bd.to_device(x), bd.upload_blocks([blk])[0])
    assert rel_l2_rows(host(y), orc.block_fwd(x, blk)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_backward_widest_row(dtype):
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, Hd = 40, 8, 4096, 64
    blk = _dense(T, D, Hd, dtype, 7)
    x = _act((B, T, D), dtype, 8)
    d_out = _act((B, T, D), dtype, 9)
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(x)
    _, saved = bd.rm_block_fwd_train(xd, dev)
    dx, g = bd.rm_block_bwd(xd, dev, saved, bd.to_device(d_out))
    torch.cuda.synchronize()
    ref = bw.block_bwd(x, blk, d_out)
    assert rel_l2_rows(host(dx), ref["dX"]) <= TOL[dtype]
    for k in ("w1", "b1", "w2", "b2"):
        assert rel_l2_groups(host(g[k]), ref[k], 1) <= TOL[dtype], k
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        assert rel_l2(host(g[k]), ref[k]) <= TOL[dtype], k


def test_moe_training_most_experts():
    # E = 32 (the lane-held gate gradients fill half a wave) and T = 1; both
    # routers' biases sit at +-3, so no gate is near the ReLU kink
    from rankmixer_token_mixing_amd import binding as bd
    from rankmixer_token_mixing_amd.binding import MOE_GRADS
    B, T, D, E, He = 70, 1, 64, 32, 32
    rng = np.random.default_rng(10)
    blk = _moe(T, D, E, He, "bf16", 11)
    blk["wr"] = si.to_bf16_bits((0.5 * rng.standard_normal((T, E, D)) / math.sqrt(D)).astype(np.float32))
    blk["br"] = (3.0 * np.where(rng.random((T, E)) < 0.5, 1.0, -1.0)).astype(np.float32)
    blk["wr_train"] = si.to_bf16_bits((0.5 * rng.standard_normal((T, E, D)) / math.sqrt(D)).astype(np.float32))
    blk["br_train"] = (3.0 * np.where(rng.random((T, E)) < 0.7, 1.0, -1.0)).astype(np.float32)
    x = _act((B, T, D), "bf16", 12)
    d_out = _act((B, T, D), "bf16", 13)
    f = mt.dtsi_fwd_saved(x, blk)
    assert min(np.abs(f["Zt"]).min(), np.abs(f["Zi"]).min()) > 0.25
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(x)
    y, l_reg, saved = bd.rm_moe_block_fwd_train(xd, dev)
    dx, g = bd.rm_moe_block_bwd(xd, dev, saved, bd.to_device(d_out), 0.5)
    torch.cuda.synchronize()
    assert rel_l2_rows(host(y), f["out"]) <= TOL["bf16"]
    assert abs(float(host(l_reg)[0]) - f["l_reg"]) <= TOL["bf16"] * f["l_reg"]
    ref = mt.dtsi_bwd(x, blk, d_out, 0.5)
    assert rel_l2_rows(host(dx), ref["dX"]) <= TOL["bf16"]
    groups = {"w1": 2, "b1": 2, "w2": 2, "b2": 2, "wr_train": 2, "wr": 2, "br_train": 1, "br": 1}
    for k in MOE_GRADS:
        e = rel_l2_groups(host(g[k]), ref[k], groups[k]) if k in groups else rel_l2(host(g[k]), ref[k])
        assert e <= TOL["bf16"], k

"""GPU parity of the block variants of "淘宝闪购-爆品团精排 Scaling Up 迭代实践"
against the fp64 oracle, through the C ABI: the SwiGLU per-token FFN (section
3.6, D -> 4/3 D) and the block without the Add & Norm after the token mix
(section 3.5), alone, combined, with the MoE, and stacked in a model."""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import rankmixer_oracle as orc
from tests.gpu_util import TOL, ensure_lib, host, note, rel_l2_rows

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _mat(a, dtype):
    a = a.astype(np.float32)
    return si.to_bf16_bits(a) if dtype == "bf16" else a


def _block(T, D, H, dtype, seed, swiglu=False, no_mix_norm=False):
    rng = np.random.default_rng(seed)
    n1 = 2 * H if swiglu else H
    p = {
        "w1": _mat(rng.standard_normal((T, n1, D)) / math.sqrt(D), dtype),
        "b1": (0.1 * rng.standard_normal((T, n1))).astype(np.float32),
        "w2": _mat(rng.standard_normal((T, D, H)) / math.sqrt(H), dtype),
        "b2": (0.1 * rng.standard_normal((T, D))).astype(np.float32),
        "ln1_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln1_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln2_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln2_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
    }
    if swiglu:
        p["swiglu"] = True
    if no_mix_norm:
        p["no_mix_norm"] = True
    return p


def _x(B, T, D, dtype, seed):
    return _mat(np.random.default_rng(seed).standard_normal((B, T, D)), dtype)


@pytest.mark.parametrize("dtype,B,T,D,Hs", [
    ("f32", 64, 4, 64, 88),        # fp32, hidden not a multiple of 64
    ("bf16", 300, 4, 96, 128),     # 4/3 D, ragged batch
    ("bf16", 1, 2, 16, 24),        # one sample
    ("bf16", 1024, 16, 768, 1024), # 4/3 D at the 100M-class width: fused SwiGLU epilogue
    ("bf16", 1100, 16, 768, 1000), # fused epilogue with a ragged last gate/up tile and ragged batch
])
def test_swiglu_block_matches_oracle(dtype, B, T, D, Hs):
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(T, D, Hs, dtype, seed=B + D, swiglu=True)
    x = _x(B, T, D, dtype, seed=Hs)
    y = host(bd.rm_block_fwd(bd.to_device(x), bd.upload_blocks([blk])[0]))
    rows = si.random_rows(B, 64, seed=1)
    assert rel_l2_rows(y[rows], orc.block_fwd(x[rows], blk)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,B,T,D,H,swiglu", [
    ("bf16", 300, 4, 128, 256, False),
    ("f32", 33, 1, 64, 96, False),   # T = 1: S = X
    ("bf16", 200, 8, 64, 96, True),  # both variants together
])
def test_no_mix_norm_block_matches_oracle(dtype, B, T, D, H, swiglu):
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(T, D, H, dtype, seed=B + 7, swiglu=swiglu, no_mix_norm=True)
    x = _x(B, T, D, dtype, seed=H + 1)
    y = host(bd.rm_block_fwd(bd.to_device(x), bd.upload_blocks([blk])[0]))
    rows = si.random_rows(B, 64, seed=2)
    assert rel_l2_rows(y[rows], orc.block_fwd(x[rows], blk)) <= TOL[dtype]


def test_no_mix_norm_moe_block_matches_oracle():
    from rankmixer_token_mixing_amd import binding as bd
    cfg = si.Config("moe-nomix", B=200, T=4, D=64, L=1, dtype="bf16", E=4, He=64)
    inputs = si.make_inputs(cfg, seed=9)
    blk = dict(inputs["blocks"][0])
    blk["no_mix_norm"] = True
    y = host(bd.rm_block_fwd(bd.to_device(inputs["x"]), bd.upload_blocks([blk])[0]))
    rows = si.random_rows(cfg.B, 48, seed=3)
    assert rel_l2_rows(y[rows], orc.block_fwd(inputs["x"][rows], blk)) <= TOL["bf16"]


def test_swiglu_model_stacks_blocks():
    from rankmixer_token_mixing_amd import binding as bd
    T, D, Hs, B = 8, 96, 128, 256
    blocks = [_block(T, D, Hs, "bf16", seed=20 + l, swiglu=True, no_mix_norm=(l == 1)) for l in range(2)]
    x = _x(B, T, D, "bf16", seed=30)
    model = bd.Model(bd.upload_blocks(blocks), T, D, torch.bfloat16)
    y = host(bd.rm_model_fwd(model, bd.to_device(x))["x"])
    rows = si.random_rows(B, 48, seed=4)
    ref = orc.model_fwd(x[rows], blocks, T, D, "bf16")["x"]
    assert rel_l2_rows(y[rows], ref) <= TOL["bf16"]

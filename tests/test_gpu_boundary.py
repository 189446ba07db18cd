"""GPU parity of block boundaries in rm_model_fwd: where a dense or SwiGLU
block is followed by a block with the Add & Norm after its mix, the model
runs LayerNorm 2 of the first and the token mix + LayerNorm 1 of the second
as one pass per sample (the output between them never reaches HBM).  Models
that mix block kinds, odd head widths, a block without the Add & Norm after
the mix, and a row too wide for the pass (so the two kernels run apart) are
compared with the fp64 oracle, and the fused model with the same blocks
called one at a time."""
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


def _ln(rng, D):
    return {"ln1_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
            "ln1_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
            "ln2_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
            "ln2_b": (0.1 * rng.standard_normal(D)).astype(np.float32)}


def _block(kind, T, D, H, dtype, seed, E=4, no_mix_norm=False):
    rng = np.random.default_rng(seed)
    if kind == "moe":
        p = {"w1": rng.standard_normal((T, E, H, D)) / math.sqrt(D), "b1": 0.1 * rng.standard_normal((T, E, H)),
             "w2": rng.standard_normal((T, E, D, H)) / math.sqrt(H), "b2": 0.1 * rng.standard_normal((T, E, D)),
             "wr": rng.standard_normal((T, E, D)) / math.sqrt(D), "br": np.full((T, E), -0.6745)}
        mats = ("w1", "w2", "wr")
    else:
        n1 = 2 * H if kind == "swiglu" else H
        p = {"w1": rng.standard_normal((T, n1, D)) / math.sqrt(D), "b1": 0.1 * rng.standard_normal((T, n1)),
             "w2": rng.standard_normal((T, D, H)) / math.sqrt(H), "b2": 0.1 * rng.standard_normal((T, D))}
        mats = ("w1", "w2")
    p = {k: v.astype(np.float32) for k, v in p.items()}
    p.update(_ln(rng, D))
    if dtype == "bf16":
        for k in mats:
            p[k] = si.to_bf16_bits(p[k])
    if kind == "swiglu":
        p["swiglu"] = True
    if no_mix_norm:
        p["no_mix_norm"] = True
    return p


def _x(B, T, D, dtype, seed):
    a = np.random.default_rng(seed).standard_normal((B, T, D)).astype(np.float32)
    return si.to_bf16_bits(a) if dtype == "bf16" else a


def _check(blocks, B, T, D, dtype, seed, chain=True):
    from rankmixer_token_mixing_amd import binding as bd
    x = _x(B, T, D, dtype, seed)
    dev = bd.upload_blocks(blocks)
    model = bd.Model(dev, T, D, DT[dtype])
    xd = bd.to_device(x)
    y = bd.rm_model_fwd(model, xd)["x"]
    ref = orc.model_fwd(x, blocks, T, D, dtype)["x"]
    assert rel_l2_rows(host(y), ref) <= TOL[dtype]
    if chain:
        # the same blocks one call at a time (no fused boundary): equal up to
        # the rounding of the block outputs
        z = xd
        for blk in dev:
            z = bd.rm_block_fwd(z, blk)
        assert rel_l2_rows(host(y), host(z)) <= (1e-5 if dtype == "f32" else 1e-2)


def test_mixed_kinds():
    # dense -> SwiGLU and SwiGLU -> MoE boundaries fuse; MoE -> dense does not
    T, D, H = 8, 128, 128
    kinds = ["dense", "swiglu", "moe", "dense"]
    blocks = [_block(k, T, D, H, "bf16", 10 + i) for i, k in enumerate(kinds)]
    _check(blocks, 300, T, D, "bf16", 1)


@pytest.mark.parametrize("dtype,B,T,D,H", [
    ("f32", 37, 8, 40, 24),     # heads of width 5
    ("bf16", 65, 32, 64, 32),   # heads of width 2
    ("bf16", 9, 1, 64, 96),     # T = 1
    ("bf16", 513, 16, 320, 64),  # the pad-split model's width
    ("bf16", 600, 32, 1536, 32),  # the ~1B-class shape: three chunks per lane, the LDS nearly full
    ("bf16", 70, 64, 128, 32),    # T > 32: each wave normalises several pairs of rows
    ("bf16", 40, 16, 2048, 32),   # four chunks per lane
    # two chunks per lane: four rows per wave in the first phase
    ("bf16", 131, 16, 768, 64),   # the ~100M-class width
    ("bf16", 77, 5, 640, 32),     # T = 5: waves of three and of two rows
    ("f32", 45, 12, 480, 32),     # fp32 rows of 120 chunks, heads of 40
    ("bf16", 50, 32, 1024, 32),   # T = 32 at the widest such row
])
def test_dense_stacks(dtype, B, T, D, H):
    blocks = [_block("dense", T, D, H, dtype, 20 + i) for i in range(3)]
    _check(blocks, B, T, D, dtype, 2)


def test_block_without_mix_norm_breaks_the_fusion():
    T, D, H = 8, 96, 64
    blocks = [_block("dense", T, D, H, "bf16", 30), _block("dense", T, D, H, "bf16", 31, no_mix_norm=True),
              _block("swiglu", T, D, H, "bf16", 32)]
    _check(blocks, 200, T, D, "bf16", 3)


@pytest.mark.parametrize("dtype,B,T,D,spec", [
    # SwiGLU, then an MoE block with E = 4 and no Add & Norm after its mix,
    # then an MoE block with E = 8 (heads of 19, one-element row chunks in fp32)
    ("f32", 329, 32, 608, [("swiglu", 24, 0, False), ("moe", 24, 4, True), ("moe", 24, 8, False)]),
    # hidden widths and expert counts that differ from block to block
    ("bf16", 300, 8, 128, [("dense", 256, 0, False), ("swiglu", 48, 0, False), ("moe", 32, 3, False),
                           ("moe", 64, 6, False), ("dense", 128, 0, False)]),
])
def test_blocks_sized_from_their_own_descriptors(dtype, B, T, D, spec):
    blocks = [_block(k, T, D, H, dtype, 50 + i, E=E or 4, no_mix_norm=nmn) for i, (k, H, E, nmn) in enumerate(spec)]
    _check(blocks, B, T, D, dtype, 5)


def test_row_too_wide_for_the_boundary_pass():
    # 16 rows of 8192 bf16 do not fit in LDS: LayerNorm 2 and the next mix run
    # as separate kernels
    T, D, H = 16, 8192, 32
    blocks = [_block("dense", T, D, H, "bf16", 40 + i) for i in range(2)]
    _check(blocks, 12, T, D, "bf16", 4, chain=False)

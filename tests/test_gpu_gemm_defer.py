"""GPU parity of the grouped products on the deferred-epilogue kernel, the
epilogue-overlap mode (rm_set_epilogue_overlap(1); bf16, K a multiple of 64
and at least 1024, M and N at least 256): each finished 256 x 256 tile is
packed to bf16 in registers and its GELU and stores run inside the next
tile's main loop, the last tile's plainly.  The shapes
make every path run: several tiles per workgroup (the deferred path) and one
(the final drain), a last M tile and a last N tile moved back over their
neighbour (rows and columns computed twice), K = 1088 (one stage past the
sixteen that carry the units), zero and non-zero bias; the training forward
writes the pre-activation and its GELU.  Outputs of sampled samples --
including the rows the moved-back tiles recompute -- are compared with the
fp64 oracle (samples never interact, so the oracle on a subset is exact)."""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import rankmixer_oracle as orc
from tests.gpu_util import TOL, ensure_lib, host, note, rel_l2_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from rankmixer_token_mixing_amd import binding as bd
    ensure_lib()
    bd.set_epilogue_overlap(True)
    yield
    bd.set_epilogue_overlap(False)


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _params(T, D, Hd, seed, bias):
    rng = np.random.default_rng(seed)
    p = {"w1": si.to_bf16_bits((rng.standard_normal((T, Hd, D)) / math.sqrt(D)).astype(np.float32)),
         "w2": si.to_bf16_bits((rng.standard_normal((T, D, Hd)) / math.sqrt(Hd)).astype(np.float32)),
         "b1": (bias * rng.standard_normal((T, Hd))).astype(np.float32),
         "b2": (bias * rng.standard_normal((T, D))).astype(np.float32)}
    return p


def _rows(B):
    # first and last samples, the band a moved-back last M tile recomputes,
    # and a seeded spread
    m_last = max(0, B - 256)
    rows = {0, 1, B - 1, B - 2, m_last, m_last + 1, (B // 256) * 256 - 1 if B >= 256 else 0}
    rows.update(si.random_rows(B, 24, seed=B).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < B))


@pytest.mark.parametrize("B,T,D,Hd,bias", [
    (1200, 8, 1024, 2304, 0.1),  # W1: 5 M tiles (last moved back), 360 tiles; W2: K = 2304
    (512, 16, 1536, 2104, 0.1),  # W1: 9 N tiles, the last moved back; 288 tiles
    (256, 2, 1088, 1024, 0.0),   # K = 1088 (17 stages), one tile per workgroup, no bias
    (1200, 16, 1024, 1024, 0.1),  # both products with 320 tiles: several per workgroup
])
def test_pffn_on_the_deferred_kernel(B, T, D, Hd, bias):
    from rankmixer_token_mixing_amd import binding as bd
    p = _params(T, D, Hd, seed=D + Hd, bias=bias)
    s = si.to_bf16_bits(np.random.default_rng(B).standard_normal((B, T, D)).astype(np.float32))
    dev = {k: bd.to_device(v) for k, v in p.items()}
    v = bd.rm_pffn_fwd(bd.to_device(s), dev)
    torch.cuda.synchronize()
    rows = _rows(B)
    ref = orc.pffn(si.bf16_bits_to_f32(s[rows]), si.bf16_bits_to_f32(p["w1"]), p["b1"],
                   si.bf16_bits_to_f32(p["w2"]), p["b2"])
    got = host(v)[rows]
    assert np.isfinite(got).all()
    assert rel_l2_rows(got, ref) <= TOL["bf16"]


def test_deferred_kernel_is_deterministic():
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, Hd = 1200, 8, 1024, 2304
    p = {k: bd.to_device(v) for k, v in _params(T, D, Hd, seed=7, bias=0.1).items()}
    s = bd.to_device(si.to_bf16_bits(np.random.default_rng(3).standard_normal((B, T, D)).astype(np.float32)))
    a = bd.rm_pffn_fwd(s, p)
    b = bd.rm_pffn_fwd(s, p)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_training_forward_keeps_the_preactivation_and_its_gelu():
    # the dual epilogue: U = W1 s + b1 (saved) and H = GELU(U); the block's
    # training forward equals its inference forward up to the rounding of U
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, Hd = 512, 4, 1024, 2048
    rng = np.random.default_rng(11)
    blk = _params(T, D, Hd, seed=5, bias=0.1)
    blk.update({"ln1_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
                "ln1_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
                "ln2_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
                "ln2_b": (0.1 * rng.standard_normal(D)).astype(np.float32)})
    x = si.to_bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32))
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(x)
    y_train, _ = bd.rm_block_fwd_train(xd, dev)
    y = bd.rm_block_fwd(xd, dev)
    torch.cuda.synchronize()
    rows = _rows(B)
    ref = orc.block_fwd(si.bf16_bits_to_f32(x[rows]), {k: (si.bf16_bits_to_f32(v) if v.dtype == np.uint16 else v)
                                                       for k, v in blk.items()})
    assert rel_l2_rows(host(y_train)[rows], ref) <= TOL["bf16"]
    assert rel_l2_rows(host(y_train), host(y)) <= 1e-2


def test_both_epilogue_modes_agree():
    # the same products with the epilogue after each tile (mode 0): equal up
    # to the bf16 rounding of outputs whose bias joins at another point
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, Hd = 1200, 8, 1024, 2304
    p = {k: bd.to_device(v) for k, v in _params(T, D, Hd, seed=9, bias=0.1).items()}
    s = bd.to_device(si.to_bf16_bits(np.random.default_rng(4).standard_normal((B, T, D)).astype(np.float32)))
    a = bd.rm_pffn_fwd(s, p)
    bd.set_epilogue_overlap(False)
    try:
        b = bd.rm_pffn_fwd(s, p)
    finally:
        bd.set_epilogue_overlap(True)
    torch.cuda.synchronize()
    assert rel_l2_rows(host(a), host(b)) <= 1e-2

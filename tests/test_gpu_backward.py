"""GPU parity of the dense block training forward and backward against the
fp64 oracle (oracle/block_backward.py), through the C ABI.  Weight gradients
sum over the whole batch, so these shapes are ones the oracle finishes in
seconds; the per-token weight and bias gradients are compared per token group
(relative L2 of each token's slice), the LayerNorm gradients as a whole, dx
per sample."""
import math

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import block_backward as bw
from oracle import rankmixer_oracle as orc
from tests.gpu_util import TOL, ensure_lib, host, note, rel_l2, rel_l2_groups, rel_l2_rows

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}
GRADS = ("w1", "b1", "w2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")
PER_TOKEN = ("w1", "b1", "w2", "b2")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _block(T, D, Hd, dtype, seed):
    rng = np.random.default_rng(seed)
    p = {
        "w1": (rng.standard_normal((T, Hd, D)) / math.sqrt(D)).astype(np.float32),
        "b1": (0.1 * rng.standard_normal((T, Hd))).astype(np.float32),
        "w2": (rng.standard_normal((T, D, Hd)) / math.sqrt(Hd)).astype(np.float32),
        "b2": (0.1 * rng.standard_normal((T, D))).astype(np.float32),
        "ln1_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln1_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln2_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln2_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
    }
    if dtype == "bf16":
        p["w1"] = si.to_bf16_bits(p["w1"])
        p["w2"] = si.to_bf16_bits(p["w2"])
    return p


def _act(shape, dtype, seed):
    a = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return si.to_bf16_bits(a) if dtype == "bf16" else a


def _run(dtype, B, T, D, Hd, seed):
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(T, D, Hd, dtype, seed)
    x = _act((B, T, D), dtype, seed + 1)
    d_out = _act((B, T, D), dtype, seed + 2)
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(x)
    y, saved = bd.rm_block_fwd_train(xd, dev)
    dx, g = bd.rm_block_bwd(xd, dev, saved, bd.to_device(d_out))
    torch.cuda.synchronize()
    return blk, x, d_out, y, dx, g


@pytest.mark.parametrize("dtype,B,T,D,Hd", [
    ("f32", 64, 4, 64, 128),      # the tiny fp32 block
    ("f32", 33, 1, 64, 96),       # T = 1, batch not a multiple of 64
    ("bf16", 300, 4, 128, 256),   # ragged batch: transposed rows padded to 320 (the transposing path)
    ("bf16", 1, 2, 16, 32),       # one sample
    ("bf16", 1024, 8, 256, 1024), # no transposes: dH with the GELU backward epilogue, dW1 / dW2 read K-major
    ("bf16", 320, 3, 384, 768),   # no transposes, ragged 256-tiles in every product (M = 320, D = 384)
    ("f32", 17, 8, 40, 24),       # heads of width 5: odd gathers
    ("bf16", 1024, 16, 256, 2048),  # dH reads W2 K-major (transposed fragment reads, 256 x 256 tiles)
    ("bf16", 1000, 32, 1024, 1024),  # ragged batch, dH and dS both read W K-major
])
def test_block_backward_matches_oracle(dtype, B, T, D, Hd):
    blk, x, d_out, y, dx, g = _run(dtype, B, T, D, Hd, seed=B + T)
    tol = TOL[dtype]
    # training forward output equals the forward oracle
    assert rel_l2_rows(host(y), orc.block_fwd(x, blk)) <= tol
    ref = bw.block_bwd(x, blk, d_out)
    err = rel_l2_rows(host(dx), ref["dX"])
    assert err <= tol, f"dX {err:.3e}"
    for k in GRADS:
        # per token group for the per-token weights and biases, whole for
        # the LayerNorm vectors every token shares
        e = rel_l2_groups(host(g[k]), ref[k], 1) if k in PER_TOKEN else rel_l2(host(g[k]), ref[k])
        assert e <= tol, f"{k} {e:.3e}"


def test_backward_is_deterministic():
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(4, 128, 256, "bf16", 3)
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(_act((200, 4, 128), "bf16", 4))
    do = bd.to_device(_act((200, 4, 128), "bf16", 5))
    y, saved = bd.rm_block_fwd_train(xd, dev)
    a = bd.rm_block_bwd(xd, dev, saved, do)
    b = bd.rm_block_bwd(xd, dev, saved, do)
    assert torch.equal(a[0], b[0])
    for k in GRADS:
        assert torch.equal(a[1][k], b[1][k]), k


def test_training_forward_matches_inference_forward():
    # the same block; only the GELU input is rounded to the dtype in between
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(8, 256, 1024, "bf16", 6)
    dev = bd.upload_blocks([blk])[0]
    xd = bd.to_device(_act((512, 8, 256), "bf16", 7))
    y_train, _ = bd.rm_block_fwd_train(xd, dev)
    y_inf = bd.rm_block_fwd(xd, dev)
    assert rel_l2_rows(host(y_train), host(y_inf)) <= 1e-2


def test_empty_batch_gives_zero_gradients():
    from rankmixer_token_mixing_amd import binding as bd
    blk = _block(4, 64, 128, "bf16", 8)
    dev = bd.upload_blocks([blk])[0]
    x = torch.empty((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    saved = torch.empty(16, dtype=torch.uint8, device="cuda")
    dx, g = bd.rm_block_bwd(x, dev, saved, x)
    torch.cuda.synchronize()
    assert dx.shape == (0, 4, 64)
    for k in GRADS:
        assert torch.count_nonzero(g[k]).item() == 0, k


@pytest.mark.parametrize("B,T,D,Hd,transpose_free", [(1024, 8, 256, 1024, True), (320, 3, 384, 768, True),
                                                     (1000, 32, 1024, 1024, False), (300, 4, 128, 256, False)])
def test_backward_path_choice(B, T, D, Hd, transpose_free):
    # a batch that is a multiple of 64 with every product at least 256 x 256
    # runs without transposes: the dH product's epilogue applies GELU' and
    # the weight-gradient products read both operands as stored
    from rankmixer_token_mixing_amd import binding as bd
    dev = bd.upload_blocks([_block(T, D, Hd, "bf16", 3)])[0]
    xd = bd.to_device(_act((B, T, D), "bf16", 4))
    y, saved = bd.rm_block_fwd_train(xd, dev)
    torch.cuda.synchronize()
    bd.profile_enable(True)
    try:
        bd.rm_block_bwd(xd, dev, saved, bd.to_device(_act((B, T, D), "bf16", 5)))
        torch.cuda.synchronize()
        names = set(bd.profile_read())
    finally:
        bd.profile_enable(False)
    assert ("gelu_bwd" not in names and "tr_S" not in names and "sums_dV" in names) == transpose_free, names

"""GPU parity of the block and the whole stack on the five workload
configurations, through the C ABI, in the launch configuration the
benchmark times (rm_model_fwd over the full batch).  The oracle evaluates a
seeded subset of samples (always the first and the last): samples never
interact, so the subset is exact."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import rankmixer_oracle as orc
from tests.gpu_util import TOL, config_inputs, ensure_lib, host, note, rel_l2, rel_l2_rows

pytestmark = pytest.mark.gpu

ORACLE_ROWS = {"c0": 64, "c1": 48, "c2": 64, "c3": 24, "c4": 32}
DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


@pytest.fixture(autouse=True)
def _name(request):
    note(f"[gpu] {request.node.nodeid}")


def _model(inputs):
    from rankmixer_token_mixing_amd import binding as bd
    cfg = inputs["config"]
    blocks = bd.upload_blocks(inputs["blocks"])
    head = None
    if "head" in inputs:
        head = {"w": bd.to_device(inputs["head"]["w"]), "c": inputs["head"]["c"]}
    model = bd.Model(blocks, cfg.T, cfg.D, DT[cfg.dtype], F=cfg.F, head=head)
    inp = bd.to_device(inputs["emb"] if cfg.F else inputs["x"])
    return model, inp


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_config_matches_oracle(name):
    from rankmixer_token_mixing_amd import binding as bd
    inputs = config_inputs(name)
    cfg = inputs["config"]
    model, inp = _model(inputs)
    note(f"[gpu] rm_model_fwd {cfg.description}")
    out = bd.rm_model_fwd(model, inp, want_x=True, want_pooled=cfg.head)
    torch.cuda.synchronize()
    rows = si.random_rows(cfg.B, ORACLE_ROWS[name])
    ref = orc.run_config(inputs, rows)
    err = rel_l2_rows(host(out["x"])[rows], ref["x"])
    assert err <= TOL[cfg.dtype], f"{name}: max relative L2 {err:.3e}"
    if cfg.head:
        err_l = rel_l2(host(out["logit"])[rows], ref["logit"])
        assert err_l <= TOL[cfg.dtype], f"{name}: logit relative L2 {err_l:.3e}"
        err_p = rel_l2_rows(host(out["pooled"])[rows], ref["pooled"])
        assert err_p <= TOL[cfg.dtype]
    # LayerNorm output statistics (gamma = 1, beta = 0): every token row has
    # mean ~0 and variance ~1 over the whole batch, not just the sample
    x = out["x"].float()
    assert x.mean(dim=-1).abs().max().item() < 0.02
    assert (x.var(dim=-1, unbiased=False) - 1).abs().max().item() < 0.03
    assert torch.isfinite(x).all()


@pytest.mark.parametrize("name", ["c1", "c4"])
def test_model_is_deterministic(name):
    from rankmixer_token_mixing_amd import binding as bd
    inputs = config_inputs(name)
    model, inp = _model(inputs)
    a = bd.rm_model_fwd(model, inp)["x"].clone()
    b = bd.rm_model_fwd(model, inp)["x"]
    assert torch.equal(a, b)


def test_block_fwd_equals_first_block_of_the_model():
    from rankmixer_token_mixing_amd import binding as bd
    inputs = config_inputs("c1")
    cfg = inputs["config"]
    blocks = bd.upload_blocks(inputs["blocks"][:1])
    x = bd.to_device(inputs["x"])
    y1 = bd.rm_block_fwd(x, blocks[0])
    y2 = bd.rm_model_fwd(bd.Model(blocks, cfg.T, cfg.D, torch.bfloat16), x)["x"]
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("dtype,B,T,D,k", [
    ("bf16", 1, 4, 64, 2),       # one sample
    ("f32", 33, 1, 64, 2),       # T = 1: the mix is the identity
    ("bf16", 20, 32, 64, 2),     # heads of width 2
    ("bf16", 300, 16, 320, 4),   # heads of width 20, ragged batch
    ("f32", 17, 8, 40, 3),       # odd hidden multiple, heads of width 5
])
def test_block_edge_shapes(dtype, B, T, D, k):
    from rankmixer_token_mixing_amd import binding as bd
    cfg = si.Config("edge", B=B, T=T, D=D, L=1, dtype=dtype, k=k, bias_var=0.01)
    inputs = si.make_inputs(cfg, seed=B + T)
    blocks = bd.upload_blocks(inputs["blocks"])
    y = bd.rm_block_fwd(bd.to_device(inputs["x"]), blocks[0])
    ref = orc.block_fwd(inputs["x"], inputs["blocks"][0])
    assert rel_l2_rows(host(y), ref) <= TOL[dtype]


def test_moe_block_edge_all_gates_off():
    # router bias far below zero: every gate is 0, so X' = LN2(S)
    from rankmixer_token_mixing_amd import binding as bd
    cfg = si.Config("moe-off", B=40, T=4, D=64, L=1, dtype="bf16", E=4, He=64)
    inputs = si.make_inputs(cfg, seed=3)
    inputs["blocks"][0]["br"][:] = -1e4
    blocks = bd.upload_blocks(inputs["blocks"])
    y = bd.rm_block_fwd(bd.to_device(inputs["x"]), blocks[0])
    ref = orc.block_fwd(inputs["x"], inputs["blocks"][0])
    assert rel_l2_rows(host(y), ref) <= TOL["bf16"]


def test_moe_block_one_expert_takes_all_rows():
    # per token one expert whose gate is on for (almost) every sample, the
    # others off: full 256-row expert tiles, a partial last tile, and empty
    # groups in the device-side tile list of the ragged products
    from rankmixer_token_mixing_amd import binding as bd
    cfg = si.Config("moe-one", B=600, T=4, D=256, L=1, dtype="bf16", E=4, He=512)
    inputs = si.make_inputs(cfg, seed=5)
    br = inputs["blocks"][0]["br"]
    br[:] = -1e4
    for t in range(cfg.T):
        br[t, t % cfg.E] = 3.0
    blocks = bd.upload_blocks(inputs["blocks"])
    y = bd.rm_block_fwd(bd.to_device(inputs["x"]), blocks[0])
    rows = si.random_rows(cfg.B, 48, seed=2)
    ref = orc.block_fwd(inputs["x"][rows], inputs["blocks"][0])
    assert rel_l2_rows(host(y)[rows], ref) <= TOL["bf16"]


def test_empty_batch_returns_empty():
    from rankmixer_token_mixing_amd import binding as bd
    cfg = si.Config("empty", B=4, T=4, D=64, L=1, dtype="bf16", k=2)
    inputs = si.make_inputs(cfg, seed=1)
    blocks = bd.upload_blocks(inputs["blocks"])
    x = bd.to_device(inputs["x"])[:0].contiguous()
    y = bd.rm_block_fwd(x, blocks[0])
    assert y.shape == (0, 4, 64)
    assert bd.rm_token_mix(x).shape == (0, 4, 64)


def test_widest_supported_rows():
    # D = 8192 (heads of 512): the widest row the LayerNorm / mix kernels hold;
    # a narrow hidden width keeps the weights small
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, Hd = 3, 16, 8192, 64
    rng = np.random.default_rng(5)
    x = si.to_bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32))
    blk = {
        "w1": si.to_bf16_bits((rng.standard_normal((T, Hd, D)) / np.sqrt(D)).astype(np.float32)),
        "b1": (0.1 * rng.standard_normal((T, Hd))).astype(np.float32),
        "w2": si.to_bf16_bits((rng.standard_normal((T, D, Hd)) / np.sqrt(Hd)).astype(np.float32)),
        "b2": (0.1 * rng.standard_normal((T, D))).astype(np.float32),
        "ln1_g": np.ones(D, np.float32), "ln1_b": np.zeros(D, np.float32),
        "ln2_g": np.ones(D, np.float32), "ln2_b": np.zeros(D, np.float32),
    }
    y = bd.rm_block_fwd(bd.to_device(x), bd.upload_blocks([blk])[0])
    ref = orc.block_fwd(x, blk)
    assert rel_l2_rows(host(y), ref) <= TOL["bf16"]
    m = bd.rm_token_mix(bd.to_device(x))
    np.testing.assert_array_equal(host(m), orc.token_mix(x))


def test_ragged_tiles_of_the_pipelined_products():
    # B = 1100 rows (last M tile holds 76), hidden 1472 (last N tile of the W1
    # product holds 192 columns): the W1 product takes 256x256 tiles and the
    # W2 product 256x128 tiles of the hand-scheduled persistent kernel, each
    # with 960 tiles (3.75 rounds of one workgroup per CU)
    from rankmixer_token_mixing_amd import binding as bd
    cfg = si.Config("ragged-pipe", B=1100, T=32, D=768, L=1, dtype="bf16", k=2, bias_var=0.01)
    inputs = si.make_inputs(cfg, seed=11)
    blk = dict(inputs["blocks"][0])
    blk["w1"] = blk["w1"][:, :1472, :].copy()
    blk["b1"] = blk["b1"][:, :1472].copy()
    blk["w2"] = np.ascontiguousarray(blk["w2"][:, :, :1472])
    blocks = bd.upload_blocks([blk])
    y = host(bd.rm_block_fwd(bd.to_device(inputs["x"]), blocks[0]))
    rows = np.unique(np.concatenate([si.random_rows(cfg.B, 24, seed=3), np.arange(1024, 1100, 7), [1099]]))
    ref = orc.block_fwd(inputs["x"][rows], blk)
    assert rel_l2_rows(y[rows], ref) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,B,T,D,F,kinds", [
    ("bf16", 4096, 16, 320, 5000, ("dense", "dense")),   # the pad-split model's shape (pieces of 4)
    ("bf16", 100, 4, 64, 100, ("dense",)),               # pieces of 8, one straddling F = 100
    ("bf16", 70, 4, 64, 4, ("moe", "dense")),            # four floats, the rest padding
    ("bf16", 33, 8, 128, 1024, ("swiglu", "dense")),     # F = T * D: no padding
    ("f32", 65, 5, 40, 196, ("dense", "moe")),           # fp32, heads of 8, pieces of 4 straddling F
])
def test_tokenizer_fused_into_the_first_mix_is_exact(dtype, B, T, D, F, kinds):
    # rm_model_fwd reads the embedding in place where F % 4 == 0 and block 0
    # starts with the token mix + LayerNorm 1; the result equals tokenizing
    # first and running the same blocks on X0, bit for bit
    from rankmixer_token_mixing_amd import binding as bd
    from tests.test_gpu_boundary import _block
    rng = np.random.default_rng(B + F)
    emb = (0.3 * rng.standard_normal((B, F))).astype(np.float32)
    np_blocks = [_block(k, T, D, 64, dtype, 60 + i) for i, k in enumerate(kinds)]
    blocks = bd.upload_blocks(np_blocks)
    head_w = (rng.standard_normal(D) / D).astype(np.float32)
    head = {"w": bd.to_device(head_w), "c": 0.25}
    fused = bd.Model(blocks, T, D, DT[dtype], F=F, head=head)
    plain = bd.Model(blocks, T, D, DT[dtype], F=0, head=head)
    embd = bd.to_device(emb)
    note(f"[gpu] fused tokenizer {dtype} B={B} T={T} D={D} F={F} {kinds}")
    a = bd.rm_model_fwd(fused, embd, want_x=True, want_pooled=True)
    x0 = bd.rm_tokenize_padsplit(embd, T, D, DT[dtype])
    b = bd.rm_model_fwd(plain, x0, want_x=True, want_pooled=True)
    torch.cuda.synchronize()
    for k in ("x", "pooled", "logit"):
        assert torch.equal(a[k], b[k]), k
    if B <= 100:
        ref = orc.model_fwd(emb, np_blocks, T, D, dtype, F, {"w": head_w, "c": head["c"]})
        assert rel_l2_rows(host(a["x"]), ref["x"]) <= TOL[dtype]

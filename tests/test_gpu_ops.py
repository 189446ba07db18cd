"""GPU parity of the single operations against the fp64 oracle, through the
C ABI: token mix and tokenizer bit-exact, per-token FFN and MoE within the
dtype tolerance, MoE routing lists checked for validity."""
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


def _rand(shape, dtype, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    t = torch.from_numpy(x).to(DT[dtype])
    return t


# --------------------------------------------------------------------------
# token mixing


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,T,D", [(3, 2, 8), (5, 4, 64), (7, 16, 320), (3, 5, 40), (2, 3, 9), (2, 32, 1536),
                                   (1, 1, 24), (65, 16, 768)])
def test_token_mix_bit_exact(dtype, B, T, D):
    from rankmixer_token_mixing_amd import binding as bd
    x = _rand((B, T, D), dtype, B * 1000 + T * 10 + D)
    y = bd.rm_token_mix(x.cuda())
    ref = orc.token_mix(x.to(torch.float64).numpy())
    np.testing.assert_array_equal(host(y), ref)
    z = bd.rm_token_mix(y)
    assert torch.equal(z.cpu(), x)  # involution, bit for bit


def test_token_mix_golden():
    import json, os
    from rankmixer_token_mixing_amd import binding as bd
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "token_mix_T3_D6.json")))
    x = torch.tensor([g["x"]], dtype=torch.float32).cuda()
    np.testing.assert_array_equal(host(bd.rm_token_mix(x))[0], np.array(g["mixed"]))


# --------------------------------------------------------------------------
# pad-split tokenizer


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,F,T,D", [(5, 5000, 16, 320), (3, 37, 4, 10), (2, 64, 4, 16), (3, 13, 3, 5),
                                     (4, 5120, 32, 160)])
def test_tokenizer_bit_exact(dtype, B, F, T, D):
    from rankmixer_token_mixing_amd import binding as bd
    emb = (np.random.default_rng(F).standard_normal((B, F)) * math.sqrt(0.1)).astype(np.float32)
    x0 = bd.rm_tokenize_padsplit(torch.from_numpy(emb).cuda(), T, D, DT[dtype])
    np.testing.assert_array_equal(host(x0), orc.tokenize_padsplit(emb, T, D, dtype))


# --------------------------------------------------------------------------
# projection tokenizer


def _proj_params(T, D, seg, dtype, seed, bias=0.1):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((T, D, seg)) / math.sqrt(seg)).astype(np.float32)
    p = {"w": si.to_bf16_bits(w) if dtype == "bf16" else w,
         "b": (bias * rng.standard_normal((T, D))).astype(np.float32)}
    return p


def _proj_dev(p):
    from rankmixer_token_mixing_amd.binding import to_device
    return {k: to_device(v) for k, v in p.items()}


@pytest.mark.parametrize("dtype,B,F,T,seg,D", [
    ("bf16", 4096, 5000, 16, 320, 320),  # the pad-split model's embedding, seg = 320 (313 rounded up to 8)
    ("bf16", 600, 4000, 32, 128, 256),   # full k tiles, N = one tile, ragged M
    ("bf16", 300, 1000, 8, 128, 136),    # N = 136: a partial N tile
    ("bf16", 1, 37, 4, 16, 8),           # one sample, F % 4 != 0: pad-split copy + product
    ("bf16", 257, 4998, 16, 320, 320),   # F % 4 != 0 at the workload's width
    ("bf16", 130, 20, 4, 8, 64),         # segments 3 and 4 entirely padding, K = 8
    ("f32", 70, 300, 4, 80, 64),         # fp32, K = 80: a partial k tile
    ("f32", 5, 5, 2, 8, 16),             # F < seg: the second segment is all padding
])
def test_projection_tokenizer_matches_oracle(dtype, B, F, T, seg, D):
    from rankmixer_token_mixing_amd import binding as bd
    rng = np.random.default_rng(F + seg)
    emb = (rng.standard_normal((B, F)) * math.sqrt(0.1)).astype(np.float32)
    p = _proj_params(T, D, seg, dtype, seed=B + D)
    note(f"[gpu] rm_tokenize_project {dtype} B={B} F={F} T={T} seg={seg} D={D}")
    x0 = host(bd.rm_tokenize_project(torch.from_numpy(emb).cuda(), _proj_dev(p), T, seg, DT[dtype]))
    rows = si.random_rows(B, 64, seed=7)
    ref = orc.tokenize_project(emb[rows], p["w"], p["b"], T, seg, dtype)
    assert rel_l2_rows(x0[rows], ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_projection_tokenizer_identity_is_padsplit(dtype):
    # W_t = I (seg = D), b = 0: every output is one exact product, so the
    # result equals the pad-split tokenizer bit for bit
    from rankmixer_token_mixing_amd import binding as bd
    B, F, T, D = 260, 1000, 8, 128
    emb = torch.from_numpy((np.random.default_rng(9).standard_normal((B, F)) * 0.3).astype(np.float32)).cuda()
    eye = np.broadcast_to(np.eye(D, dtype=np.float32), (T, D, D)).copy()
    p = {"w": si.to_bf16_bits(eye) if dtype == "bf16" else eye, "b": np.zeros((T, D), np.float32)}
    x0 = bd.rm_tokenize_project(emb, _proj_dev(p), T, D, DT[dtype])
    assert torch.equal(x0, bd.rm_tokenize_padsplit(emb, T, D, DT[dtype]))


def test_projection_tokenizer_locality():
    # changing the floats of segment 2 changes token 2 only
    from rankmixer_token_mixing_amd import binding as bd
    B, F, T, seg, D = 64, 500, 4, 128, 64
    emb = torch.from_numpy((np.random.default_rng(2).standard_normal((B, F)) * 0.3).astype(np.float32)).cuda()
    p = _proj_dev(_proj_params(T, D, seg, "bf16", seed=4))
    x = bd.rm_tokenize_project(emb, p, T, seg)
    emb2 = emb.clone()
    emb2[:, 2 * seg:2 * seg + 40] += 1.0
    x2 = bd.rm_tokenize_project(emb2, p, T, seg)
    diff = (x2.float() - x.float()).abs().amax(dim=(0, 2)).cpu()
    assert diff[2] > 0 and torch.all(diff[[0, 1, 3]] == 0)


# --------------------------------------------------------------------------
# per-token FFN


def _dense_params(T, D, Hd, dtype, seed, bias=0.1):
    rng = np.random.default_rng(seed)
    p = {
        "w1": (rng.standard_normal((T, Hd, D)) / math.sqrt(D)).astype(np.float32),
        "b1": (bias * rng.standard_normal((T, Hd))).astype(np.float32),
        "w2": (rng.standard_normal((T, D, Hd)) / math.sqrt(Hd)).astype(np.float32),
        "b2": (bias * rng.standard_normal((T, D))).astype(np.float32),
        "ln1_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln1_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln2_g": (1 + 0.1 * rng.standard_normal(D)).astype(np.float32),
        "ln2_b": (0.1 * rng.standard_normal(D)).astype(np.float32),
    }
    if dtype == "bf16":
        for k in ("w1", "w2"):
            p[k] = si.to_bf16_bits(p[k])
    return p


def _dev(p):
    from rankmixer_token_mixing_amd.binding import upload_blocks
    return upload_blocks([p])[0]


@pytest.mark.parametrize("dtype,B,T,D,Hd", [
    ("f32", 64, 4, 64, 128),     # the tiny fp32 block's shapes
    ("f32", 70, 3, 64, 96),      # ragged M and N tiles
    ("bf16", 300, 4, 128, 320),  # ragged M, N = 2.5 tiles
    ("bf16", 130, 4, 72, 88),    # K = 72: a partial k tile
    ("bf16", 1, 2, 16, 24),      # one sample
    ("bf16", 520, 2, 256, 1024),  # several full 256 x 256 tiles
])
def test_pffn_matches_oracle(dtype, B, T, D, Hd):
    from rankmixer_token_mixing_amd import binding as bd
    p = _dense_params(T, D, Hd, dtype, seed=B + D)
    s = _rand((B, T, D), dtype, seed=Hd)
    v = bd.rm_pffn_fwd(s.cuda(), _dev(p))
    ref = orc.pffn(s.to(torch.float64).numpy(), p["w1"], p["b1"], p["w2"], p["b2"])
    assert rel_l2_rows(host(v), ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pffn_token_locality(dtype):
    from rankmixer_token_mixing_amd import binding as bd
    T, D, Hd, B = 4, 64, 128, 32
    p = _dev(_dense_params(T, D, Hd, dtype, seed=3))
    s = _rand((B, T, D), dtype, 4).cuda()
    v = bd.rm_pffn_fwd(s, p)
    s2 = s.clone()
    s2[:, 1] += 1.0
    v2 = bd.rm_pffn_fwd(s2, p)
    diff = (v2.float() - v.float()).abs().amax(dim=(0, 2)).cpu()
    assert diff[1] > 0 and torch.all(diff[[0, 2, 3]] == 0)


# --------------------------------------------------------------------------
# MoE


def _moe_params(T, D, E, He, dtype, seed, bias=-0.6745):
    rng = np.random.default_rng(seed)
    p = {
        "w1": (rng.standard_normal((T, E, He, D)) / math.sqrt(D)).astype(np.float32),
        "b1": (0.1 * rng.standard_normal((T, E, He))).astype(np.float32),
        "w2": (rng.standard_normal((T, E, D, He)) / math.sqrt(He)).astype(np.float32),
        "b2": (0.1 * rng.standard_normal((T, E, D))).astype(np.float32),
        "wr": (rng.standard_normal((T, E, D)) / math.sqrt(D)).astype(np.float32),
        "br": np.full((T, E), bias, np.float32),
    }
    if dtype == "bf16":
        for k in ("w1", "w2", "wr"):
            p[k] = si.to_bf16_bits(p[k])
    return p


@pytest.mark.parametrize("dtype,B,T,D,E,He", [
    ("f32", 100, 4, 64, 4, 96),
    ("bf16", 300, 4, 128, 8, 256),
    ("bf16", 5, 2, 64, 3, 64),
])
def test_moe_matches_oracle(dtype, B, T, D, E, He):
    from rankmixer_token_mixing_amd import binding as bd
    p = _moe_params(T, D, E, He, dtype, seed=B + E)
    s_np = orc.layer_norm(np.random.default_rng(7).standard_normal((B, T, D)), np.ones(D), np.zeros(D))
    s = torch.from_numpy(s_np.astype(np.float32)).to(DT[dtype])
    v, gates = bd.rm_moe_relu_fwd(s.cuda(), _dev(p), return_gates=True)
    V_ref, G_ref = orc.moe_relu_pffn(s.to(torch.float64).numpy(), **{k: p[k] for k in ("w1", "b1", "w2", "b2", "wr", "br")})
    assert rel_l2_rows(host(v), V_ref) <= TOL[dtype]
    assert np.abs(host(gates) - G_ref).max() <= (1e-5 if dtype == "f32" else 1e-4)
    assert 0.05 < (G_ref > 0).mean() < 0.6


def test_moe_route_lists_are_valid_and_stable():
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, E = 777, 4, 64, 8
    p = _moe_params(T, D, E, 64, "bf16", seed=11)
    s = _rand((B, T, D), "bf16", 12).cuda()
    dp = _dev(p)
    gates, offsets, rows = bd.rm_moe_route(s, dp["wr"], dp["br"])
    g = host(gates).reshape(B, T * E)
    off = offsets.cpu().numpy()
    r = rows.cpu().numpy()
    assert off[0] == 0 and np.all(np.diff(off) >= 0)
    for grp in range(T * E):
        expect = np.nonzero(g[:, grp] > 0)[0]
        np.testing.assert_array_equal(r[off[grp]:off[grp + 1]], expect)
    # where the fp64 router output z is clearly away from 0, the decision agrees
    S64 = s.to(torch.float64).cpu().numpy()
    z = (orc.moe_gates(S64, p["wr"], p["br"]) - orc.moe_gates(S64, -orc.as_f64(p["wr"]), -p["br"])).reshape(B, T * E)
    clear = np.abs(z) > 1e-3
    np.testing.assert_array_equal((g > 0)[clear], (z > 0)[clear])


def test_moe_zero_gates_give_zero():
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, E, He = 64, 4, 64, 4, 64
    p = _moe_params(T, D, E, He, "bf16", seed=5, bias=-1e4)
    s = _rand((B, T, D), "bf16", 6).cuda()
    v, gates = bd.rm_moe_relu_fwd(s, _dev(p), return_gates=True)
    assert torch.all(gates == 0) and torch.all(v == 0)


def test_moe_single_expert_always_on_equals_pffn():
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, He = 96, 4, 64, 128
    p = _moe_params(T, D, 1, He, "f32", seed=8, bias=1.0)
    p["wr"][:] = 0.0
    s = _rand((B, T, D), "f32", 9).cuda()
    v = bd.rm_moe_relu_fwd(s, _dev(p))
    dense = {"w1": p["w1"][:, 0].copy(), "b1": p["b1"][:, 0].copy(), "w2": p["w2"][:, 0].copy(),
             "b2": p["b2"][:, 0].copy()}
    v2 = bd.rm_pffn_fwd(s, _dev(dense))
    assert rel_l2_rows(host(v), host(v2)) <= 1e-6


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_moe_groups_of_every_size(dtype):
    # expert groups of every size class: router biases spread the densities
    # from ~3 % to ~97 %, so group counts (B = 1100) land on both sides of
    # every 256-row tile boundary, with short and long last tiles
    from rankmixer_token_mixing_amd import binding as bd
    B, T, D, E, He = 1100, 4, 128, 8, 256
    p = _moe_params(T, D, E, He, dtype, seed=21)
    p["br"] = np.linspace(-1.9, 1.9, T * E).reshape(T, E).astype(np.float32)
    s_np = orc.layer_norm(np.random.default_rng(22).standard_normal((B, T, D)), np.ones(D), np.zeros(D))
    s = torch.from_numpy(s_np.astype(np.float32)).to(DT[dtype])
    v, gates = bd.rm_moe_relu_fwd(s.cuda(), _dev(p), return_gates=True)
    torch.cuda.synchronize()
    counts = (host(gates) > 0).reshape(B, T * E).sum(axis=0)
    rem = counts % 256
    assert ((rem > 0) & (rem <= 128)).sum() >= 4 and (rem > 128).sum() >= 4, counts
    rows = si.random_rows(B, 64, seed=23)
    V_ref, _ = orc.moe_relu_pffn(s.to(torch.float64).numpy()[rows], **{k: p[k] for k in ("w1", "b1", "w2", "b2", "wr", "br")})
    assert rel_l2_rows(host(v)[rows], V_ref) <= TOL[dtype]

"""Pins of the fp64 oracle against things other than itself: worked examples,
closed forms, library routines the method reduces to in special cases,
invariants the pages state, and brute-force index loops on tiny shapes.

Each test names the passage it follows.  A plausible slip in the oracle (a
dropped residual or bias, a transposed weight, a wrong head index, a wrong
GELU form, a missing epsilon) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import rankmixer_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _torch_float64():
    """torch references in this module compute in fp64, like the oracle; the
    default dtype is restored for the modules after it."""
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(old)


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# token mixing ("Rankmixer: 硬件效率优化", section "Token Mixing机制")


@pytest.mark.parametrize("name", ["token_mix_T2_D4.json", "token_mix_T3_D6.json"])
def test_token_mix_worked_examples(name):
    g = _golden(name)
    x = np.array(g["x"], dtype=np.float64)[None]
    got = orc.token_mix(x)[0]
    np.testing.assert_array_equal(got, np.array(g["mixed"], dtype=np.float64))


@pytest.mark.parametrize("T,D", [(1, 8), (2, 4), (4, 64), (16, 320), (5, 35), (8, 8)])
def test_token_mix_is_the_head_token_transpose(T, D):
    # SplitHead + Concat with H = T is the [T, H, D/H] -> [H, T, D/H] transpose
    # of each sample; torch.permute is an independent routine for it.
    x = _rng(T * 100 + D).standard_normal((3, T, D))
    ref = torch.from_numpy(x).reshape(3, T, T, D // T).permute(0, 2, 1, 3).reshape(3, T, D).numpy()
    np.testing.assert_array_equal(orc.token_mix(x), ref)


@pytest.mark.parametrize("T,D", [(2, 4), (4, 64), (16, 768), (32, 1536), (3, 9)])
def test_token_mix_involution_and_permutation(T, D):
    x = _rng(T + D).standard_normal((2, T, D))
    m = orc.token_mix(x)
    np.testing.assert_array_equal(orc.token_mix(m), x)          # TM(TM(X)) = X when H = T
    np.testing.assert_array_equal(np.sort(m.reshape(2, -1)), np.sort(x.reshape(2, -1)))


def test_token_mix_T1_is_identity():
    x = _rng(1).standard_normal((4, 1, 16))
    np.testing.assert_array_equal(orc.token_mix(x), x)


def test_token_mix_rejects_indivisible_width():
    with pytest.raises(ValueError):
        orc.token_mix(np.zeros((1, 3, 10)))


# --------------------------------------------------------------------------
# LayerNorm, GELU, bf16 rounding: library routines and closed forms


def test_layer_norm_matches_torch():
    rng = _rng(2)
    y = rng.standard_normal((5, 7, 48)) * 3 + 1.5
    g = rng.standard_normal(48)
    b = rng.standard_normal(48)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(y), (48,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(orc.layer_norm(y, g, b), ref, rtol=0, atol=1e-12)


def test_layer_norm_output_statistics():
    # gamma = 1, beta = 0: each row has mean 0 and variance var/(var+eps)
    y = _rng(3).standard_normal((64, 256)) * 0.01
    out = orc.layer_norm(y, np.ones(256), np.zeros(256))
    var_in = y.var(axis=1)
    np.testing.assert_allclose(out.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(out.var(axis=1), var_in / (var_in + 1e-5), rtol=1e-10)


def test_gelu_closed_forms_and_torch():
    # GELU(x) = x Phi(x): Phi(1) = 0.8413447460685429, Phi(-1) = 1 - Phi(1)
    assert orc.gelu(np.array([0.0]))[0] == 0.0
    assert abs(orc.gelu(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15
    assert abs(orc.gelu(np.array([-1.0]))[0] + 0.15865525393145707) < 1e-15
    assert abs(orc.gelu(np.array([10.0]))[0] - 10.0) < 1e-12
    assert abs(orc.gelu(np.array([-10.0]))[0]) < 1e-12
    x = np.linspace(-8, 8, 20001)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(orc.gelu(x), ref, rtol=1e-14, atol=1e-15)
    # the tanh approximation differs by more than the fp32 bar: the form matters
    tanh = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.abs(orc.gelu(x) - tanh).max() > 1e-4


def test_round_to_bf16_matches_torch():
    rng = _rng(4)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.0e38], dtype=np.float32),
    ])
    # exact ties: 8-bit significand + a half ulp, both parities
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    x = np.concatenate([x, (ties + np.uint32(0x3F800000 - (1 << 16))).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_to_bf16(x.astype(np.float64)), ref)


def test_bf16_bit_decoding():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F], dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.as_f64(bits), ref)


# --------------------------------------------------------------------------
# pad-split tokenizer ("淘宝闪购-爆品团精排 Scaling Up 迭代实践", section 3.4)


def test_padsplit_layout_and_padding():
    g = _golden("padsplit_shapes.json")
    F = g["embedding_floats"]
    for T, D in g["splits"]:
        assert T * D == g["padded_width"]
        emb = (np.arange(2 * F, dtype=np.float32).reshape(2, F) + 1.0) / 64.0
        x0 = orc.tokenize_padsplit(emb, T, D, "f32")
        flat = x0.reshape(2, T * D)
        np.testing.assert_array_equal(flat[:, :F], emb)
        assert np.all(flat[:, F:] == 0.0)
        assert (flat[0] == 0).sum() == T * D - F
        # token t holds floats [t*D, (t+1)*D)
        np.testing.assert_array_equal(x0[1, 3], emb[1, 3 * D:4 * D])


def test_padsplit_bf16_cast_is_torch_rne():
    emb = (_rng(5).standard_normal((3, 5000)) * math.sqrt(0.1)).astype(np.float32)
    x0 = orc.tokenize_padsplit(emb, 16, 320, "bf16")
    ref = torch.from_numpy(emb).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(x0.reshape(3, -1)[:, :5000], ref)


def test_padsplit_rejects_overlong():
    with pytest.raises(ValueError):
        orc.tokenize_padsplit(np.zeros((1, 10), np.float32), 2, 4, "f32")


# --------------------------------------------------------------------------
# per-token FFN ("Rankmixer: 硬件效率优化", section "Per-Token FFN")


def _dense_params(rng, T, D, Hd, bias=True):
    p = {
        "w1": rng.standard_normal((T, Hd, D)) / math.sqrt(D),
        "b1": rng.standard_normal((T, Hd)) * 0.1 if bias else np.zeros((T, Hd)),
        "w2": rng.standard_normal((T, D, Hd)) / math.sqrt(Hd),
        "b2": rng.standard_normal((T, D)) * 0.1 if bias else np.zeros((T, D)),
        "ln1_g": 1 + 0.1 * rng.standard_normal(D), "ln1_b": 0.1 * rng.standard_normal(D),
        "ln2_g": 1 + 0.1 * rng.standard_normal(D), "ln2_b": 0.1 * rng.standard_normal(D),
    }
    return p


def _torch_ffn(w1, b1, w2, b2):
    D = w1.shape[1]
    Hd = w1.shape[0]
    l1 = torch.nn.Linear(D, Hd)
    l2 = torch.nn.Linear(Hd, D)
    with torch.no_grad():
        l1.weight.copy_(torch.from_numpy(w1)); l1.bias.copy_(torch.from_numpy(b1))
        l2.weight.copy_(torch.from_numpy(w2)); l2.bias.copy_(torch.from_numpy(b2))
    return torch.nn.Sequential(l1, torch.nn.GELU(approximate="none"), l2)


def test_pffn_with_equal_weights_is_a_shared_ffn():
    # all W_t, b_t equal => the textbook FFN applied to every token
    rng = _rng(6)
    T, D, Hd = 5, 12, 20
    p = _dense_params(rng, 1, D, Hd)
    rep = {k: np.repeat(p[k], T, axis=0) for k in ("w1", "b1", "w2", "b2")}
    s = rng.standard_normal((4, T, D))
    ffn = _torch_ffn(p["w1"][0], p["b1"][0], p["w2"][0], p["b2"][0])
    with torch.no_grad():
        ref = ffn(torch.from_numpy(s)).numpy()
    np.testing.assert_allclose(orc.pffn(s, **rep), ref, rtol=1e-12, atol=1e-12)


def test_pffn_token_t_uses_only_its_own_weights():
    # each token t through the textbook FFN with (W1_t, b1_t, W2_t, b2_t)
    rng = _rng(7)
    T, D, Hd = 4, 8, 24
    p = _dense_params(rng, T, D, Hd)
    s = rng.standard_normal((3, T, D))
    got = orc.pffn(s, p["w1"], p["b1"], p["w2"], p["b2"])
    for t in range(T):
        ffn = _torch_ffn(p["w1"][t], p["b1"][t], p["w2"][t], p["b2"][t])
        with torch.no_grad():
            ref = ffn(torch.from_numpy(s[:, t])).numpy()
        np.testing.assert_allclose(got[:, t], ref, rtol=1e-12, atol=1e-12)


def test_pffn_locality():
    # perturbing s_t changes v_t only ("each FFN sees only its own token")
    rng = _rng(8)
    T, D, Hd = 6, 12, 24
    p = _dense_params(rng, T, D, Hd)
    s = rng.standard_normal((2, T, D))
    v = orc.pffn(s, p["w1"], p["b1"], p["w2"], p["b2"])
    s2 = s.copy()
    s2[:, 2] += rng.standard_normal((2, D))
    v2 = orc.pffn(s2, p["w1"], p["b1"], p["w2"], p["b2"])
    changed = np.abs(v2 - v).max(axis=(0, 2)) > 0
    assert changed.tolist() == [t == 2 for t in range(T)]


# --------------------------------------------------------------------------
# brute force: every index written out, scalar math only


def _bf_block(x, p, moe=None, swiglu=False, no_mix_norm=False):
    B, T, D = x.shape
    d = D // T

    def ln(row, g, b):
        mu = sum(row) / len(row)
        var = sum((v - mu) ** 2 for v in row) / len(row)
        return [(v - mu) / math.sqrt(var + 1e-5) * g[i] + b[i] for i, v in enumerate(row)]

    def gel(v):
        return 0.5 * v * (1 + math.erf(v / math.sqrt(2)))

    out = np.zeros((B, T, D))
    for b in range(B):
        S = []
        for t in range(T):
            # element k of mixed token t is element (t*d + k%d) of token k//d
            if no_mix_norm:
                S.append([x[b, k // d, t * d + k % d] for k in range(D)])
            else:
                row = [x[b, k // d, t * d + k % d] + x[b, t, k] for k in range(D)]
                S.append(ln(row, p["ln1_g"], p["ln1_b"]))
        for t in range(T):
            s = S[t]
            if swiglu:
                Hs = p["w1"].shape[1] // 2
                gate = [sum(p["w1"][t, n, k] * s[k] for k in range(D)) + p["b1"][t, n] for n in range(Hs)]
                up = [sum(p["w1"][t, Hs + n, k] * s[k] for k in range(D)) + p["b1"][t, Hs + n] for n in range(Hs)]
                h = [gate[n] / (1 + math.exp(-gate[n])) * up[n] for n in range(Hs)]
                v = [sum(p["w2"][t, k, n] * h[n] for n in range(Hs)) + p["b2"][t, k] for k in range(D)]
            elif moe is None:
                Hd = p["w1"].shape[1]
                h = [gel(sum(p["w1"][t, n, k] * s[k] for k in range(D)) + p["b1"][t, n]) for n in range(Hd)]
                v = [sum(p["w2"][t, k, n] * h[n] for n in range(Hd)) + p["b2"][t, k] for k in range(D)]
            else:
                E = moe["w1"].shape[1]
                He = moe["w1"].shape[2]
                v = [0.0] * D
                for j in range(E):
                    g = max(0.0, sum(moe["wr"][t, j, k] * s[k] for k in range(D)) + moe["br"][t, j])
                    h = [gel(sum(moe["w1"][t, j, n, k] * s[k] for k in range(D)) + moe["b1"][t, j, n])
                         for n in range(He)]
                    for k in range(D):
                        y = sum(moe["w2"][t, j, k, n] * h[n] for n in range(He)) + moe["b2"][t, j, k]
                        v[k] += g * y
            out[b, t] = ln([v[k] + s[k] for k in range(D)], p["ln2_g"], p["ln2_b"])
    return out


@pytest.mark.parametrize("T,D,Hd", [(1, 4, 8), (2, 4, 6), (4, 8, 16), (3, 6, 5)])
def test_block_matches_brute_force(T, D, Hd):
    rng = _rng(9 + T)
    p = _dense_params(rng, T, D, Hd)
    x = rng.standard_normal((2, T, D))
    np.testing.assert_allclose(orc.block_fwd(x, p), _bf_block(x, p), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,D,E,He", [(2, 4, 3, 5), (4, 8, 2, 6)])
def test_moe_block_matches_brute_force(T, D, E, He):
    rng = _rng(20 + T)
    p = _dense_params(rng, T, D, 4)
    moe = {
        "w1": rng.standard_normal((T, E, He, D)) / math.sqrt(D),
        "b1": 0.1 * rng.standard_normal((T, E, He)),
        "w2": rng.standard_normal((T, E, D, He)) / math.sqrt(He),
        "b2": 0.1 * rng.standard_normal((T, E, D)),
        "wr": rng.standard_normal((T, E, D)) / math.sqrt(D),
        "br": 0.2 * rng.standard_normal((T, E)),
    }
    blk = dict(p)
    blk.update(moe)
    x = rng.standard_normal((3, T, D))
    np.testing.assert_allclose(orc.block_fwd(x, blk), _bf_block(x, p, moe), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,D,Hs", [(1, 4, 6), (2, 4, 4), (4, 8, 12)])
def test_swiglu_block_matches_brute_force(T, D, Hs):
    # [TB] section 3.6: the SwiGLU per-token FFN in place of the GELU FFN
    rng = _rng(30 + T)
    p = _dense_params(rng, T, D, 2 * Hs)
    p["w2"] = rng.standard_normal((T, D, Hs)) / math.sqrt(Hs)
    p["swiglu"] = True
    x = rng.standard_normal((2, T, D))
    np.testing.assert_allclose(orc.block_fwd(x, p), _bf_block(x, p, swiglu=True), rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,D,Hd", [(2, 4, 6), (4, 8, 16)])
def test_no_mix_norm_block_matches_brute_force(T, D, Hd):
    # [TB] section 3.5: the block without the Add & Norm after the token mix
    rng = _rng(40 + T)
    p = _dense_params(rng, T, D, Hd)
    p["no_mix_norm"] = True
    x = rng.standard_normal((2, T, D))
    np.testing.assert_allclose(orc.block_fwd(x, p), _bf_block(x, p, no_mix_norm=True), rtol=0, atol=1e-12)


def test_silu_matches_torch_and_closed_forms():
    x = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(orc.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14,
                               atol=1e-300)
    assert orc.silu(0.0) == 0.0
    assert orc.silu(40.0) == pytest.approx(40.0, rel=1e-15)


def test_swiglu_with_constant_up_branch_is_a_silu_ffn():
    # Wu = 0, bu = 1: SwiGLU(s) = W2 SiLU(Wg s + bg) + b2, a plain FFN with SiLU (torch layers)
    rng = _rng(50)
    T, D, Hs = 3, 8, 10
    w1 = np.concatenate([rng.standard_normal((T, Hs, D)), np.zeros((T, Hs, D))], axis=1)
    b1 = np.concatenate([rng.standard_normal((T, Hs)), np.ones((T, Hs))], axis=1)
    w2 = rng.standard_normal((T, D, Hs))
    b2 = rng.standard_normal((T, D))
    S = rng.standard_normal((4, T, D))
    got = orc.swiglu_pffn(S, w1, b1, w2, b2)
    for t in range(T):
        with torch.no_grad():
            h = torch.nn.functional.silu(torch.from_numpy(S[:, t]) @ torch.from_numpy(w1[t, :Hs]).T
                                         + torch.from_numpy(b1[t, :Hs]))
            ref = h @ torch.from_numpy(w2[t]).T + torch.from_numpy(b2[t])
        np.testing.assert_allclose(got[:, t], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_no_mix_norm_T1_block_is_ffn_plus_residual_then_norm():
    # T = 1 and no Add & Norm after the mix: S = X, X' = LN2(FFN(X) + X)
    rng = _rng(51)
    D, Hd = 16, 24
    p = _dense_params(rng, 1, D, Hd)
    p["no_mix_norm"] = True
    x = rng.standard_normal((5, 1, D))
    ffn = _torch_ffn(p["w1"][0], p["b1"][0], p["w2"][0], p["b2"][0])
    with torch.no_grad():
        xt = torch.from_numpy(x[:, 0])
        ref = torch.nn.functional.layer_norm(ffn(xt) + xt, (D,), torch.from_numpy(p["ln2_g"]),
                                             torch.from_numpy(p["ln2_b"]), 1e-5)
    np.testing.assert_allclose(orc.block_fwd(x, p)[:, 0], ref.numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# whole-block special cases


def test_block_T1_is_a_post_ln_ffn_block():
    # T = 1: the mix is the identity, so X' = LN2(FFN(LN1(2X)) + LN1(2X))
    rng = _rng(10)
    D, Hd = 16, 40
    p = _dense_params(rng, 1, D, Hd)
    x = rng.standard_normal((5, 1, D))
    ffn = _torch_ffn(p["w1"][0], p["b1"][0], p["w2"][0], p["b2"][0])
    F = torch.nn.functional
    with torch.no_grad():
        xt = torch.from_numpy(x[:, 0])
        s = F.layer_norm(2 * xt, (D,), torch.from_numpy(p["ln1_g"]), torch.from_numpy(p["ln1_b"]), 1e-5)
        ref = F.layer_norm(ffn(s) + s, (D,), torch.from_numpy(p["ln2_g"]), torch.from_numpy(p["ln2_b"]), 1e-5)
    np.testing.assert_allclose(orc.block_fwd(x, p)[:, 0], ref.numpy(), rtol=0, atol=1e-12)


def test_block_first_ln_sees_mix_plus_residual():
    # with W2 = 0 and b2 = 0 the block is LN2(S) with S = LN1(TM(X) + X);
    # the transpose form of TM is taken from torch
    rng = _rng(11)
    T, D, Hd = 4, 16, 8
    p = _dense_params(rng, T, D, Hd)
    p["w2"] = np.zeros_like(p["w2"])
    p["b2"] = np.zeros_like(p["b2"])
    x = rng.standard_normal((3, T, D)) + 0.5
    F = torch.nn.functional
    xt = torch.from_numpy(x)
    mixed = xt.reshape(3, T, T, D // T).permute(0, 2, 1, 3).reshape(3, T, D)
    s = F.layer_norm(mixed + xt, (D,), torch.from_numpy(p["ln1_g"]), torch.from_numpy(p["ln1_b"]), 1e-5)
    ref = F.layer_norm(s, (D,), torch.from_numpy(p["ln2_g"]), torch.from_numpy(p["ln2_b"]), 1e-5)
    np.testing.assert_allclose(orc.block_fwd(x, p), ref.numpy(), rtol=0, atol=1e-12)


def test_block_mixing_spreads_a_token_to_all_tokens():
    rng = _rng(12)
    T, D, Hd = 4, 16, 32
    p = _dense_params(rng, T, D, Hd)
    x = rng.standard_normal((1, T, D))
    y = orc.block_fwd(x, p)
    x2 = x.copy()
    x2[0, 1] += 0.5
    y2 = orc.block_fwd(x2, p)
    assert np.all(np.abs(y2 - y).max(axis=2) > 1e-6)


# --------------------------------------------------------------------------
# ReLU-gated MoE ("Rankmixer: 硬件效率优化", section "Sparse MoE扩展")


def _moe(rng, T, D, E, He):
    return {
        "w1": rng.standard_normal((T, E, He, D)) / math.sqrt(D),
        "b1": 0.1 * rng.standard_normal((T, E, He)),
        "w2": rng.standard_normal((T, E, D, He)) / math.sqrt(He),
        "b2": 0.1 * rng.standard_normal((T, E, D)),
        "wr": rng.standard_normal((T, E, D)) / math.sqrt(D),
        "br": 0.2 * rng.standard_normal((T, E)),
    }


def test_moe_zero_gates_contribute_nothing():
    rng = _rng(13)
    T, D, E, He = 4, 16, 3, 12
    m = _moe(rng, T, D, E, He)
    m["br"][:] = -1e4
    s = rng.standard_normal((5, T, D))
    V, G = orc.moe_relu_pffn(s, **m)
    assert np.all(G == 0) and np.all(V == 0)
    p = _dense_params(rng, T, D, 4)
    blk = dict(p); blk.update(m)
    x = rng.standard_normal((5, T, D))
    S = orc.layer_norm(orc.token_mix(x) + x, p["ln1_g"], p["ln1_b"])
    np.testing.assert_allclose(orc.block_fwd(x, blk), orc.layer_norm(S, p["ln2_g"], p["ln2_b"]), atol=1e-12)


def test_moe_single_always_on_expert_is_the_pffn():
    rng = _rng(14)
    T, D, He = 3, 8, 16
    m = _moe(rng, T, D, 1, He)
    m["wr"][:] = 0.0
    m["br"][:] = 1.0
    s = rng.standard_normal((4, T, D))
    V, G = orc.moe_relu_pffn(s, **m)
    assert np.all(G == 1.0)
    ref = orc.pffn(s, m["w1"][:, 0], m["b1"][:, 0], m["w2"][:, 0], m["b2"][:, 0])
    np.testing.assert_allclose(V, ref, atol=1e-12)


def test_moe_positive_homogeneity_of_the_router():
    rng = _rng(15)
    T, D, E, He = 4, 16, 5, 8
    m = _moe(rng, T, D, E, He)
    s = rng.standard_normal((6, T, D))
    V1, G1 = orc.moe_relu_pffn(s, **m)
    m2 = dict(m); m2["wr"] = 2.5 * m["wr"]; m2["br"] = 2.5 * m["br"]
    V2, G2 = orc.moe_relu_pffn(s, **m2)
    np.testing.assert_allclose(G2, 2.5 * G1, atol=1e-12)
    np.testing.assert_allclose(V2, 2.5 * V1, atol=1e-11)
    assert (G1 > 0).any() and (G1 == 0).any()


def test_moe_gate_density_of_the_router_bias_recipe():
    # router N(0, 1/D), unit-variance input, bias -Phi^-1(0.75): about 25 % on
    from synthetic_inputs import MOE_ROUTER_BIAS
    rng = _rng(16)
    T, D, E = 4, 768, 8
    s = orc.layer_norm(rng.standard_normal((512, T, D)), np.ones(D), np.zeros(D))
    wr = rng.standard_normal((T, E, D)) / math.sqrt(D)
    G = orc.moe_gates(s, wr, np.full((T, E), MOE_ROUTER_BIAS))
    assert 0.22 < (G > 0).mean() < 0.28


# --------------------------------------------------------------------------
# pooling and logit


def test_mean_pool_and_logit_match_torch():
    rng = _rng(17)
    x = rng.standard_normal((7, 16, 20))
    w = rng.standard_normal(20)
    p = orc.mean_pool(x)
    np.testing.assert_allclose(p, torch.from_numpy(x).mean(dim=1).numpy(), atol=1e-14)
    lin = torch.nn.Linear(20, 1)
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(w)[None]); lin.bias.fill_(0.25)
        ref = lin(torch.from_numpy(p))[:, 0].numpy()
    blocks = []
    out = orc.model_fwd(x, blocks, 16, 20, "f32", head={"w": w, "c": 0.25})
    np.testing.assert_allclose(out["logit"], ref, atol=1e-12)


def test_model_stacks_blocks_in_order():
    rng = _rng(18)
    T, D, Hd = 2, 8, 12
    p1 = _dense_params(rng, T, D, Hd)
    p2 = _dense_params(rng, T, D, Hd)
    x = rng.standard_normal((3, T, D))
    out = orc.model_fwd(x, [p1, p2], T, D, "f32")["x"]
    np.testing.assert_allclose(out, _bf_block(_bf_block(x, p1), p2), atol=1e-12)
    # order matters
    assert np.abs(out - orc.model_fwd(x, [p2, p1], T, D, "f32")["x"]).max() > 1e-6


def test_subset_rows_give_the_same_outputs():
    # samples never interact: the oracle on a subset equals the full run's rows
    rng = _rng(19)
    T, D, Hd = 4, 16, 8
    p = _dense_params(rng, T, D, Hd)
    x = rng.standard_normal((10, T, D))
    full = orc.model_fwd(x, [p], T, D, "f32")["x"]
    part = orc.model_fwd(x[[0, 3, 9]], [p], T, D, "f32")["x"]
    np.testing.assert_array_equal(full[[0, 3, 9]], part)


# ---------------------------------------------------------------------------
# projection tokenizer ([WL] "特征的Tokenization")

def test_tokenize_project_hand_worked_example():
    g = _golden("tokenize_project_T2_seg2.json")
    x0 = orc.tokenize_project(np.array(g["emb"], np.float32), np.array(g["w"]), np.array(g["b"]), g["T"], g["seg"],
                              "f32")
    np.testing.assert_allclose(x0, np.array(g["x0"]), rtol=0, atol=1e-12)


def test_tokenize_project_with_identity_weights_is_padsplit():
    # seg = D and W_t = I, b = 0: each token is its own segment, i.e. the
    # pad-split tokenizer (pinned above against its own layout table)
    rng = np.random.default_rng(4)
    B, F, T, D = 3, 37, 5, 8
    emb = rng.standard_normal((B, F)).astype(np.float32)
    w = np.broadcast_to(np.eye(D), (T, D, D)).copy()
    for dt in ("f32", "bf16"):
        x0 = orc.tokenize_project(emb, w, np.zeros((T, D)), T, D, dt)
        np.testing.assert_array_equal(x0, orc.tokenize_padsplit(emb, T, D, dt))


def test_tokenize_project_brute_force_loops():
    rng = np.random.default_rng(5)
    B, F, T, seg, D = 2, 7, 3, 3, 2
    emb = rng.standard_normal((B, F)).astype(np.float32)
    w = rng.standard_normal((T, D, seg))
    b = rng.standard_normal((T, D))
    x0 = orc.tokenize_project(emb, w, b, T, seg, "f32")
    for bb in range(B):
        for t in range(T):
            for d in range(D):
                acc = b[t, d]
                for s in range(seg):
                    pos = t * seg + s  # position in the concatenated embedding
                    if pos < F:
                        acc += w[t, d, s] * float(emb[bb, pos])
                assert abs(x0[bb, t, d] - acc) < 1e-12


def test_tokenize_project_tokens_see_only_their_segment():
    rng = np.random.default_rng(6)
    B, F, T, seg, D = 2, 40, 4, 10, 6
    emb = rng.standard_normal((B, F)).astype(np.float32)
    w = rng.standard_normal((T, D, seg))
    b = rng.standard_normal((T, D))
    x0 = orc.tokenize_project(emb, w, b, T, seg, "f32")
    emb2 = emb.copy()
    emb2[:, 2 * seg:3 * seg] += 1.0  # segment 2 only
    x1 = orc.tokenize_project(emb2, w, b, T, seg, "f32")
    changed = np.abs(x1 - x0).max(axis=(0, 2)) > 0
    assert changed.tolist() == [False, False, True, False]


def test_tokenize_project_rejects_overlong():
    with pytest.raises(ValueError):
        orc.tokenize_project(np.zeros((1, 9), np.float32), np.zeros((2, 1, 4)), np.zeros((2, 1)), 2, 4, "f32")

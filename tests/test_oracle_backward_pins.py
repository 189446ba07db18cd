"""Pins of the backward oracle (oracle/block_backward.py) against things other
than itself: central finite differences of the forward oracle for every
gradient it returns, the invariants a LayerNorm input gradient must satisfy,
and closed forms of the GELU derivative.  A plausible slip (a dropped residual
branch, the token mix's transpose taken as something other than itself, a
transposed weight gradient, a missing 1/sigma, the tanh GELU) fails one of
them."""
import math

import numpy as np
import pytest

from oracle import block_backward as bw
from oracle import rankmixer_oracle as orc


def _block(T, D, Hd, seed):
    rng = np.random.default_rng(seed)
    return {
        "w1": rng.standard_normal((T, Hd, D)) / math.sqrt(D),
        "b1": 0.3 * rng.standard_normal((T, Hd)),
        "w2": rng.standard_normal((T, D, Hd)) / math.sqrt(Hd),
        "b2": 0.3 * rng.standard_normal((T, D)),
        "ln1_g": 1 + 0.3 * rng.standard_normal(D), "ln1_b": 0.3 * rng.standard_normal(D),
        "ln2_g": 1 + 0.3 * rng.standard_normal(D), "ln2_b": 0.3 * rng.standard_normal(D),
    }


def _loss(X, blk, d_out):
    return float((orc.block_fwd(X, blk) * d_out).sum())


def _fd(f, a, h=1e-6):
    """central differences of the scalar f() over every entry of array a
    (perturbed in place and restored)"""
    g = np.empty_like(a)
    flat = a.reshape(-1)
    gf = g.reshape(-1)
    for i in range(flat.size):
        x0 = flat[i]
        flat[i] = x0 + h
        fp = f()
        flat[i] = x0 - h
        fm = f()
        flat[i] = x0
        gf[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("B,T,D,Hd,seed", [(3, 2, 4, 6, 0), (2, 4, 8, 8, 1), (2, 1, 4, 4, 2)])
def test_every_gradient_matches_finite_differences(B, T, D, Hd, seed):
    # [FR] "RankMixer整体架构": the block is X' = LN(PFFN(S) + S), S = LN(TM(X) + X);
    # the loss L = sum(d_out * X') has dL/dX' = d_out
    rng = np.random.default_rng(seed + 10)
    X = rng.standard_normal((B, T, D))
    blk = _block(T, D, Hd, seed)
    d_out = rng.standard_normal((B, T, D))
    got = bw.block_bwd(X, blk, d_out)
    num = _fd(lambda: _loss(X, blk, d_out), X)
    np.testing.assert_allclose(got["dX"], num, rtol=1e-6, atol=1e-7)
    for k in ("w1", "b1", "w2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        num = _fd(lambda: _loss(X, blk, d_out), blk[k])
        np.testing.assert_allclose(got[k], num, rtol=1e-6, atol=1e-7, err_msg=k)


def test_layer_norm_input_gradient_invariants():
    # LN output is invariant to adding a constant to the row and (up to eps)
    # to scaling it, so the input gradient is orthogonal to 1 and to xhat
    rng = np.random.default_rng(3)
    Y = 2 + 3 * rng.standard_normal((5, 16))
    d = rng.standard_normal((5, 16))
    g = 1 + rng.standard_normal(16)
    dY, dg, db = bw.layer_norm_bwd(d, Y, g)
    np.testing.assert_allclose(dY.sum(axis=1), 0, atol=1e-12)
    sigma = np.sqrt(Y.var(1, keepdims=True) + orc.LN_EPS)
    xhat = (Y - Y.mean(1, keepdims=True)) / sigma
    # orthogonal to xhat up to the epsilon: sum(dY xhat) = sum(g xhat) (1 - mean(xhat^2)) / sigma,
    # and mean(xhat^2) = var / (var + eps)
    gx = (d * g * xhat).sum(axis=1)
    expect = gx * (1 - (xhat ** 2).mean(axis=1)) / sigma[:, 0]
    np.testing.assert_allclose((dY * xhat).sum(axis=1), expect, rtol=1e-6, atol=1e-13)
    assert np.abs(expect).max() < 1e-4
    np.testing.assert_allclose(db, d.sum(axis=0), rtol=1e-14)
    np.testing.assert_allclose(dg, (d * xhat).sum(axis=0), rtol=1e-12)


def test_layer_norm_gradient_matches_finite_differences():
    rng = np.random.default_rng(4)
    Y = rng.standard_normal((3, 8))
    d = rng.standard_normal((3, 8))
    g = 1 + rng.standard_normal(8)
    b = rng.standard_normal(8)
    dY, _, _ = bw.layer_norm_bwd(d, Y, g)
    num = _fd(lambda: float((orc.layer_norm(Y, g, b) * d).sum()), Y)
    np.testing.assert_allclose(dY, num, rtol=1e-6, atol=1e-8)


def test_gelu_derivative_closed_forms():
    # GELU(u) = u Phi(u): derivative 1/2 at 0, tends to 1 / 0 far right / left,
    # equals the finite difference of the forward definition everywhere
    assert bw.gelu_grad(0.0) == pytest.approx(0.5, abs=1e-15)
    assert bw.gelu_grad(12.0) == pytest.approx(1.0, abs=1e-12)
    assert bw.gelu_grad(-12.0) == pytest.approx(0.0, abs=1e-12)
    u = np.linspace(-6, 6, 97)
    h = 1e-6
    num = (orc.gelu(u + h) - orc.gelu(u - h)) / (2 * h)
    np.testing.assert_allclose(bw.gelu_grad(u), num, rtol=1e-7, atol=1e-9)
    # the tanh approximation's derivative differs by more than the check above allows
    t = 0.5 * (1 + np.tanh(math.sqrt(2 / math.pi) * (u + 0.044715 * u ** 3)))
    assert np.abs(t - bw.gelu_grad(u)).max() > 1e-4


def test_single_token_gradient_doubles_through_the_identity_mix():
    # T = 1: TM is the identity, so Y1 = 2X and dX = 2 dY1, whose rows (an LN
    # input gradient) sum to zero
    rng = np.random.default_rng(5)
    X = rng.standard_normal((4, 1, 8))
    blk = _block(1, 8, 16, 6)
    d_out = rng.standard_normal((4, 1, 8))
    got = bw.block_bwd(X, blk, d_out)
    f = bw.block_fwd_saved(X, blk)
    np.testing.assert_allclose(f["Y1"], 2 * X, rtol=1e-15)
    dS_total = got["dX"] / 2  # = dY1
    assert np.abs(dS_total.sum(axis=-1)).max() < 1e-12  # dY1 is an LN input gradient


def test_moe_block_is_rejected():
    blk = _block(2, 4, 4, 7)
    blk["wr"] = np.zeros((2, 2, 4))
    with pytest.raises(ValueError):
        bw.block_bwd(np.zeros((1, 2, 4)), blk, np.zeros((1, 2, 4)))


@pytest.mark.parametrize("B,T,D,Hd,t", [(4, 3, 6, 5, 1), (3, 2, 4, 8, 0), (5, 4, 8, 6, 3)])
def test_single_token_gradients_match_finite_differences(B, T, D, Hd, t):
    # token t's parameter gradients over the whole batch, from token t's own
    # forward: central differences of L = sum(d_out * X') in token t's weights,
    # and the t-slices of the whole backward
    rng = np.random.default_rng(40 + t)
    X = rng.standard_normal((B, T, D))
    blk = _block(T, D, Hd, 20 + t)
    d_out = rng.standard_normal((B, T, D))
    got = bw.block_bwd_token(X, blk, d_out, t)
    full = bw.block_bwd(X, blk, d_out)
    for k in ("w1", "b1", "w2", "b2"):
        sl = blk[k][t]
        np.testing.assert_allclose(got[k], _fd(lambda: _loss(X, blk, d_out), sl), rtol=1e-6, atol=1e-7, err_msg=k)
        np.testing.assert_allclose(got[k], full[k][t], rtol=1e-12, atol=1e-12, err_msg=k)

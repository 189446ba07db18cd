"""Pins of the DTSI-MoE training oracle (oracle/moe_training.py) against
things other than itself: central finite differences of the forward oracle
(L_task for everything the training forward touches, lambda * L_reg for the
inference router), the inference forward it must reduce to, and the sparsity
loss counted by hand."""
import math

import numpy as np
import pytest

from oracle import moe_training as mt
from oracle import rankmixer_oracle as orc


def _blk(T, D, E, He, seed):
    rng = np.random.default_rng(seed)
    return {
        "w1": rng.standard_normal((T, E, He, D)) / math.sqrt(D),
        "b1": 0.3 * rng.standard_normal((T, E, He)),
        "w2": rng.standard_normal((T, E, D, He)) / math.sqrt(He),
        "b2": 0.3 * rng.standard_normal((T, E, D)),
        "wr": rng.standard_normal((T, E, D)) / math.sqrt(D),
        "br": 0.2 * rng.standard_normal((T, E)),
        "wr_train": rng.standard_normal((T, E, D)) / math.sqrt(D),
        "br_train": 0.5 + 0.2 * rng.standard_normal((T, E)),
        "ln1_g": 1 + 0.3 * rng.standard_normal(D), "ln1_b": 0.3 * rng.standard_normal(D),
        "ln2_g": 1 + 0.3 * rng.standard_normal(D), "ln2_b": 0.3 * rng.standard_normal(D),
    }


def _fd(f, a, h=1e-6):
    g = np.empty_like(a)
    flat, gf = a.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        x0 = flat[i]
        flat[i] = x0 + h
        fp = f()
        flat[i] = x0 - h
        fm = f()
        flat[i] = x0
        gf[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("B,T,D,E,He,seed", [(3, 2, 4, 3, 5, 0), (2, 4, 8, 2, 4, 1)])
def test_gradients_match_finite_differences(B, T, D, E, He, seed):
    rng = np.random.default_rng(seed + 10)
    X = rng.standard_normal((B, T, D))
    blk = _blk(T, D, E, He, seed)
    d_out = rng.standard_normal((B, T, D))
    lam = 0.7
    # keep every router pre-activation away from the ReLU kink for the differences
    f = mt.dtsi_fwd_saved(X, blk)
    assert np.abs(f["Zt"]).min() > 1e-3 and np.abs(f["Zi"]).min() > 1e-3
    got = mt.dtsi_bwd(X, blk, d_out, lam)
    task = lambda: float((mt.dtsi_fwd_saved(X, blk)["out"] * d_out).sum())
    reg = lambda: lam * mt.dtsi_fwd_saved(X, blk)["l_reg"]
    np.testing.assert_allclose(got["dX"], _fd(task, X), rtol=1e-6, atol=1e-7)
    for k in ("w1", "b1", "w2", "b2", "wr_train", "br_train", "ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        np.testing.assert_allclose(got[k], _fd(task, blk[k]), rtol=1e-6, atol=1e-7, err_msg=k)
    for k in ("wr", "br"):
        np.testing.assert_allclose(got[k], _fd(reg, blk[k]), rtol=1e-6, atol=1e-7, err_msg=k)
        # and the task loss does not depend on the inference router at all
        assert np.abs(_fd(task, blk[k])).max() < 1e-9


def test_training_forward_with_equal_routers_is_the_inference_block():
    # h_train = h_infer: the training forward is the inference MoE block
    rng = np.random.default_rng(3)
    blk = _blk(2, 8, 3, 6, 4)
    blk["wr_train"], blk["br_train"] = blk["wr"].copy(), blk["br"].copy()
    X = rng.standard_normal((4, 2, 8))
    np.testing.assert_allclose(mt.dtsi_fwd_saved(X, blk)["out"], orc.block_fwd(X, blk), rtol=0, atol=1e-12)


def test_sparsity_loss_sums_the_inference_gates():
    # L_reg = sum over samples, tokens and experts of ReLU(h_infer(s)), by hand
    rng = np.random.default_rng(5)
    blk = _blk(2, 4, 3, 4, 6)
    X = rng.standard_normal((3, 2, 4))
    f = mt.dtsi_fwd_saved(X, blk)
    total = 0.0
    for b in range(3):
        for t in range(2):
            s = f["S"][b, t]
            for j in range(3):
                z = sum(blk["wr"][t, j, k] * s[k] for k in range(4)) + blk["br"][t, j]
                total += max(0.0, z)
    assert f["l_reg"] == pytest.approx(total, rel=1e-12)


@pytest.mark.parametrize("B,T,D,E,He,t,seed", [(3, 2, 4, 3, 5, 1, 0), (4, 3, 6, 2, 4, 0, 2)])
def test_single_token_gradients_match_finite_differences(B, T, D, E, He, t, seed):
    # token t's expert and router gradients over the whole batch, from token
    # t's own forward: central differences of the task loss (experts, training
    # router) and of lambda * L_reg (inference router), and the t-slices of
    # the whole backward
    rng = np.random.default_rng(seed + 30)
    X = rng.standard_normal((B, T, D))
    blk = _blk(T, D, E, He, seed + 3)
    d_out = rng.standard_normal((B, T, D))
    lam = 0.7
    f = mt.dtsi_fwd_saved(X, blk)
    assert np.abs(f["Zt"]).min() > 1e-3 and np.abs(f["Zi"]).min() > 1e-3
    got = mt.dtsi_bwd_token(X, blk, d_out, lam, t)
    full = mt.dtsi_bwd(X, blk, d_out, lam)
    task = lambda: float((mt.dtsi_fwd_saved(X, blk)["out"] * d_out).sum())
    reg = lambda: lam * mt.dtsi_fwd_saved(X, blk)["l_reg"]
    for k in ("w1", "b1", "w2", "b2", "wr_train", "br_train"):
        np.testing.assert_allclose(got[k], _fd(task, blk[k][t]), rtol=1e-6, atol=1e-7, err_msg=k)
    for k in ("wr", "br"):
        np.testing.assert_allclose(got[k], _fd(reg, blk[k][t]), rtol=1e-6, atol=1e-7, err_msg=k)
    for k in got:
        if k != "dG":
            np.testing.assert_allclose(got[k], full[k][t], rtol=1e-12, atol=1e-12, err_msg=k)


def test_single_token_gate_gradient_matches_finite_differences():
    # dG[b, j] = d L_task / d G_train[b, t, j]: with one sample in the batch a
    # shift of br_train[t, j] moves that one gate by the same amount while it
    # is on, so central differences in br_train give dG wherever z > 0; a
    # large training-router bias switches every gate on
    B, T, D, E, He, t = 3, 2, 6, 3, 4, 1
    rng = np.random.default_rng(41)
    X = rng.standard_normal((B, T, D))
    d_out = rng.standard_normal((B, T, D))
    for shift in (0.0, 10.0):
        blk = _blk(T, D, E, He, 7)
        blk["br_train"] = blk["br_train"] + shift
        dG = mt.dtsi_bwd_token(X, blk, d_out, 0.3, t)["dG"]
        zt = mt.dtsi_fwd_saved(X, blk)["Zt"][:, t]
        assert np.abs(zt).min() > 1e-3
        if shift:
            assert (zt > 0).all()
        for b in range(B):
            task = lambda: float((mt.dtsi_fwd_saved(X[b:b + 1], blk)["out"] * d_out[b:b + 1]).sum())
            fd = _fd(task, blk["br_train"][t])
            np.testing.assert_allclose(fd, dG[b] * (zt[b] > 0), rtol=1e-6, atol=1e-7)

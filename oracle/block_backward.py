"""fp64 CPU oracle for the backward pass of one dense RankMixer block.

TEST INFRASTRUCTURE ONLY, like ``rankmixer_oracle``: only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path never does, and this module never imports the product path.

The forward is the block of [FR] "Rankmixer: 硬件效率优化", section
"RankMixer整体架构" (the block equations), with the per-token FFN of section
"Per-Token FFN":

    Y1 = TM(X) + X          S  = LN1(Y1)
    U_t = W1_t s_t + b1_t   H_t = GELU(U_t)     V_t = W2_t H_t + b2_t
    Y2 = V + S              X' = LN2(Y2)

The pages train this block (their cost figures are training flops) but print
no backward; every function below is the chain rule applied to one forward
equation, written out in float64 numpy per token, nothing fused or reordered.
Given dX' = dL/dX' for some loss L it returns dL/dX and the gradients of every
parameter.  Readings: the token mix is a permutation that is its own
inverse when H = T, so its transpose is itself; the MoE block's backward
(with its two routers) is in ``moe_training``.

Parity pins (tests/test_oracle_backward_pins.py): central finite differences
of the forward oracle on small blocks for every output, LayerNorm gradient
invariants, GELU derivative closed forms.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

from oracle.rankmixer_oracle import LN_EPS, as_f64, gelu, layer_norm, token_mix


def layer_norm_bwd(d_out, Y, gamma, eps: float = LN_EPS):
    """Gradients of out = LN(Y) = xhat * gamma + beta, xhat = (Y - mu) / sigma,
    sigma = sqrt(var + eps), mean and biased variance over the last axis.

    d xhat_i / d y_j = (delta_ij - 1/D - xhat_i xhat_j / D) / sigma, so with
    g = d_out * gamma:  dY = (g - mean(g) - xhat * mean(g * xhat)) / sigma.
    dgamma = sum over all rows of d_out * xhat; dbeta = sum over all rows of
    d_out.  Returns (dY, dgamma, dbeta)."""
    Y = as_f64(Y)
    d_out = as_f64(d_out)
    gamma = as_f64(gamma)
    mu = Y.mean(axis=-1, keepdims=True)
    var = ((Y - mu) ** 2).mean(axis=-1, keepdims=True)
    sigma = np.sqrt(var + eps)
    xhat = (Y - mu) / sigma
    g = d_out * gamma
    dY = (g - g.mean(axis=-1, keepdims=True) - xhat * (g * xhat).mean(axis=-1, keepdims=True)) / sigma
    rows = d_out.reshape(-1, d_out.shape[-1])
    dgamma = (rows * xhat.reshape(rows.shape)).sum(axis=0)
    dbeta = rows.sum(axis=0)
    return dY, dgamma, dbeta


def gelu_grad(u) -> np.ndarray:
    """d/du of GELU(u) = u Phi(u): Phi(u) + u phi(u), phi the standard normal
    density."""
    u = np.asarray(u, dtype=np.float64)
    Phi = 0.5 * (1.0 + _erf(u / math.sqrt(2.0)))
    phi = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return Phi + u * phi


def block_fwd_saved(X, blk: dict) -> dict:
    """The dense block forward, keeping every intermediate the backward uses:
    Y1, S, U, H, V, Y2 and the output X' (float64, [B,T,*])."""
    if "wr" in blk:
        raise ValueError("the MoE block has no backward here")
    X = as_f64(X)
    B, T, D = X.shape
    Y1 = token_mix(X) + X
    S = layer_norm(Y1, blk["ln1_g"], blk["ln1_b"])
    Hd = blk["w1"].shape[1]
    U = np.empty((B, T, Hd))
    V = np.empty((B, T, D))
    for t in range(T):
        U[:, t, :] = S[:, t, :] @ as_f64(blk["w1"][t]).T + as_f64(blk["b1"][t])
        V[:, t, :] = gelu(U[:, t, :]) @ as_f64(blk["w2"][t]).T + as_f64(blk["b2"][t])
    H = gelu(U)
    Y2 = V + S
    return {"Y1": Y1, "S": S, "U": U, "H": H, "V": V, "Y2": Y2,
            "out": layer_norm(Y2, blk["ln2_g"], blk["ln2_b"])}


def block_bwd(X, blk: dict, d_out) -> dict:
    """Backward of one dense block.  d_out = dL/dX' [B,T,D].  Returns float64
    gradients: dX [B,T,D]; w1 [T,Hd,D], b1 [T,Hd], w2 [T,D,Hd], b2 [T,D];
    ln1_g, ln1_b, ln2_g, ln2_b [D]."""
    f = block_fwd_saved(X, blk)
    d_out = as_f64(d_out)
    B, T, D = d_out.shape
    Hd = blk["w1"].shape[1]
    # X' = LN2(Y2)
    dY2, dg2, db2n = layer_norm_bwd(d_out, f["Y2"], blk["ln2_g"])
    # Y2 = V + S: both terms receive dY2
    dV = dY2
    dS = dY2.copy()
    dw1 = np.empty((T, Hd, D))
    db1 = np.empty((T, Hd))
    dw2 = np.empty((T, D, Hd))
    db2 = np.empty((T, D))
    for t in range(T):
        W1 = as_f64(blk["w1"][t])
        W2 = as_f64(blk["w2"][t])
        # V_t = W2_t H_t + b2_t, summed over the samples b
        db2[t] = dV[:, t, :].sum(axis=0)
        dw2[t] = dV[:, t, :].T @ f["H"][:, t, :]
        dH = dV[:, t, :] @ W2
        # H_t = GELU(U_t)
        dU = dH * gelu_grad(f["U"][:, t, :])
        # U_t = W1_t s_t + b1_t
        db1[t] = dU.sum(axis=0)
        dw1[t] = dU.T @ f["S"][:, t, :]
        dS[:, t, :] += dU @ W1
    # S = LN1(Y1)
    dY1, dg1, db1n = layer_norm_bwd(dS, f["Y1"], blk["ln1_g"])
    # Y1 = TM(X) + X, TM a permutation with TM^-1 = TM^T = TM
    dX = dY1 + token_mix(dY1)
    return {"dX": dX, "w1": dw1, "b1": db1, "w2": dw2, "b2": db2,
            "ln1_g": dg1, "ln1_b": db1n, "ln2_g": dg2, "ln2_b": db2n}


def block_bwd_token(X, blk: dict, d_out, t: int) -> dict:
    """The parameter gradients of token t alone (w1[t], b1[t], w2[t], b2[t]),
    summed over the whole batch, from token t's own forward: S needs the whole
    token mix of every sample, but U_t, H_t, V_t, Y2_t and LN2's backward
    involve token t's rows only (LN2 normalises each (sample, token) row by
    itself), so this is exact at any batch size for a fraction of
    ``block_bwd``'s work."""
    X = as_f64(X)
    d_out = as_f64(d_out)
    S = layer_norm(token_mix(X) + X, blk["ln1_g"], blk["ln1_b"])
    S_t = S[:, t, :]
    W1 = as_f64(blk["w1"][t])
    W2 = as_f64(blk["w2"][t])
    U = S_t @ W1.T + as_f64(blk["b1"][t])
    H = gelu(U)
    Y2 = H @ W2.T + as_f64(blk["b2"][t]) + S_t
    dV, _, _ = layer_norm_bwd(d_out[:, t, :], Y2, blk["ln2_g"])
    dU = (dV @ W2) * gelu_grad(U)
    return {"w1": dU.T @ S_t, "b1": dU.sum(axis=0), "w2": dV.T @ H, "b2": dV.sum(axis=0)}

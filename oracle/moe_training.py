"""fp64 CPU oracle for training the ReLU-routed MoE block with the
dense-training / sparse-inference routers (DTSI-MoE).

TEST INFRASTRUCTURE ONLY, like ``rankmixer_oracle``: only the tests, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product
path never does, and this module never imports the product path.

[FR] "Rankmixer: 硬件效率优化", section "Sparse MoE扩展", and [WL] (ReLU routing,
dense training + sparse inference): two routers per token, h_train and
h_infer, both affine maps R^D -> R^{N_e}:

    G_train = ReLU(h_train(s)),  G_infer = ReLU(h_infer(s))
    v_t = sum_j G_train[t, j] e_{t,j}(s_t)            (the training forward)
    L_reg = sum over tokens and experts of G_infer     (summed over the batch)
    L = L_task + lambda * L_reg

and only h_infer is subject to L_reg.  At inference only h_infer routes (the
forward of ``rankmixer_oracle.block_fwd`` with wr/br = h_infer).  Readings:
L_reg's gradient reaches h_infer's weights and bias only, not S (the pages
restrict the regulariser to h_infer); L_task reaches everything but h_infer,
which does not take part in the training forward.

Every function is the chain rule through one forward equation, in float64.
Parity pins (tests/test_oracle_moe_training_pins.py): central finite
differences of L_task for everything but h_infer and of lambda * L_reg for
h_infer's parameters, the inference special case, and gate counting.
"""
from __future__ import annotations

import numpy as np

from oracle.block_backward import gelu_grad, layer_norm_bwd
from oracle.rankmixer_oracle import as_f64, gelu, layer_norm, token_mix


def dtsi_fwd_saved(X, blk: dict) -> dict:
    """Training forward of one MoE block: blk holds the experts (w1 [T,E,He,D],
    b1 [T,E,He], w2 [T,E,D,He], b2 [T,E,D]), the inference router (wr [T,E,D],
    br [T,E]), the training router (wr_train, br_train) and the LayerNorms.
    Returns the intermediates the backward uses, the output and L_reg."""
    X = as_f64(X)
    B, T, D = X.shape
    E = blk["w1"].shape[1]
    He = blk["w1"].shape[2]
    Y1 = token_mix(X) + X
    S = layer_norm(Y1, blk["ln1_g"], blk["ln1_b"])
    Zt = np.empty((B, T, E))
    Zi = np.empty((B, T, E))
    U = np.empty((B, T, E, He))
    Yx = np.empty((B, T, E, D))
    for t in range(T):
        Zt[:, t] = S[:, t] @ as_f64(blk["wr_train"][t]).T + as_f64(blk["br_train"][t])
        Zi[:, t] = S[:, t] @ as_f64(blk["wr"][t]).T + as_f64(blk["br"][t])
        for j in range(E):
            U[:, t, j] = S[:, t] @ as_f64(blk["w1"][t, j]).T + as_f64(blk["b1"][t, j])
            Yx[:, t, j] = gelu(U[:, t, j]) @ as_f64(blk["w2"][t, j]).T + as_f64(blk["b2"][t, j])
    Gt = np.maximum(Zt, 0.0)
    Gi = np.maximum(Zi, 0.0)
    V = (Gt[..., None] * Yx).sum(axis=2)
    Y2 = V + S
    return {"Y1": Y1, "S": S, "Zt": Zt, "Zi": Zi, "Gt": Gt, "Gi": Gi, "U": U, "Yx": Yx, "Y2": Y2,
            "out": layer_norm(Y2, blk["ln2_g"], blk["ln2_b"]), "l_reg": float(Gi.sum())}


def dtsi_bwd(X, blk: dict, d_out, lam: float) -> dict:
    """Gradients of L = sum(d_out * X') + lam * L_reg.  Returns float64 dX and
    the gradients of w1, b1, w2, b2, wr_train, br_train, wr (h_infer), br
    (h_infer), ln1_g, ln1_b, ln2_g, ln2_b."""
    f = dtsi_fwd_saved(X, blk)
    d_out = as_f64(d_out)
    B, T, D = d_out.shape
    E = blk["w1"].shape[1]
    He = blk["w1"].shape[2]
    # X' = LN2(V + S)
    dY2, dg2, db2n = layer_norm_bwd(d_out, f["Y2"], blk["ln2_g"])
    dV = dY2
    dS = dY2.copy()
    g = {k: np.zeros(np.shape(blk[k])) for k in ("w1", "b1", "w2", "b2", "wr_train", "br_train", "wr", "br")}
    for t in range(T):
        S_t = f["S"][:, t]
        # v_t = sum_j G_train[t, j] y_{t,j}: dG = dV . y, dy = G dV
        dG = np.einsum("bd,bjd->bj", dV[:, t], f["Yx"][:, t])
        for j in range(E):
            dy = f["Gt"][:, t, j:j + 1] * dV[:, t]
            # y = W2 H + b2, H = GELU(U), U = W1 s + b1
            W1 = as_f64(blk["w1"][t, j])
            W2 = as_f64(blk["w2"][t, j])
            g["b2"][t, j] = dy.sum(axis=0)
            g["w2"][t, j] = dy.T @ gelu(f["U"][:, t, j])
            dU = (dy @ W2) * gelu_grad(f["U"][:, t, j])
            g["b1"][t, j] = dU.sum(axis=0)
            g["w1"][t, j] = dU.T @ S_t
            dS[:, t] += dU @ W1
        # G_train = ReLU(z_train), z_train = Wr_train s + br_train
        dz = dG * (f["Zt"][:, t] > 0)
        g["br_train"][t] = dz.sum(axis=0)
        g["wr_train"][t] = dz.T @ S_t
        dS[:, t] += dz @ as_f64(blk["wr_train"][t])
        # lam * L_reg = lam * sum ReLU(z_infer): reaches h_infer's parameters only
        dzi = lam * (f["Zi"][:, t] > 0)
        g["br"][t] = dzi.sum(axis=0)
        g["wr"][t] = dzi.T @ S_t
    # S = LN1(TM(X) + X); TM is its own transpose
    dY1, dg1, db1n = layer_norm_bwd(dS, f["Y1"], blk["ln1_g"])
    g["dX"] = dY1 + token_mix(dY1)
    g["ln1_g"], g["ln1_b"], g["ln2_g"], g["ln2_b"] = dg1, db1n, dg2, db2n
    return g


def dtsi_bwd_token(X, blk: dict, d_out, lam: float, t: int, train_on=None, infer_on=None) -> dict:
    """The parameter gradients of token t alone -- its experts (w1[t], b1[t],
    w2[t], b2[t], all E of them), its training router (wr_train[t],
    br_train[t]) and its inference router (wr[t], br[t]) -- summed over the
    whole batch, from token t's own forward.  S needs every sample's whole
    token mix; the rest involves token t's rows only (LN2 normalises each row
    by itself), so this is exact at any batch size.

    train_on / infer_on ([B, E] booleans, optional) are the ReLU decisions
    z > 0 of the two routers for token t, for a caller that must take them in
    another precision than this fp64 evaluation (a decision, unlike a value,
    does not converge as the precision grows; the gates' values stay fp64).
    Also returned: "dG" [B, E], the task loss's gradient with respect to each
    sample's training gate of token t (what one decision adds to the router's
    gradients, times s_t)."""
    X = as_f64(X)
    d_out = as_f64(d_out)
    E = blk["w1"].shape[1]
    S = layer_norm(token_mix(X) + X, blk["ln1_g"], blk["ln1_b"])
    S_t = S[:, t]
    Zt = S_t @ as_f64(blk["wr_train"][t]).T + as_f64(blk["br_train"][t])
    Zi = S_t @ as_f64(blk["wr"][t]).T + as_f64(blk["br"][t])
    on_t = Zt > 0 if train_on is None else np.asarray(train_on, dtype=bool)
    on_i = Zi > 0 if infer_on is None else np.asarray(infer_on, dtype=bool)
    Gt = np.where(on_t, Zt, 0.0)
    U = [S_t @ as_f64(blk["w1"][t, j]).T + as_f64(blk["b1"][t, j]) for j in range(E)]
    Yx = [gelu(U[j]) @ as_f64(blk["w2"][t, j]).T + as_f64(blk["b2"][t, j]) for j in range(E)]
    V = sum(Gt[:, j:j + 1] * Yx[j] for j in range(E))
    dV, _, _ = layer_norm_bwd(d_out[:, t], V + S_t, blk["ln2_g"])
    g = {k: np.zeros(np.shape(blk[k])[1:]) for k in ("w1", "b1", "w2", "b2", "wr_train", "br_train", "wr", "br")}
    dG = np.stack([(dV * Yx[j]).sum(axis=1) for j in range(E)], axis=1)
    for j in range(E):
        dy = Gt[:, j:j + 1] * dV
        g["b2"][j] = dy.sum(axis=0)
        g["w2"][j] = dy.T @ gelu(U[j])
        dU = (dy @ as_f64(blk["w2"][t, j])) * gelu_grad(U[j])
        g["b1"][j] = dU.sum(axis=0)
        g["w1"][j] = dU.T @ S_t
    dz = dG * on_t
    g["br_train"] = dz.sum(axis=0)
    g["wr_train"] = dz.T @ S_t
    dzi = lam * on_i
    g["br"] = dzi.sum(axis=0)
    g["wr"] = dzi.T @ S_t
    g["dG"] = dG
    return g

"""fp64 CPU oracle for the RankMixer block forward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The product path (the HIP
library and its Python binding) never calls it, and this module never imports
the product path; the two share no code.  Both read the same seeded arrays
from ``synthetic_inputs``.

Every function is the plain definition from the source pages, written out in
float64 numpy, per sample and per token, with no blocking, fusion or
reordering beyond what the definition states.  A matrix product or ``erf``
from numpy/scipy serves as a step.  Intermediate results are never rounded to
bf16: only the pad-split tokenizer rounds, because its defined output is the
model input in the configured dtype.

Pages cited (titles as printed on them):
  [FR]  "Rankmixer: 硬件效率优化" (fun-rec textbook chapter, datawhalechina)
  [WL]  "特征交叉 —— RankMixer 精读笔记" (reading notes on arXiv 2507.15551)
  [TB]  "淘宝闪购-爆品团精排 Scaling Up 迭代实践" (BestBlogs.dev report)
  [SX]  "重新理解 RankMixer：扩参为什么有效，又为什么划算？" (sxkj888.cn blog)

Readings taken where the pages are silent:
  * LayerNorm: epsilon 1e-5, biased variance over the D entries of one token,
    one gamma/beta pair of length D per LayerNorm.
  * GELU is the exact erf form x * Phi(x).
  * W1_t maps R^D -> R^{kD} (stored [kD][D]); W2_t maps back (stored [D][kD]).
    [FR] prints the shapes as R^{D x kD} / R^{kD x D} but multiplies W1 s_t
    with s_t in R^D, so the matrix-vector reading wins.
  * Head h of token t is the contiguous slice [h*D/H, (h+1)*D/H); Concat is in
    token order; H = T.
  * MoE router: per token t an affine map R^D -> R^{N_e}; the gate multiplies
    the whole expert output including its output bias; no softmax, no top-k.
  * Pad-split pads with zeros at the end, tokens are consecutive slices.

Parity pins: every function here is checked in tests/test_oracle_pins.py
against something other than itself (library routines, closed forms,
invariants the pages state, brute-force index loops).  None is unpinned.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
from scipy.special import erf as _erf

LN_EPS = 1e-5


# ----------------------------------------------------------------------------
# decoding and the one rounding the method defines


def as_f64(a) -> np.ndarray:
    """Array -> float64.  uint16 arrays are bf16 bit patterns (the upper half
    of an IEEE binary32 word) and are decoded exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float values to the nearest bf16 value (8 significant bits, the
    float32 exponent range), ties to even.  Written from the definition of
    round-to-nearest-even: scale the significand to 8 integer bits, round
    half to even, scale back.  Returns float64 holding bf16 values."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # below 2**-126: fixed subnormal spacing
    quantum = np.ldexp(1.0, e - 8)          # spacing of 8-bit significands at this exponent
    out = np.rint(x / quantum) * quantum    # np.rint rounds halves to even
    return np.where(x == 0, x, out)


# ----------------------------------------------------------------------------
# the block's building blocks


def tokenize_padsplit(emb, T: int, D: int, dtype: str) -> np.ndarray:
    """Pad-split tokenizer ([TB] section 3.4): concatenate the embedding floats
    of a sample, pad with zeros to T*D, cut into T consecutive tokens of width
    D.  No projection.  The result is cast to the model dtype."""
    e = as_f64(emb)
    B, F = e.shape
    if F > T * D:
        raise ValueError("embedding longer than T*D")
    padded = np.zeros((B, T * D))
    padded[:, :F] = e
    X0 = padded.reshape(B, T, D)
    return round_to_bf16(X0) if dtype == "bf16" else X0.astype(np.float32).astype(np.float64)


def tokenize_project(emb, w, b, T: int, seg: int, dtype: str) -> np.ndarray:
    """Projection tokenizer ([WL] section "特征的Tokenization"): the
    concatenated embedding e_input of a sample is cut evenly into T segments
    and each segment is mapped to R^D by its own linear layer,
    x_t = W_t seg_t + b_t.  Readings: the segments have length seg (at least
    ceil(F / T)) and e_input is zero-padded to T*seg, as the pad-split
    tokenizer pads; the embedding is cast to the model dtype first, as the
    pad-split tokenizer casts; "linear layer" includes a bias.  w is
    [T][D][seg] (W_t maps R^seg -> R^D), b is [T][D]."""
    e = as_f64(emb)
    B, F = e.shape
    if F > T * seg:
        raise ValueError("embedding longer than T*seg")
    padded = np.zeros((B, T * seg))
    padded[:, :F] = e
    if dtype == "bf16":
        padded = round_to_bf16(padded)
    else:
        padded = padded.astype(np.float32).astype(np.float64)
    segs = padded.reshape(B, T, seg)
    W = as_f64(w)
    return np.einsum("bts,tds->btd", segs, W) + np.asarray(b, np.float64)[None, :, :]


def token_mix(X) -> np.ndarray:
    """Multi-head token mixing with H = T ([FR] section "Token Mixing机制";
    [WL] "Multi-Head Token Mixer").  SplitHead cuts every token x_t into H
    heads x_t^(h) of width D/H; Concat joins head h of all tokens in token
    order, s^h = [x_1^(h) | ... | x_T^(h)].  With H = T the H new vectors have
    width D again and form the new token sequence."""
    X = as_f64(X)
    B, T, D = X.shape
    H = T
    if D % H:
        raise ValueError("D must be divisible by H = T")
    heads = X.reshape(B, T, H, D // H)          # [b, t, h, :] = x_t^(h)
    S = np.empty((B, H, T, D // H))
    for h in range(H):
        for t in range(T):
            S[:, h, t, :] = heads[:, t, h, :]   # s^h = Concat_t x_t^(h)
    return S.reshape(B, H, D)


def layer_norm(Y, gamma, beta, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis with the biased variance."""
    Y = as_f64(Y)
    mu = Y.mean(axis=-1, keepdims=True)
    var = ((Y - mu) ** 2).mean(axis=-1, keepdims=True)
    return (Y - mu) / np.sqrt(var + eps) * as_f64(gamma) + as_f64(beta)


def gelu(x) -> np.ndarray:
    """GELU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def pffn(S, w1, b1, w2, b2) -> np.ndarray:
    """Per-token FFN ([FR] section "Per-Token FFN"; [WL] "Per-Token FFN"):
    v_t = W2_t GELU(W1_t s_t + b1_t) + b2_t with independent weights for
    every token position t.  S: [B,T,D]; w1 [T,Hd,D]; w2 [T,D,Hd]."""
    S = as_f64(S)
    B, T, D = S.shape
    V = np.empty((B, T, D))
    for t in range(T):
        W1 = as_f64(w1[t])
        W2 = as_f64(w2[t])
        h = gelu(S[:, t, :] @ W1.T + as_f64(b1[t]))
        V[:, t, :] = h @ W2.T + as_f64(b2[t])
    return V


def silu(x) -> np.ndarray:
    """SiLU (Swish with beta = 1): x * sigmoid(x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu_pffn(S, w1, b1, w2, b2) -> np.ndarray:
    """Per-token SwiGLU FFN ([TB] section 3.6, "SwiGLU D->4/3D", a drop-in for
    the per-token FFN): for every token t,
      v_t = W2_t (SiLU(Wg_t s_t + bg_t) * (Wu_t s_t + bu_t)) + b2_t,
    '*' elementwise.  w1 [T, 2*Hs, D] holds the gate rows Wg_t (0 .. Hs-1) and
    then the up rows Wu_t (Hs .. 2Hs-1); b1 [T, 2*Hs] likewise; w2 [T, D, Hs].
    Reading: the pages name the variant only; it is taken with a bias on every
    linear map, like the per-token FFN here (zero biases give the bias-free
    form)."""
    S = as_f64(S)
    B, T, D = S.shape
    Hs = w1.shape[1] // 2
    V = np.empty((B, T, D))
    for t in range(T):
        W1 = as_f64(w1[t])
        bb = as_f64(b1[t])
        g = S[:, t, :] @ W1[:Hs].T + bb[:Hs]
        u = S[:, t, :] @ W1[Hs:].T + bb[Hs:]
        V[:, t, :] = (silu(g) * u) @ as_f64(w2[t]).T + as_f64(b2[t])
    return V


def moe_gates(S, wr, br) -> np.ndarray:
    """ReLU router ([FR] section "Sparse MoE扩展"; [WL] ReLU routing):
    G_{t,j} = ReLU(h(s_t))_j with h the per-token affine router.  Returns
    float64 [B,T,E]."""
    S = as_f64(S)
    B, T, D = S.shape
    E = wr.shape[1]
    G = np.empty((B, T, E))
    for t in range(T):
        z = S[:, t, :] @ as_f64(wr[t]).T + as_f64(br[t])
        G[:, t, :] = np.maximum(z, 0.0)
    return G


def moe_relu_pffn(S, w1, b1, w2, b2, wr, br):
    """ReLU-gated per-token sparse MoE: v_t = sum_j G_{t,j} e_{t,j}(s_t), where
    e_{t,j} is expert j of token t, an FFN of the same form as the per-token
    FFN.  A zero gate means the expert is not active and contributes nothing.
    Returns (V [B,T,D], G [B,T,E])."""
    S = as_f64(S)
    B, T, D = S.shape
    E = w1.shape[1]
    G = moe_gates(S, wr, br)
    V = np.zeros((B, T, D))
    for t in range(T):
        for j in range(E):
            h = gelu(S[:, t, :] @ as_f64(w1[t, j]).T + as_f64(b1[t, j]))
            y = h @ as_f64(w2[t, j]).T + as_f64(b2[t, j])
            V[:, t, :] += G[:, t, j:j + 1] * y
    return V, G


# ----------------------------------------------------------------------------
# block and model


def block_fwd(X, blk: dict) -> np.ndarray:
    """One RankMixer block ([FR] section "RankMixer整体架构", block equations):
    S = LN(TokenMixing(X) + X);  X' = LN(PFFN(S) + S).  A block whose params
    hold a router ("wr") uses the ReLU-gated MoE in place of the PFFN; one
    marked "swiglu" uses the SwiGLU FFN.  A block marked "no_mix_norm" drops
    the Add & Norm after the token mix ([TB] section 3.5, the variant that lost
    it): S = TokenMixing(X)."""
    X = as_f64(X)
    if blk.get("no_mix_norm"):
        S = token_mix(X)
    else:
        S = layer_norm(token_mix(X) + X, blk["ln1_g"], blk["ln1_b"])
    if "wr" in blk:
        V, _ = moe_relu_pffn(S, blk["w1"], blk["b1"], blk["w2"], blk["b2"], blk["wr"], blk["br"])
    elif blk.get("swiglu"):
        V = swiglu_pffn(S, blk["w1"], blk["b1"], blk["w2"], blk["b2"])
    else:
        V = pffn(S, blk["w1"], blk["b1"], blk["w2"], blk["b2"])
    return layer_norm(V + S, blk["ln2_g"], blk["ln2_b"])


def mean_pool(X) -> np.ndarray:
    """Average of the last block's tokens over the sequence ([WL], model output;
    [FR] "RankMixer整体架构": mean pooling produces the output)."""
    return as_f64(X).mean(axis=1)


def model_fwd(inp, blocks, T: int, D: int, dtype: str, F: int = 0,
              head: Optional[dict] = None) -> dict:
    """L stacked blocks, X_L = block_L(...block_1(X_0)); optional pad-split
    tokenizer in front and mean pooling plus a D -> 1 linear logit behind.
    ``inp`` is the embedding [B,F] when F > 0, else X_0 [B,T,D]."""
    X = tokenize_padsplit(inp, T, D, dtype) if F else as_f64(inp)
    for blk in blocks:
        X = block_fwd(X, blk)
    out = {"x": X}
    if head is not None:
        p = mean_pool(X)
        out["pooled"] = p
        out["logit"] = p @ as_f64(head["w"]) + float(head["c"])
    return out


def subset_inputs(inputs: dict, rows) -> dict:
    """The same inputs restricted to the sample indices ``rows``.  Samples do
    not interact anywhere in the forward (LayerNorm and routing are per token,
    there is no batch statistic), so the oracle on a subset is exact."""
    out = dict(inputs)
    rows = np.asarray(rows)
    if "x" in inputs:
        out["x"] = inputs["x"][rows]
    if "emb" in inputs:
        out["emb"] = inputs["emb"][rows]
    return out


def run_config(inputs: dict, rows=None) -> dict:
    """Oracle forward of a whole drawn config (see synthetic_inputs), or of the
    samples ``rows`` only."""
    cfg = inputs["config"]
    if rows is not None:
        inputs = subset_inputs(inputs, rows)
    inp = inputs["emb"] if cfg.F else inputs["x"]
    return model_fwd(inp, inputs["blocks"], cfg.T, cfg.D, cfg.dtype, cfg.F, inputs.get("head"))

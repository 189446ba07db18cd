"""Seeded synthetic inputs for the RankMixer block forward: the five workload
configurations and the tensors they are built from.

This module only draws random numbers and packs them. It holds none of the
method's arithmetic (no mixing, normalisation, FFN or routing): both the fp64
oracle and the HIP path read the arrays it returns.

Recipe (the same for every config):

* Every random tensor is drawn as float32 from numpy's PCG64 generator and
  scaled by its standard deviation.  ``N(0, v)`` in a config means variance
  ``v`` (standard deviation ``sqrt(v)``); ``N(0, 1/fan_in)`` uses the input
  width of the matrix it initialises (D for W1 and the router, the hidden
  width for W2, D for the logit head).
* Tensors are drawn in a fixed order: the model input (X or the concatenated
  embedding), then per block W1, b1, W2, b2 (dense) or W1, b1, W2, b2, Wr (MoE),
  then the logit head.  A tensor whose distribution is a constant (zero biases,
  the MoE router bias, LayerNorm gamma=1 / beta=0) is filled, not drawn.
* Each tensor is cut into chunks of ``CHUNK`` elements; chunk ``c`` of tensor
  ``i`` comes from ``default_rng(SeedSequence([seed, i, c]))``.  The result
  does not depend on how many threads draw it.
* bf16 configs round every weight matrix and the block input to bf16 once,
  round-to-nearest-even, and hand them over as uint16 bit patterns (the upper
  half of the IEEE binary32 word).  Biases, LayerNorm affine parameters, the
  router bias and the logit head stay float32.  The pad-split embedding stays
  float32: the tokenizer itself casts it.

Sources for the shapes: the RankMixer block equations (token mixing with H=T,
per-token FFN of hidden width kD, ReLU-routed per-token MoE) and the pad-split
tokenizer of 5000 concatenated floats padded to 5120 and cut into 16 tokens of
320 ("Taobao flash-sale RankMixer" report, section 3.4).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Dict, List, Optional

import numpy as np

CHUNK = 1 << 24  # elements per independently seeded chunk

# Router bias for the ReLU-gated MoE config.  With router weights N(0, 1/D) and
# a LayerNorm output s of unit variance, the pre-activation is close to
# N(bias, 1); a bias of -Phi^-1(0.75) leaves about 25 % of the gates positive.
MOE_ROUTER_BIAS = -0.6744897501960817


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    T: int
    D: int
    L: int
    dtype: str            # "f32" or "bf16"
    k: int = 4            # dense FFN hidden = k * D
    E: int = 0            # experts per token (0 = dense block)
    He: int = 0           # expert hidden width
    F: int = 0            # >0: input is an embedding vector of F floats, pad-split
    emb_var: float = 0.0  # variance of the embedding floats
    bias_var: float = 0.0  # variance of dense biases (0 = zero biases)
    head: bool = False    # mean-pool over tokens, then a D -> 1 logit
    description: str = ""

    @property
    def hidden(self) -> int:
        return self.He if self.E else self.k * self.D

    @property
    def d(self) -> int:
        return self.D // self.T


CONFIGS: Dict[str, Config] = {
    "c0": Config("c0", B=64, T=4, D=64, L=1, dtype="f32", k=2,
                 description="tiny fp32 block: B=64, T=4, D=64, k=2, L=1"),
    "c1": Config("c1", B=2048, T=16, D=768, L=2, dtype="bf16", k=4, bias_var=0.01,
                 description="~100M-class dense: B=2048, T=16, D=768, k=4, L=2, bf16"),
    "c2": Config("c2", B=4096, T=16, D=320, L=4, dtype="bf16", k=4, F=5000,
                 emb_var=0.1, head=True,
                 description="pad-split model: B=4096, 5000 floats -> 16x320, k=4, L=4, "
                             "mean pool + 320->1 logit, bf16"),
    "c3": Config("c3", B=1024, T=32, D=1536, L=2, dtype="bf16", k=4,
                 description="~1B-class dense: B=1024, T=32, D=1536, k=4, L=2, bf16"),
    "c4": Config("c4", B=2048, T=16, D=768, L=2, dtype="bf16", E=8, He=1536,
                 description="ReLU-routed per-token MoE: B=2048, T=16, D=768, 8 experts "
                             "of 768->1536->768, L=2, bf16"),
}
SEEDS = {"c0": 0, "c1": 1, "c2": 2, "c3": 3, "c4": 4}


def scaled(cfg: Config, **changes) -> Config:
    """A copy of ``cfg`` with some fields replaced (for smaller test shapes)."""
    return dataclasses.replace(cfg, **changes)


# ----------------------------------------------------------------------------
# drawing


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_normal(out: np.ndarray, seed: int, tensor_id: int, std: float) -> None:
    flat = out.reshape(-1)
    nchunks = (flat.size + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        lo = c * CHUNK
        hi = min(flat.size, lo + CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([seed, tensor_id, c]))
        seg = flat[lo:hi]
        rng.standard_normal(out=seg, dtype=np.float32)
        seg *= np.float32(std)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    out = np.empty(a.shape, dtype=np.uint16)
    fo = out.reshape(-1)
    fu = u.reshape(-1)
    step = CHUNK

    def work(lo: int) -> None:
        seg = fu[lo:lo + step]
        r = ((seg >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
        fo[lo:lo + step] = ((seg + r) >> np.uint32(16)).astype(np.uint16)

    starts = range(0, fu.size, step)
    if fu.size <= step:
        for lo in starts:
            work(lo)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, starts))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


class _Drawer:
    def __init__(self, seed: int):
        self.seed = seed
        self.next_id = 0

    def normal(self, shape, var: float) -> np.ndarray:
        out = np.empty(shape, dtype=np.float32)
        _fill_normal(out, self.seed, self.next_id, math.sqrt(var))
        self.next_id += 1
        return out


def make_inputs(cfg: Config, seed: Optional[int] = None) -> dict:
    """Draw every tensor of ``cfg``.

    Returns a dict with
      ``x``      block input [B,T,D]  (uint16 bf16 bits, or float32)   if cfg.F == 0
      ``emb``    float32 [B,F]                                          if cfg.F > 0
      ``blocks`` list of L dicts: ln1_g, ln1_b, ln2_g, ln2_b (float32 [D]) and
                 dense: w1 [T,Hd,D], b1 [T,Hd], w2 [T,D,Hd], b2 [T,D]
                 MoE:   w1 [T,E,He,D], b1 [T,E,He], w2 [T,E,D,He], b2 [T,E,D],
                        wr [T,E,D], br [T,E]
      ``head``   dict(w=float32 [D], c=float) if cfg.head
    Weight matrices and ``x`` are uint16 bf16 bits for bf16 configs.
    """
    if seed is None:
        seed = SEEDS.get(cfg.name, 0)
    dr = _Drawer(seed)
    bf = cfg.dtype == "bf16"
    mat = (lambda a: to_bf16_bits(a)) if bf else (lambda a: a)
    B, T, D = cfg.B, cfg.T, cfg.D
    out: dict = {"config": cfg, "seed": seed}
    if cfg.F:
        out["emb"] = dr.normal((B, cfg.F), cfg.emb_var)
    else:
        out["x"] = mat(dr.normal((B, T, D), 1.0))
    blocks: List[dict] = []
    for _ in range(cfg.L):
        blk = {
            "ln1_g": np.ones(D, np.float32), "ln1_b": np.zeros(D, np.float32),
            "ln2_g": np.ones(D, np.float32), "ln2_b": np.zeros(D, np.float32),
        }
        if cfg.E == 0:
            Hd = cfg.k * D
            blk["w1"] = mat(dr.normal((T, Hd, D), 1.0 / D))
            blk["b1"] = dr.normal((T, Hd), cfg.bias_var) if cfg.bias_var else np.zeros((T, Hd), np.float32)
            blk["w2"] = mat(dr.normal((T, D, Hd), 1.0 / Hd))
            blk["b2"] = dr.normal((T, D), cfg.bias_var) if cfg.bias_var else np.zeros((T, D), np.float32)
        else:
            E, He = cfg.E, cfg.He
            blk["w1"] = mat(dr.normal((T, E, He, D), 1.0 / D))
            blk["b1"] = dr.normal((T, E, He), cfg.bias_var) if cfg.bias_var else np.zeros((T, E, He), np.float32)
            blk["w2"] = mat(dr.normal((T, E, D, He), 1.0 / He))
            blk["b2"] = dr.normal((T, E, D), cfg.bias_var) if cfg.bias_var else np.zeros((T, E, D), np.float32)
            blk["wr"] = mat(dr.normal((T, E, D), 1.0 / D))
            blk["br"] = np.full((T, E), MOE_ROUTER_BIAS, np.float32)
        blocks.append(blk)
    out["blocks"] = blocks
    if cfg.head:
        out["head"] = {"w": dr.normal((D,), 1.0 / D), "c": 0.0}
    return out


# the projection tokenizer's workload: the pad-split model's embedding
# (B = 4096 samples of F = 5000 floats ~ N(0, 0.1)) cut into T = 16 segments
# of seg = 320 floats (ceil(5000 / 16) = 313, rounded up to a multiple of 8),
# each mapped to D = 320
PROJ_WORKLOAD = dict(B=4096, F=5000, T=16, seg=320, D=320, dtype="bf16")


def make_proj_inputs(B: int, F: int, T: int, seg: int, D: int, dtype: str, seed: int = 2,
                     emb_var: float = 0.1, bias_var: float = 0.0) -> dict:
    """Draw the projection tokenizer's tensors: ``emb`` float32 [B,F] ~ N(0,
    emb_var); ``w`` [T,D,seg] ~ N(0, 1/seg) (uint16 bf16 bits for bf16);
    ``b`` float32 [T,D] ~ N(0, bias_var) (zeros when bias_var is 0)."""
    dr = _Drawer(seed)
    emb = dr.normal((B, F), emb_var)
    w = dr.normal((T, D, seg), 1.0 / seg)
    b = dr.normal((T, D), bias_var) if bias_var else np.zeros((T, D), np.float32)
    return {"emb": emb, "w": to_bf16_bits(w) if dtype == "bf16" else w, "b": b}


def make_variant_block(T: int, D: int, hidden: int, dtype: str, swiglu: bool = False, no_mix_norm: bool = False,
                       seed: int = 1) -> dict:
    """One block of the [TB] variants with the workload recipe: W ~ N(0,
    1/fan_in), zero biases, gamma = 1, beta = 0.  SwiGLU blocks get w1
    [T, 2*hidden, D] (gate rows, then up rows) and w2 [T, D, hidden]."""
    dr = _Drawer(seed)
    bf = dtype == "bf16"
    n1 = 2 * hidden if swiglu else hidden
    blk = {
        "w1": dr.normal((T, n1, D), 1.0 / D),
        "b1": np.zeros((T, n1), np.float32),
        "w2": dr.normal((T, D, hidden), 1.0 / hidden),
        "b2": np.zeros((T, D), np.float32),
        "ln1_g": np.ones(D, np.float32), "ln1_b": np.zeros(D, np.float32),
        "ln2_g": np.ones(D, np.float32), "ln2_b": np.zeros(D, np.float32),
    }
    if bf:
        blk["w1"] = to_bf16_bits(blk["w1"])
        blk["w2"] = to_bf16_bits(blk["w2"])
    if swiglu:
        blk["swiglu"] = True
    if no_mix_norm:
        blk["no_mix_norm"] = True
    return blk


# Training-router bias of the dense-training / sparse-inference MoE: with the
# same N(0, 1/D) weights the pre-activation is close to N(bias, 1), and a bias
# of +Phi^-1(0.75) leaves about 75 % of the training gates positive (the
# training router is the dense one; the inference router keeps
# MOE_ROUTER_BIAS, about 25 %).
MOE_TRAIN_ROUTER_BIAS = 0.6744897501960817


def add_training_router(blk: dict, dtype: str, seed: int = 7, bias: float = MOE_TRAIN_ROUTER_BIAS) -> dict:
    """A copy of MoE block ``blk`` with a training router: ``wr_train``
    [T,E,D] ~ N(0, 1/D) (uint16 bf16 bits for bf16) and ``br_train`` [T,E]
    filled with ``bias``."""
    T, E, D = blk["wr"].shape
    dr = _Drawer(seed)
    w = dr.normal((T, E, D), 1.0 / D)
    out = dict(blk)
    out["wr_train"] = to_bf16_bits(w) if dtype == "bf16" else w
    out["br_train"] = np.full((T, E), bias, np.float32)
    return out


def random_rows(B: int, n: int, seed: int = 12345) -> np.ndarray:
    """A seeded, sorted subset of n sample indices that always holds 0 and B-1."""
    if n >= B:
        return np.arange(B)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, B - 1), size=max(0, n - 2), replace=False)
    return np.unique(np.concatenate([[0, B - 1], mid])).astype(np.int64)

"""Seeded random model stacks for the shape sweep of rm_model_fwd.

Each case draws a dtype, a token count T (H = T heads), a head width (D = T
times it, a multiple of 8), a batch, up to three blocks of random kinds
(dense GELU FFN, SwiGLU, ReLU-routed MoE), hidden widths and expert counts
that differ from block to block, the Add & Norm after the mix switched off
now and then, the router bias at values that open about a quarter, none or
all of the gates, and, now and then, the pad-split tokenizer in front and the
pooled logit head behind.  The batch is cut so the fp64 oracle finishes a
case in well under a second.  Nothing here computes any part of the method:
it only draws shapes and seeded N(0, sigma^2) tensors (bf16 bit patterns for
the weight matrices of bf16 stacks)."""
import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

import synthetic_inputs as si

TS = (1, 2, 3, 4, 5, 6, 8, 12, 16, 24, 32, 40)
# router biases: about 25 % of the gates open for z ~ N(0, 1), most closed,
# about half, nearly all
ROUTER_BIAS = (-0.6745, -3.0, 0.0, 3.0)
WORK_CAP = 1e9  # B * sum over blocks of T * D * hidden * (1, 2 or E)


@dataclass
class Case:
    seed: int
    dtype: str
    B: int
    T: int
    D: int
    spec: list  # (kind, hidden, E, no_mix_norm, router bias)
    F: int = 0
    head: bool = False
    blocks: List[dict] = field(default_factory=list)
    inp: Optional[np.ndarray] = None
    head_params: Optional[dict] = None

    def describe(self) -> str:
        kinds = ", ".join(f"{k} h{h}" + (f" E{e} br{br:+.2f}" if k == "moe" else "") + (" no-mix-norm" if n else "")
                          for k, h, e, n, br in self.spec)
        extra = (f", pad-split F={self.F}" if self.F else "") + (", head" if self.head else "")
        return f"seed {self.seed}: {self.dtype} B={self.B} T={self.T} D={self.D} [{kinds}]{extra}"


def _block(rng, kind, T, D, H, E, nmn, br, dtype):
    if kind == "moe":
        p = {"w1": rng.standard_normal((T, E, H, D)) / math.sqrt(D), "b1": 0.1 * rng.standard_normal((T, E, H)),
             "w2": rng.standard_normal((T, E, D, H)) / math.sqrt(H), "b2": 0.1 * rng.standard_normal((T, E, D)),
             "wr": rng.standard_normal((T, E, D)) / math.sqrt(D), "br": np.full((T, E), br)}
        mats = ("w1", "w2", "wr")
    else:
        n1 = 2 * H if kind == "swiglu" else H
        p = {"w1": rng.standard_normal((T, n1, D)) / math.sqrt(D), "b1": 0.1 * rng.standard_normal((T, n1)),
             "w2": rng.standard_normal((T, D, H)) / math.sqrt(H), "b2": 0.1 * rng.standard_normal((T, D))}
        mats = ("w1", "w2")
    for k in ("ln1", "ln2"):
        p[k + "_g"] = 1 + 0.1 * rng.standard_normal(D)
        p[k + "_b"] = 0.1 * rng.standard_normal(D)
    p = {k: v.astype(np.float32) for k, v in p.items()}
    if dtype == "bf16":
        for k in mats:
            p[k] = si.to_bf16_bits(p[k])
    if kind == "swiglu":
        p["swiglu"] = True
    if nmn:
        p["no_mix_norm"] = True
    return p


def draw(seed: int) -> Case:
    rng = np.random.default_rng(seed)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    T = int(rng.choice(TS))
    while True:
        D = T * int(rng.integers(1, 65))
        if D % 8 == 0 and 16 <= D <= 1024:
            break
    spec = []
    for _ in range(int(rng.integers(1, 4))):
        kind = str(rng.choice(["dense", "swiglu", "moe"], p=[0.4, 0.25, 0.35]))
        H = 8 * int(rng.integers(1, 49))
        E = int(rng.integers(1, 9)) if kind == "moe" else 0
        spec.append((kind, H, E, bool(rng.random() < 0.2), float(rng.choice(ROUTER_BIAS))))
    work = sum(T * D * H * (E if k == "moe" else 2 if k == "swiglu" else 1) for k, H, E, _, _ in spec)
    B = max(1, min(int(rng.integers(1, 400)), int(WORK_CAP // work)))
    F = int(rng.integers(1, T * D + 1)) if rng.random() < 0.3 else 0
    case = Case(seed, dtype, B, T, D, spec, F=F, head=bool(rng.random() < 0.4))
    case.blocks = [_block(rng, k, T, D, H, E, n, br, dtype) for k, H, E, n, br in spec]
    if F:
        case.inp = (math.sqrt(0.1) * rng.standard_normal((B, F))).astype(np.float32)
    else:
        x = rng.standard_normal((B, T, D)).astype(np.float32)
        case.inp = si.to_bf16_bits(x) if dtype == "bf16" else x
    if case.head:
        case.head_params = {"w": (rng.standard_normal(D) / D).astype(np.float32), "c": float(rng.standard_normal())}
    return case


SEEDS = tuple(range(1000, 1048))


# ---------------------------------------------------------------------------
# training: one dense (GELU FFN) or MoE block with the Add & Norm after the
# mix, its training forward and backward.  MoE routers keep every
# pre-activation far from the ReLU kink (biases +-3, |w . s| near 0.5), so
# the fp64 oracle and the kernels take the same gate decisions.

TRAIN_WORK_CAP = 1.5e8  # B * T * D * hidden * (E or 1)
# at least 16 samples: a per-token gradient is a sum over the batch, and over
# a handful of samples that sum can nearly cancel; in bf16 each summand
# carries the rounding of D-long dot products of rounded activations, so the
# error of a nearly cancelled token group, measured against the group's own
# norm, says nothing about the kernels (the same case in fp32 agrees to
# 1e-6).  The fixed tests cover B = 1 on short rows.
TRAIN_MIN_B = 16


@dataclass
class TrainCase:
    seed: int
    kind: str
    dtype: str
    B: int
    T: int
    D: int
    H: int
    E: int
    blk: dict = field(default_factory=dict)
    x: Optional[np.ndarray] = None
    d_out: Optional[np.ndarray] = None

    def describe(self) -> str:
        moe = f" E={self.E}" if self.kind == "moe" else ""
        return f"seed {self.seed}: {self.kind} {self.dtype} B={self.B} T={self.T} D={self.D} hidden={self.H}{moe}"


def _act(rng, shape, dtype):
    a = rng.standard_normal(shape).astype(np.float32)
    return si.to_bf16_bits(a) if dtype == "bf16" else a


def draw_train(seed: int) -> TrainCase:
    rng = np.random.default_rng(seed)
    kind = "moe" if rng.random() < 0.45 else "dense"
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    T = int(rng.choice(TS))
    while True:
        D = T * int(rng.integers(1, 97))
        if D % 8 == 0 and 16 <= D <= 768:
            break
    E = 0
    if kind == "moe":
        # the training path keeps T * E a multiple of 8
        E = int(rng.choice([e for e in range(1, 9) if (T * e) % 8 == 0]))
        H = 8 * int(rng.integers(1, 49))
    else:
        H = 8 * int(rng.integers(1, 65))
    B = int(rng.integers(TRAIN_MIN_B, 1100 if T <= 4 else 400))
    B = max(TRAIN_MIN_B, min(B, int(TRAIN_WORK_CAP // (T * D * H * max(E, 1)))))
    if rng.random() < 0.25:
        # the backward's transpose-free path: bf16, whole 64-row blocks of at
        # least 256 rows, widths of at least 256
        dtype, T = "bf16", int(rng.choice([1, 2]))
        D, H = int(rng.choice([256, 320, 384])), int(rng.choice([256, 320]))
        B = int(rng.choice([256, 320, 384]))
        if kind == "moe":
            E = 8 // T
    case = TrainCase(seed, kind, dtype, B, T, D, H, E)
    if kind == "moe":
        sign = np.where(rng.random((2, T, E)) < 0.6, 1.0, -1.0)
        p = {"w1": rng.standard_normal((T, E, H, D)) / math.sqrt(D), "b1": 0.1 * rng.standard_normal((T, E, H)),
             "w2": rng.standard_normal((T, E, D, H)) / math.sqrt(H), "b2": 0.1 * rng.standard_normal((T, E, D)),
             "wr": 0.5 * rng.standard_normal((T, E, D)) / math.sqrt(D), "br": 3.0 * sign[0],
             "wr_train": 0.5 * rng.standard_normal((T, E, D)) / math.sqrt(D), "br_train": 3.0 * sign[1]}
        mats = ("w1", "w2", "wr", "wr_train")
    else:
        p = {"w1": rng.standard_normal((T, H, D)) / math.sqrt(D), "b1": 0.1 * rng.standard_normal((T, H)),
             "w2": rng.standard_normal((T, D, H)) / math.sqrt(H), "b2": 0.1 * rng.standard_normal((T, D))}
        mats = ("w1", "w2")
    for k in ("ln1", "ln2"):
        p[k + "_g"] = 1 + 0.1 * rng.standard_normal(D)
        p[k + "_b"] = 0.1 * rng.standard_normal(D)
    p = {k: v.astype(np.float32) for k, v in p.items()}
    if dtype == "bf16":
        for k in mats:
            p[k] = si.to_bf16_bits(p[k])
    case.blk = p
    case.x = _act(rng, (B, T, D), dtype)
    case.d_out = _act(rng, (B, T, D), dtype)
    return case


TRAIN_SEEDS = tuple(range(2000, 2032))

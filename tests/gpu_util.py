"""Shared helpers of the GPU parity tests: building/loading the library,
cached seeded inputs, the relative-L2 metric."""
import functools
import os
import sys

import numpy as np
import torch

import synthetic_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

TOL = {"f32": 1e-4, "bf16": 2e-2}  # max relative L2 error per sample


def note(msg: str) -> None:
    """Name the case on the real stderr before a GPU step (survives capture)."""
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


def ensure_lib():
    """The built library, refusing one built from other sources than the
    tree's (GPU runs never compile: build on the host first)."""
    from rankmixer_token_mixing_amd import binding as bd
    bd.check_fresh()
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return bd.load()


@functools.lru_cache(maxsize=2)
def config_inputs(name: str) -> dict:
    return si.make_inputs(si.CONFIGS[name])


def rel_l2_rows(y, ref) -> float:
    """max over samples b of ||y_b - ref_b|| / ||ref_b|| (first axis = samples)."""
    y = np.asarray(y, dtype=np.float64).reshape(len(y), -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(len(ref), -1)
    num = np.linalg.norm(y - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    return float((num / den).max())


def rel_l2(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> float64 numpy (exact for bf16 and fp32)."""
    return t.detach().to(torch.float64).cpu().numpy()


def rel_l2_groups(y, ref, n_lead: int, floor: float = 0.25) -> float:
    """max over the groups indexed by the leading n_lead axes (the token t, or
    the (token, expert) pair) of each group's L2 error, relative to the
    larger of the group's own norm and `floor` times the root-mean-square
    group norm.  An error confined to one group's tile is not diluted by the
    others; the floor keeps a group whose gradient nearly cancels (one sample,
    a gate barely open) from being judged on the rounding of that
    cancellation, while a wrong tile still reads as an O(1) error."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    k = int(np.prod(ref.shape[:n_lead]))
    y = y.reshape(k, -1)
    ref = ref.reshape(k, -1)
    num = np.linalg.norm(y - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    rms = float(np.sqrt(np.mean(den * den)))
    if rms == 0.0:
        return 0.0 if not num.any() else float("inf")
    return float((num / np.maximum(den, floor * rms)).max())

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
    from rankmixer_token_mixing_amd import binding as bd
    if not os.path.exists(bd.lib_path()):
        from rankmixer_token_mixing_amd.build import build
        build()
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

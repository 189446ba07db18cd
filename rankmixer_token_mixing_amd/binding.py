"""ctypes binding of librankmixer.so.

Argument marshalling only: torch device tensors in, pointers and sizes to the
C entry points of include/rankmixer.h, results in freshly allocated torch
tensors.  Every step of the forward runs in the library's HIP kernels; there
is no fallback path.  If the library is missing, the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import threading
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))

RM_OK, RM_ERR_INVALID, RM_ERR_UNSUPPORTED, RM_ERR_WORKSPACE, RM_ERR_HIP = range(5)
RM_F32, RM_BF16 = 0, 1
RM_BLOCK_DENSE, RM_BLOCK_MOE, RM_BLOCK_SWIGLU = 0, 1, 2
RM_BLOCK_NO_MIX_NORM = 1
_DT = {torch.float32: RM_F32, torch.bfloat16: RM_BF16}


class RankMixerError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


# ---------------------------------------------------------------------------
# C structs (layout of include/rankmixer.h)


class PffnParams(C.Structure):
    _fields_ = [("w1", C.c_void_p), ("b1", C.c_void_p), ("w2", C.c_void_p), ("b2", C.c_void_p)]


class ProjParams(C.Structure):
    _fields_ = [("w", C.c_void_p), ("b", C.c_void_p)]


class MoeParams(C.Structure):
    _fields_ = [("wr", C.c_void_p), ("br", C.c_void_p), ("w1", C.c_void_p), ("b1", C.c_void_p),
                ("w2", C.c_void_p), ("b2", C.c_void_p)]


class BlockParams(C.Structure):
    _fields_ = [("kind", C.c_int), ("ln1_g", C.c_void_p), ("ln1_b", C.c_void_p), ("ln2_g", C.c_void_p),
                ("ln2_b", C.c_void_p), ("pffn", PffnParams), ("moe", MoeParams), ("flags", C.c_int),
                ("hidden", C.c_int), ("E", C.c_int)]


class BlockGrads(C.Structure):
    _fields_ = [("w1", C.c_void_p), ("b1", C.c_void_p), ("w2", C.c_void_p), ("b2", C.c_void_p),
                ("ln1_g", C.c_void_p), ("ln1_b", C.c_void_p), ("ln2_g", C.c_void_p), ("ln2_b", C.c_void_p)]


class MoeGrads(C.Structure):
    _fields_ = [(k, C.c_void_p) for k in ("w1", "b1", "w2", "b2", "wr_train", "br_train", "wr_infer", "br_infer",
                                          "ln1_g", "ln1_b", "ln2_g", "ln2_b")]


class ModelDesc(C.Structure):
    _fields_ = [("T", C.c_int), ("D", C.c_int), ("dtype", C.c_int), ("L", C.c_int),
                ("blocks", C.POINTER(BlockParams)), ("F", C.c_int64), ("head_w", C.c_void_p), ("head_c", C.c_float)]


_vp, _i64, _int, _sz = C.c_void_p, C.c_int64, C.c_int, C.c_size_t

_SIGNATURES = {
    "rm_tokenize_padsplit": (_int, [_vp, _i64, _i64, _int, _int, _int, _vp, _vp]),
    "rm_tokenize_project": (_int, [_vp, C.POINTER(ProjParams), _i64, _i64, _int, _int, _int, _int, _vp, _vp, _sz,
                                   _vp]),
    "rm_tokenize_project_workspace_bytes": (_sz, [_i64, _i64, _int, _int, _int]),
    "rm_token_mix": (_int, [_vp, _vp, _i64, _int, _int, _int, _vp]),
    "rm_pffn_fwd": (_int, [_vp, C.POINTER(PffnParams), _vp, _i64, _int, _int, _int, _int, _vp, _sz, _vp]),
    "rm_pffn_workspace_bytes": (_sz, [_i64, _int, _int, _int, _int]),
    "rm_moe_relu_fwd": (_int, [_vp, C.POINTER(MoeParams), _vp, _vp, _i64, _int, _int, _int, _int, _int, _vp, _sz,
                               _vp]),
    "rm_moe_workspace_bytes": (_sz, [_i64, _int, _int, _int, _int, _int]),
    "rm_moe_route": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _int, _int, _int, _int, _vp, _sz, _vp]),
    "rm_block_fwd": (_int, [_vp, C.POINTER(BlockParams), _vp, _i64, _int, _int, _int, _int, _int, _vp, _sz, _vp]),
    "rm_block_workspace_bytes": (_sz, [_int, _i64, _int, _int, _int, _int, _int]),
    "rm_block_saved_bytes": (_sz, [_i64, _int, _int, _int, _int]),
    "rm_block_fwd_train": (_int, [_vp, C.POINTER(BlockParams), _vp, _vp, _sz, _i64, _int, _int, _int, _int, _vp,
                                  _sz, _vp]),
    "rm_block_bwd_workspace_bytes": (_sz, [_i64, _int, _int, _int, _int]),
    "rm_block_bwd": (_int, [_vp, C.POINTER(BlockParams), _vp, _sz, _vp, _vp, C.POINTER(BlockGrads), _i64, _int, _int,
                            _int, _int, _vp, _sz, _vp]),
    "rm_moe_saved_bytes": (_sz, [_i64, _int, _int, _int, _int, _int]),
    "rm_moe_train_workspace_bytes": (_sz, [_i64, _int, _int, _int, _int, _int]),
    "rm_moe_block_fwd_train": (_int, [_vp, C.POINTER(BlockParams), _vp, _vp, _vp, _vp, _vp, _sz, _i64, _int, _int,
                                      _int, _int, _int, _vp, _sz, _vp]),
    "rm_moe_block_bwd": (_int, [_vp, C.POINTER(BlockParams), _vp, _vp, C.c_float, _vp, _sz, _vp, _vp,
                                C.POINTER(MoeGrads), _i64, _int, _int, _int, _int, _int, _vp, _sz, _vp]),
    "rm_model_fwd": (_int, [C.POINTER(ModelDesc), _vp, _vp, _vp, _vp, _i64, _vp, _sz, _vp]),
    "rm_model_workspace_bytes": (_sz, [C.POINTER(ModelDesc), _i64]),
    "rm_status_string": (C.c_char_p, [_int]),
    "rm_last_error": (C.c_char_p, []),
    "rm_version": (C.c_char_p, []),
    "rm_probe_mfma_frag_bytes": (_sz, []),
    "rm_probe_mfma_out_floats": (_i64, []),
    "rm_probe_mfma_flop": (C.c_double, [_int]),
    "rm_probe_mfma_bf16": (_int, [_vp, _vp, _int, _vp]),
    "rm_probe_kstep_slab_bytes": (_sz, []),
    "rm_probe_kstep_out_floats": (_i64, []),
    "rm_probe_kstep_flop": (C.c_double, [_int]),
    "rm_probe_kstep_bf16": (_int, [_vp, _vp, _int, _vp]),
    "rm_probe_copy": (_int, [_vp, _vp, _sz, _vp]),
    "rm_moe_route_noalloc_scratch_bytes": (_sz, [_i64, _int, _int]),
    "rm_moe_route_noalloc_max_scratch_bytes": (_sz, []),
    "rm_moe_route_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _int, _int, _int, _int, _vp]),
    "rm_set_epilogue_overlap": (_int, [_int]),
    "rm_get_epilogue_overlap": (_int, []),
    "rm_audit_enable": (_int, [_int]),
    "rm_audit_count": (_int, []),
    "rm_audit_read": (_int, [_int, C.c_char_p, _sz, C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]),
    "rm_profile_enable": (_int, [_int]),
    "rm_profile_only": (_int, [C.c_char_p]),
    "rm_profile_count": (_int, []),
    "rm_profile_read": (_int, [_int, C.c_char_p, _sz, C.POINTER(C.c_double), C.POINTER(C.c_int)]),
}

_lib = None
_lock = threading.Lock()


def lib_path() -> str:
    return os.environ.get("RANKMIXER_LIB", os.path.join(_PKG, "librankmixer.so"))


def load():
    """Load librankmixer.so once (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise RankMixerError(RM_ERR_HIP, f"{path} is missing: build it with "
                                                 "`python -m rankmixer_token_mixing_amd.build`")
            lib = C.CDLL(path)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def check_fresh() -> None:
    """Raise if the loaded library was built from other sources than the
    ones in this tree (rm_version carries the hash of what it was built from)."""
    from rankmixer_token_mixing_amd.build import source_hash
    built = load().rm_version().decode().rsplit(" src ", 1)[-1]
    want = source_hash()
    if built != want:
        raise RankMixerError(RM_ERR_HIP, f"{lib_path()} was built from sources {built}, the tree holds {want}: "
                                         "rebuild with `python -m rankmixer_token_mixing_amd.build`")


def _check(status: int) -> None:
    if status != RM_OK:
        lib = load()
        raise RankMixerError(status, lib.rm_last_error().decode() or lib.rm_status_string(status).decode())


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to librankmixer must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


# one workspace per device, grown on demand (caller-owned memory of the C ABI)
_ws: Dict[int, torch.Tensor] = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    idx = device.index if device.index is not None else torch.cuda.current_device()
    cur = _ws.get(idx)
    if cur is None or cur.numel() < nbytes:
        _ws.pop(idx, None)
        cur = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws[idx] = cur
    return cur


def workspace_bytes(op: str, **kw) -> int:
    lib = load()
    dt = kw.get("dtype", RM_BF16)
    if op == "pffn":
        return lib.rm_pffn_workspace_bytes(kw["B"], kw["T"], kw["D"], kw["hidden"], dt)
    if op == "moe":
        return lib.rm_moe_workspace_bytes(kw["B"], kw["T"], kw["D"], kw["E"], kw["hidden"], dt)
    if op == "block":
        return lib.rm_block_workspace_bytes(kw["kind"], kw["B"], kw["T"], kw["D"], kw["hidden"], kw.get("E", 0), dt)
    raise ValueError(op)


# ---------------------------------------------------------------------------
# parameter structs from dicts of device tensors


def _pffn_struct(p: dict) -> PffnParams:
    return PffnParams(_p(p["w1"]), _p(p["b1"]), _p(p["w2"]), _p(p["b2"]))


def _moe_struct(p: dict) -> MoeParams:
    return MoeParams(_p(p["wr"]), _p(p["br"]), _p(p["w1"]), _p(p["b1"]), _p(p["w2"]), _p(p["b2"]))


def _block_struct(p: dict) -> BlockParams:
    """Block dict -> rm_block_params: a router ("wr") makes it an MoE block,
    "swiglu": True a SwiGLU block, "no_mix_norm": True sets the flag; hidden
    and E are the block's own widths, read off its weights."""
    moe = "wr" in p
    bp = BlockParams()
    bp.kind = RM_BLOCK_MOE if moe else (RM_BLOCK_SWIGLU if p.get("swiglu") else RM_BLOCK_DENSE)
    bp.flags = RM_BLOCK_NO_MIX_NORM if p.get("no_mix_norm") else 0
    bp.hidden, bp.E = _block_dims(p)
    bp.ln1_g, bp.ln1_b, bp.ln2_g, bp.ln2_b = _p(p["ln1_g"]), _p(p["ln1_b"]), _p(p["ln2_g"]), _p(p["ln2_b"])
    if moe:
        bp.moe = _moe_struct(p)
    else:
        bp.pffn = _pffn_struct(p)
    return bp


def _block_dims(p: dict):
    """(hidden, E) of a block's parameter dict."""
    if "wr" in p:
        return int(p["w1"].shape[2]), int(p["w1"].shape[1])
    if p.get("swiglu"):
        return int(p["w1"].shape[1]) // 2, 0
    return int(p["w1"].shape[1]), 0


def check_block(p: dict, T: int, D: int, dtype) -> None:
    """Every tensor of a block dict has the shape and dtype its widths imply
    (the C side sees only pointers, so a short tensor would be read past its
    end): weight matrices in the activation dtype, vectors fp32."""
    hidden, E = _block_dims(p)
    if "wr" in p:
        shapes = {"wr": (T, E, D), "br": (T, E), "w1": (T, E, hidden, D), "b1": (T, E, hidden),
                  "w2": (T, E, D, hidden), "b2": (T, E, D)}
        mats = ("wr", "w1", "w2")
    else:
        n1 = 2 * hidden if p.get("swiglu") else hidden
        shapes = {"w1": (T, n1, D), "b1": (T, n1), "w2": (T, D, hidden), "b2": (T, D)}
        mats = ("w1", "w2")
    shapes.update({k: (D,) for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b")})
    for k, shp in shapes.items():
        t = p[k]
        if tuple(t.shape) != shp:
            raise ValueError(f"block tensor {k} has shape {tuple(t.shape)}, expected {shp}")
        want = dtype if k in mats else torch.float32
        if t.dtype != want:
            raise ValueError(f"block tensor {k} is {t.dtype}, expected {want}")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)


def rm_tokenize_padsplit(emb: torch.Tensor, T: int, D: int, out_dtype=torch.bfloat16) -> torch.Tensor:
    B, F = emb.shape
    x0 = torch.empty((B, T, D), dtype=out_dtype, device=emb.device)
    _check(load().rm_tokenize_padsplit(_p(emb), B, F, T, D, _DT[out_dtype], _p(x0), _stream(emb.device)))
    return x0


def rm_tokenize_project(emb: torch.Tensor, p: dict, T: int, seg: int, out_dtype=torch.bfloat16,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """p: {"w": [T][D][seg] out_dtype, "b": [T][D] fp32} device tensors."""
    lib = load()
    B, F = emb.shape
    D = p["w"].shape[1]
    if p["w"].dtype != out_dtype or tuple(p["w"].shape) != (T, D, seg):
        raise ValueError("w must be [T][D][seg] in the output dtype")
    x0 = torch.empty((B, T, D), dtype=out_dtype, device=emb.device) if out is None else out
    n = lib.rm_tokenize_project_workspace_bytes(B, F, T, seg, _DT[out_dtype])
    ws = _workspace(emb.device, n)
    st = ProjParams(_p(p["w"]), _p(p["b"]))
    _check(lib.rm_tokenize_project(_p(emb), C.byref(st), B, F, T, seg, D, _DT[out_dtype], _p(x0), _p(ws),
                                   ws.numel(), _stream(emb.device)))
    return x0


def rm_token_mix(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    B, T, D = x.shape
    y = torch.empty_like(x) if out is None else out
    _check(load().rm_token_mix(_p(x), _p(y), B, T, D, _dt(x), _stream(x.device)))
    return y


def rm_pffn_fwd(s: torch.Tensor, p: dict, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    B, T, D = s.shape
    Hd = p["w1"].shape[1]
    v = torch.empty_like(s) if out is None else out
    n = lib.rm_pffn_workspace_bytes(B, T, D, Hd, _dt(s))
    ws = _workspace(s.device, n)
    st = _pffn_struct(p)
    _check(lib.rm_pffn_fwd(_p(s), C.byref(st), _p(v), B, T, D, Hd, _dt(s), _p(ws), ws.numel(), _stream(s.device)))
    return v


def rm_moe_relu_fwd(s: torch.Tensor, p: dict, return_gates: bool = False, out: Optional[torch.Tensor] = None):
    lib = load()
    B, T, D = s.shape
    E, He = p["w1"].shape[1], p["w1"].shape[2]
    v = torch.empty_like(s) if out is None else out
    gates = torch.empty((B, T, E), dtype=torch.float32, device=s.device) if return_gates else None
    n = lib.rm_moe_workspace_bytes(B, T, D, E, He, _dt(s))
    ws = _workspace(s.device, n)
    st = _moe_struct(p)
    _check(lib.rm_moe_relu_fwd(_p(s), C.byref(st), _p(v), _p(gates), B, T, D, E, He, _dt(s), _p(ws), ws.numel(),
                               _stream(s.device)))
    return (v, gates) if return_gates else v


def rm_moe_route(s: torch.Tensor, wr: torch.Tensor, br: torch.Tensor):
    """Returns (gates [B,T,E] fp32, offsets [T*E+1] int32, rows [B*T*E] int32);
    only rows[:offsets[-1]] is written."""
    lib = load()
    B, T, D = s.shape
    E = wr.shape[1]
    gates = torch.empty((B, T, E), dtype=torch.float32, device=s.device)
    offsets = torch.empty(T * E + 1, dtype=torch.int32, device=s.device)
    rows = torch.empty(B * T * E, dtype=torch.int32, device=s.device)
    n = lib.rm_moe_workspace_bytes(B, T, D, E, 8, _dt(s))
    ws = _workspace(s.device, n)
    _check(lib.rm_moe_route(_p(s), _p(wr), _p(br), _p(gates), _p(offsets), _p(rows), B, T, D, E, _dt(s), _p(ws),
                            ws.numel(), _stream(s.device)))
    return gates, offsets, rows


def rm_moe_route_noalloc(s: torch.Tensor, wr: torch.Tensor, br: torch.Tensor, gates: torch.Tensor,
                         offsets: torch.Tensor, rows: torch.Tensor) -> None:
    """rm_moe_route into caller-allocated outputs (gates [B,T,E] fp32, offsets
    [T*E+1] int32, rows [B*T*E] int32) with the library's fixed scratch."""
    B, T, D = s.shape
    E = wr.shape[1]
    _check(load().rm_moe_route_noalloc(_p(s), _p(wr), _p(br), _p(gates), _p(offsets), _p(rows), B, T, D, E, _dt(s),
                                       _stream(s.device)))


def rm_block_fwd(x: torch.Tensor, p: dict, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = load()
    B, T, D = x.shape
    check_block(p, T, D, x.dtype)
    hidden, E = _block_dims(p)
    bp = _block_struct(p)
    y = torch.empty_like(x) if out is None else out
    n = lib.rm_block_workspace_bytes(bp.kind, B, T, D, hidden, E, _dt(x))
    ws = _workspace(x.device, n)
    _check(lib.rm_block_fwd(_p(x), C.byref(bp), _p(y), B, T, D, hidden, E, _dt(x), _p(ws), ws.numel(),
                            _stream(x.device)))
    return y


def rm_block_fwd_train(x: torch.Tensor, p: dict, out: Optional[torch.Tensor] = None):
    """Dense block forward that also returns the buffer rm_block_bwd needs:
    (x_out, saved)."""
    lib = load()
    B, T, D = x.shape
    Hd = p["w1"].shape[1]
    y = torch.empty_like(x) if out is None else out
    saved = torch.empty(lib.rm_block_saved_bytes(B, T, D, Hd, _dt(x)), dtype=torch.uint8, device=x.device)
    n = lib.rm_block_workspace_bytes(RM_BLOCK_DENSE, B, T, D, Hd, 0, _dt(x))
    ws = _workspace(x.device, n)
    st = _block_struct(p)
    _check(lib.rm_block_fwd_train(_p(x), C.byref(st), _p(y), _p(saved), saved.numel(), B, T, D, Hd, _dt(x), _p(ws),
                                  ws.numel(), _stream(x.device)))
    return y, saved


def rm_block_bwd(x: torch.Tensor, p: dict, saved: torch.Tensor, d_out: torch.Tensor):
    """Dense block backward: (dx, grads) with grads a dict of fp32 tensors
    named like the parameters (w1, b1, w2, b2, ln1_g, ln1_b, ln2_g, ln2_b)."""
    lib = load()
    B, T, D = x.shape
    Hd = p["w1"].shape[1]
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"w1": torch.empty((T, Hd, D), **f32), "b1": torch.empty((T, Hd), **f32),
         "w2": torch.empty((T, D, Hd), **f32), "b2": torch.empty((T, D), **f32),
         "ln1_g": torch.empty(D, **f32), "ln1_b": torch.empty(D, **f32),
         "ln2_g": torch.empty(D, **f32), "ln2_b": torch.empty(D, **f32)}
    dx = torch.empty_like(x)
    gs = BlockGrads(*[_p(g[k]) for k in ("w1", "b1", "w2", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")])
    n = lib.rm_block_bwd_workspace_bytes(B, T, D, Hd, _dt(x))
    ws = _workspace(dev, n)
    st = _block_struct(p)
    _check(lib.rm_block_bwd(_p(x), C.byref(st), _p(saved), saved.numel(), _p(d_out), _p(dx), C.byref(gs), B, T, D, Hd,
                            _dt(x), _p(ws), ws.numel(), _stream(dev)))
    return dx, g


MOE_GRADS = ("w1", "b1", "w2", "b2", "wr_train", "br_train", "wr", "br", "ln1_g", "ln1_b", "ln2_g", "ln2_b")


def rm_moe_block_fwd_train(x: torch.Tensor, p: dict, out: Optional[torch.Tensor] = None):
    """MoE block training forward (dense-training / sparse-inference routers).
    p: an MoE block dict (its "wr"/"br" are h_infer) plus "wr_train" [T][E][D]
    in x's dtype and "br_train" [T][E] fp32.  Returns (x_out, l_reg [1] fp32,
    saved)."""
    lib = load()
    B, T, D = x.shape
    He, E = _block_dims(p)
    y = torch.empty_like(x) if out is None else out
    l_reg = torch.empty(1, dtype=torch.float32, device=x.device)
    saved = torch.empty(max(lib.rm_moe_saved_bytes(B, T, D, He, E, _dt(x)), 16), dtype=torch.uint8, device=x.device)
    ws = _workspace(x.device, lib.rm_moe_train_workspace_bytes(B, T, D, He, E, _dt(x)))
    st = _block_struct(p)
    _check(lib.rm_moe_block_fwd_train(_p(x), C.byref(st), _p(p["wr_train"]), _p(p["br_train"]), _p(y), _p(l_reg),
                                      _p(saved), saved.numel(), B, T, D, He, E, _dt(x), _p(ws), ws.numel(),
                                      _stream(x.device)))
    return y, l_reg, saved


def rm_moe_block_bwd(x: torch.Tensor, p: dict, saved: torch.Tensor, d_out: torch.Tensor, lam: float):
    """MoE block backward of <d_out, x_out> + lam * L_reg: (dx, grads), grads
    a dict of fp32 tensors named like the parameters (MOE_GRADS; "wr"/"br"
    are h_infer's)."""
    lib = load()
    B, T, D = x.shape
    He, E = _block_dims(p)
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    shapes = {"w1": (T, E, He, D), "b1": (T, E, He), "w2": (T, E, D, He), "b2": (T, E, D),
              "wr_train": (T, E, D), "br_train": (T, E), "wr": (T, E, D), "br": (T, E),
              "ln1_g": (D,), "ln1_b": (D,), "ln2_g": (D,), "ln2_b": (D,)}
    g = {k: torch.empty(shapes[k], **f32) for k in MOE_GRADS}
    dx = torch.empty_like(x)
    gs = MoeGrads(*[_p(g[k]) for k in MOE_GRADS])
    ws = _workspace(dev, lib.rm_moe_train_workspace_bytes(B, T, D, He, E, _dt(x)))
    st = _block_struct(p)
    _check(lib.rm_moe_block_bwd(_p(x), C.byref(st), _p(p["wr_train"]), _p(p["br_train"]), float(lam), _p(saved),
                                saved.numel(), _p(d_out), _p(dx), C.byref(gs), B, T, D, He, E, _dt(x), _p(ws),
                                ws.numel(), _stream(dev)))
    return dx, g


class Model:
    """A model descriptor kept alive across calls (blocks, head, dims)."""

    def __init__(self, blocks: Sequence[dict], T: int, D: int, dtype=torch.bfloat16, F: int = 0,
                 head: Optional[dict] = None):
        self.blocks = list(blocks)
        # each block carries its own hidden width and expert count
        for b in self.blocks:
            check_block(b, T, D, dtype)
        if head is not None and (tuple(head["w"].shape) != (D,) or head["w"].dtype != torch.float32):
            raise ValueError("head w must be a [D] fp32 tensor")
        self._arr = (BlockParams * max(1, len(self.blocks)))(*[_block_struct(b) for b in self.blocks])
        self.head = head
        self.desc = ModelDesc(T, D, _DT[dtype], len(self.blocks), self._arr, F,
                              _p(head["w"]) if head else None, float(head["c"]) if head else 0.0)
        self.T, self.D, self.dtype, self.F = T, D, dtype, F

    def workspace_bytes(self, B: int) -> int:
        return load().rm_model_workspace_bytes(C.byref(self.desc), B)


def rm_model_fwd(model: Model, inp: torch.Tensor, want_x: bool = True, want_pooled: bool = False,
                 out: Optional[dict] = None) -> dict:
    lib = load()
    B = inp.shape[0]
    dev = inp.device
    res = out if out is not None else {}
    if want_x and "x" not in res:
        res["x"] = torch.empty((B, model.T, model.D), dtype=model.dtype, device=dev)
    if model.head is not None:
        if "logit" not in res:
            res["logit"] = torch.empty(B, dtype=torch.float32, device=dev)
        if want_pooled and "pooled" not in res:
            res["pooled"] = torch.empty((B, model.D), dtype=torch.float32, device=dev)
    n = lib.rm_model_workspace_bytes(C.byref(model.desc), B)
    ws = _workspace(dev, n)
    _check(lib.rm_model_fwd(C.byref(model.desc), _p(inp), _p(res.get("x")), _p(res.get("pooled")),
                            _p(res.get("logit")), B, _p(ws), ws.numel(), _stream(dev)))
    return res


def probe_mfma_bf16(frags: torch.Tensor, out: torch.Tensor, iters: int) -> None:
    """The MFMA ceiling probe (see rm_probe_mfma_bf16); frags: random bytes of
    rm_probe_mfma_frag_bytes(), out: rm_probe_mfma_out_floats() fp32."""
    _check(load().rm_probe_mfma_bf16(_p(frags), _p(out), iters, _stream(frags.device)))


def probe_kstep_bf16(slab: torch.Tensor, out: torch.Tensor, iters: int) -> None:
    """The k-step probe (see rm_probe_kstep_bf16); slab: rm_probe_kstep_slab_bytes()
    bytes of bf16, out: rm_probe_kstep_out_floats() fp32."""
    _check(load().rm_probe_kstep_bf16(_p(slab), _p(out), iters, _stream(slab.device)))


def probe_copy(src: torch.Tensor, dst: torch.Tensor, nbytes: int) -> None:
    _check(load().rm_probe_copy(_p(src), _p(dst), nbytes, _stream(src.device)))


def set_epilogue_overlap(on: bool) -> None:
    """The bf16 products' epilogue mode (rm_set_epilogue_overlap)."""
    _check(load().rm_set_epilogue_overlap(1 if on else 0))


def get_epilogue_overlap() -> bool:
    return bool(load().rm_get_epilogue_overlap())


def profile_enable(on: bool = True) -> None:
    _check(load().rm_profile_enable(1 if on else 0))


def profile_only(name: Optional[str] = None) -> None:
    """Record only the launch groups called `name` (None: every group)."""
    _check(load().rm_profile_only(name.encode() if name else None))


def profile_read() -> Dict[str, tuple]:
    """{name: (total_ms, launches)} of the launch groups timed since enabling."""
    lib = load()
    out = {}
    buf = C.create_string_buffer(128)
    for i in range(lib.rm_profile_count()):
        tot = C.c_double()
        n = C.c_int()
        _check(lib.rm_profile_read(i, buf, 128, C.byref(tot), C.byref(n)))
        out[buf.value.decode()] = (tot.value, n.value)
    return out


# ---------------------------------------------------------------------------
# numpy arrays from synthetic_inputs -> device tensors


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """uint16 arrays are bf16 bit patterns; everything else keeps its dtype."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def upload_blocks(blocks: List[dict], device="cuda") -> List[dict]:
    """Arrays to device tensors; flags ("swiglu", "no_mix_norm") pass through."""
    return [{k: (to_device(v, device) if isinstance(v, np.ndarray) else v) for k, v in b.items()} for b in blocks]

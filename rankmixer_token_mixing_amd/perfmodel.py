"""Algorithmic work of each step: the flops and bytes the method must spend,
used to turn measured times into TFLOP/s, GB/s and roofline fractions.

Flops count every multiply-add of a matrix product as two operations
(2*M*N*K per product).  This is the count that reproduces the matrix GFLOPs
printed in Appendix B of "重新理解 RankMixer：扩参为什么有效，又为什么划算？"
(e.g. 6.442451 GFLOPs for the 3-layer 8x256-token Mixer at batch 256).
LayerNorm, GELU, bias and routing arithmetic are not counted as flops, the
same as that table's matrix-only numerator.
"""
from __future__ import annotations

# MI355X published peaks (dense, no sparsity).
PEAK_BF16_TFLOPS = 2516.6     # 2.5 PFLOP/s bf16/fp16 dense MFMA
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0         # HBM3E, 8 TB/s
ELEM_BYTES = {"bf16": 2, "f32": 4}


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def pffn_flops(B: int, T: int, D: int, Hd: int) -> int:
    """Two grouped products per token: [B,D]x[D,Hd] and [B,Hd]x[Hd,D]."""
    return T * (gemm_flops(B, Hd, D) + gemm_flops(B, D, Hd))


def block_flops(B: int, T: int, D: int, Hd: int) -> int:
    """Dense block: the token mix and LayerNorms add no matrix work."""
    return pffn_flops(B, T, D, Hd)


def moe_flops(active_pairs: int, B: int, T: int, D: int, E: int, He: int) -> int:
    """ReLU MoE: each active (sample, token, expert) runs one expert FFN
    (4*D*He); the router is a D -> E product for every (sample, token)."""
    return active_pairs * 4 * D * He + B * T * gemm_flops(1, E, D)


def block_params(T: int, D: int, k: int) -> int:
    """Per-token FFN weights of one block: 2*T*k*D^2 (biases excluded), as
    stated in "Rankmixer: 硬件效率优化", section "Per-Token FFN"."""
    return 2 * T * k * D * D


def token_mix_bytes(B: int, T: int, D: int, dtype: str) -> int:
    return 2 * B * T * D * ELEM_BYTES[dtype]


def tokenize_bytes(B: int, F: int, T: int, D: int, dtype: str) -> int:
    return B * F * 4 + B * T * D * ELEM_BYTES[dtype]


def block_min_bytes(B: int, T: int, D: int, Hd: int, dtype: str) -> int:
    """Compulsory HBM traffic of one dense block: read X and the weights once,
    write X' once (biases and LayerNorm vectors are negligible)."""
    e = ELEM_BYTES[dtype]
    return 2 * B * T * D * e + 2 * T * D * Hd * e


# --- the comparison backbones of Appendix B, for pinning the convention ----

def mixer_backbone_flops(batch: int, tokens: int, token_width: int, hidden: int, layers: int) -> int:
    return layers * tokens * (gemm_flops(batch, hidden, token_width) + gemm_flops(batch, token_width, hidden))


def dcn_flops(batch: int, width: int, layers: int) -> int:
    return layers * gemm_flops(batch, 1, width)


def dcnv2_full_flops(batch: int, width: int, layers: int) -> int:
    return layers * gemm_flops(batch, width, width)


def dcnv2_lowrank_flops(batch: int, width: int, rank: int, layers: int) -> int:
    return layers * (gemm_flops(batch, rank, width) + gemm_flops(batch, width, rank))


def project_bytes(B: int, F: int, T: int, seg: int, D: int, dtype: str) -> int:
    """Compulsory HBM traffic of the projection tokenizer: the fp32 embedding
    read once, the T weight matrices and biases read once, x0 written once."""
    e = ELEM_BYTES[dtype]
    return B * F * 4 + T * D * seg * e + T * D * 4 + B * T * D * e


def project_flops(B: int, T: int, seg: int, D: int) -> int:
    """T products [B, seg] x [seg, D] (the padded segment length counts)."""
    return T * gemm_flops(B, D, seg)

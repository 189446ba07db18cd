"""Writes gemm_defer_kstep.inc: the k-step bodies of the deferred-epilogue
grouped GEMM (kernels_gemm_defer.hip) as inline-asm functions.

    python rankmixer_token_mixing_amd/csrc/gemm_defer_gen.py

One k-step is 16 v_mfma_f32_32x32x16_bf16 (a wave's 4 x 4 grid of 32 x 32
blocks, 16 k), the eight fragment reads of the next k-step behind the first
eight MFMAs, 0, 4 or 8 LDS DMA ops behind the next ones, and optionally one
"unit" of the previous tile's epilogue -- four output values of one row,
held as two packed bf16 registers that already include the bias: unpack,
GELU, pack -- spread one value per four MFMAs, so the epilogue's ALU work
issues while the matrix cores run.  dk_bias_add adds the column bias to a
finished tile's accumulators with one MFMA per block.  The GELU is the same instruction sequence as gelu_erf in
common.hpp (x Phi(x) = max(x, 0) - |x| Phi(-|x|), Phi(-a) = exp2(P(min(a,
6.5)))), with the polynomial coefficients read from common.hpp, so the two
agree bit for bit.

The build does not run this script; the generated file is committed, and a
CPU test checks that it is what the script writes.
"""
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def tail_coefficients():
    """The seven coefficients of phi_tail_log2 in common.hpp, highest degree
    first, as fp32 bit patterns."""
    src = open(os.path.join(HERE, "common.hpp")).read()
    body = re.search(r"phi_tail_log2\(float ac\) \{(.*?)\n\}", src, re.S).group(1)
    vals = [float(x) for x in re.findall(r"(-?\d\.\d+e-\d+|-?\d+\.\d+)f", body)]
    assert len(vals) == 7, vals
    return [int(np.float32(v).view(np.uint32)) for v in vals]


C = tail_coefficients()  # C[0] degree 6 (in a register), C[1..6] degrees 5..0

# block b = 4 i + j of the wave's accumulators is AGPRs a[16 b : 16 b + 15],
# named in the asm text: the accumulators are never C++ values, every asm
# statement that touches them lists all 256 AGPRs as clobbered (so the kernel
# allocates them), and the build keeps the compiler from spilling into AGPRs
MF = "v_mfma_f32_32x32x16_bf16 a[{lo}:{hi}], %[w{j}], %[a{i}], {src}"
AGPR_CLOBBERS = ", ".join(f'"a{r}"' for r in range(256))


def gelu_value(e, x, p, hi):
    """Instructions of one value: x = bf16(p half), x = GELU(x)."""
    unpack = (f"v_and_b32 %[{x}], 0xffff0000, %[{p}]" if hi else f"v_lshlrev_b32 %[{x}], 16, %[{p}]")
    return [unpack, *gelu_core(x)]


def gelu_core(x):
    return [f"v_med3_f32 %[ua], |%[{x}]|, 0, %[us65]",
            f"v_fmaak_f32 %[ut], %[ua], %[uc6], 0x{C[1]:08x}",
            f"v_fmaak_f32 %[ut], %[ut], %[ua], 0x{C[2]:08x}",
            f"v_fmaak_f32 %[ut], %[ut], %[ua], 0x{C[3]:08x}",
            f"v_fmaak_f32 %[ut], %[ut], %[ua], 0x{C[4]:08x}",
            f"v_fmaak_f32 %[ut], %[ut], %[ua], 0x{C[5]:08x}",
            f"v_fmaak_f32 %[ut], %[ut], %[ua], 0x{C[6]:08x}",
            "v_exp_f32 %[ut], %[ut]",
            # one independent instruction between the transcendental and its use
            f"v_max_i32 %[ua], 0, %[{x}]",
            f"v_fma_f32 %[{x}], -|%[{x}]|, %[ut], %[ua]"]


def unit_stream():
    """Instruction lists of one GELU unit, one list per value (each spread
    over four MFMAs), the last list followed by the packs."""
    vals = [gelu_value(e, f"ux{e}", f"up{e // 2}", e % 2) for e in range(4)]
    vals[3] += ["v_cvt_pk_bf16_f32 %[uo0], %[ux0], %[ux1]", "v_cvt_pk_bf16_f32 %[uo1], %[ux2], %[ux3]"]
    return vals


def spread(lst, n):
    """Split lst into n consecutive chunks of near-equal size."""
    out, k = [], 0
    for i in range(n):
        m = (len(lst) - k) // (n - i)
        out.append(lst[k:k + m])
        k += m
    return out


# next-fragment reads in the order the next k-step's MFMAs consume them
READS = [("na0", "la", 0), ("nw0", "lb", 0), ("nw1", "lb", 4096), ("nw2", "lb", 8192), ("nw3", "lb", 12288),
         ("na1", "la", 4096), ("na2", "la", 8192), ("na3", "la", 12288)]


def kstep_asm(zero, ndma, epi):
    gaps = [[] for _ in range(16)]
    for m, (dst, base, off) in enumerate(READS):
        gaps[m].append(f"ds_read_b128 %[{dst}], %[{base}] offset:{off}")
    if ndma:
        # M0 (the LDS destination) is written at least one instruction before
        # the DMA that reads it: set in gap 6, advanced right after each DMA
        # (an MFMA follows before the next one)
        # Op d reads rows 32 d further than op 0: its lane offset is vo + d *
        # sblk, advanced in two temporaries in turn (each written one MFMA
        # after the DMA that last read it)
        gaps[6].append("s_mov_b32 m0, %[mb]")
        for d in range(ndma):
            g = gaps[8 + d]
            src = "vo" if d == 0 else f"vt{(d - 1) % 2}"
            g.append(f"global_load_lds_dwordx4 %[{src}], %[sb]")
            if d + 1 < ndma:
                g.append("s_add_u32 m0, m0, 4096")
                g.append(f"v_add_u32 %[vt{d % 2}], %[sblk], %[{src}]")
    if epi:
        for v, ins in enumerate(unit_stream()):
            for k, chunk in enumerate(spread(ins, 4)):
                gaps[4 * v + k] += chunk
    lines = []
    for m in range(16):
        i, j = divmod(m, 4)
        b = 4 * i + j
        acc = f"a[{16 * b}:{16 * b + 15}]"
        lines.append(MF.format(lo=16 * b, hi=16 * b + 15, i=i, j=j, src="0" if zero else acc))
        lines += gaps[m]
    lines.append("s_waitcnt lgkmcnt(0)")
    return lines


def agprs(b):
    return f"a[{16 * b}:{16 * b + 15}]"


def pack_function(b):
    """Block b's 16 accumulators (AGPRs 16 b .. 16 b + 15) as 8 packed bf16
    pairs: out[2 q], out[2 q + 1] = registers 4 q, 4 q + 1 and 4 q + 2, 4 q + 3."""
    lines = []
    for q in range(4):
        for h in range(2):
            r = 16 * b + 4 * q + 2 * h
            lines += [f"v_accvgpr_read_b32 %[t0], a{r}", f"v_accvgpr_read_b32 %[t1], a{r + 1}",
                      f"v_cvt_pk_bf16_f32 %[o{2 * q + h}], %[t0], %[t1]"]
    asm = "\n".join(f'      "{ln}\\n\\t"' for ln in lines)
    outs = ", ".join(f'[o{k}] "=&v"(out[{k}])' for k in range(8))
    return (f"__device__ __forceinline__ void dk_pack_b{b}(uint32_t (&out)[8]) {{\n"
            f"  float t0, t1;\n  asm volatile(\n{asm}\n      : {outs}, [t0] \"=&v\"(t0), [t1] \"=&v\"(t1)\n"
            f"      :\n      : DK_AGPRS);\n}}")


def function(zero, ndma, epi):
    name = f"dk_{'z' if zero else 'a'}_d{ndma}_{epi or 'none'}"
    args = ["const Frag8& cu", "Frag8& nx", "uint32_t la", "uint32_t lb"]
    if ndma:
        args += ["uint32_t mb", "uint32_t vo", "const void* sb", "uint32_t sblk"]
    if epi:
        args += ["uint32_t up0", "uint32_t up1", "uint32_t& uo0", "uint32_t& uo1", "float uc6", "float us65"]
    outs = [f'[n{s}{k}] "=&v"(nx.{s}{k})' for s in "aw" for k in range(4)]
    ins = [f'[{s}{k}] "v"(cu.{s}{k})' for s in "aw" for k in range(4)] + ['[la] "v"(la)', '[lb] "v"(lb)']
    body = []
    if epi:
        body.append("  float ux0, ux1, ux2, ux3, ua, ut;")
        outs += [f'[ux{e}] "=&v"(ux{e})' for e in range(4)] + ['[ua] "=&v"(ua)', '[ut] "=&v"(ut)',
                                                              '[uo0] "=&v"(uo0)', '[uo1] "=&v"(uo1)']
        ins += ['[up0] "v"(up0)', '[up1] "v"(up1)', '[uc6] "v"(uc6)', '[us65] "s"(us65)']
    if ndma:
        body.append("  uint32_t vt0, vt1;")
        outs += ['[vt0] "=&v"(vt0)', '[vt1] "=&v"(vt1)']
        ins += ['[mb] "s"(mb)', '[vo] "v"(vo)', '[sb] "s"(sb)', '[sblk] "s"(sblk)']
    clob = ('"m0", "scc", ' if ndma else "") + "DK_AGPRS"
    asm = "\n".join(f'      "{ln}\\n\\t"' for ln in kstep_asm(zero, ndma, epi))
    text = [f"__device__ __forceinline__ void {name}({', '.join(args)}) {{", *body, "  asm volatile(", asm,
            "      : " + ",\n        ".join(outs), "      : " + ",\n        ".join(ins)]
    text.append(f"      : {clob});")
    text.append("}")
    return "\n".join(text)


def bias_add_function():
    """acc(i, j) += W'_j x ONES over the 16 blocks: W'_j's lane with row lr
    holds, in its first two k elements, the bf16 high and low parts of the
    bias of block column j's column lr (zero elsewhere), ONES holds 1.0 in the
    same two k elements of every row, so every row of the block gains
    bias_hi + bias_lo, within 2^-17 of the fp32 bias."""
    lines = ["s_nop 4"]  # W' and ONES were just written by vector ALU code
    for b in range(16):
        i, j = divmod(b, 4)
        acc = f"a[{16 * b}:{16 * b + 15}]"
        lines.append(f"v_mfma_f32_32x32x16_bf16 {acc}, %[wb{j}], %[ones], {acc}")
    asm = "\n".join(f'      "{ln}\\n\\t"' for ln in lines)
    ins = ", ".join(f'[wb{j}] "v"(wb[{j}])' for j in range(4))
    return ("__device__ __forceinline__ void dk_bias_add(const u32x4 (&wb)[4], const u32x4& ones) {\n"
            f"  asm volatile(\n{asm}\n      :\n      : {ins}, [ones] \"v\"(ones)\n      : DK_AGPRS);\n}}")


def render() -> str:
    """The text of gemm_defer_kstep.inc."""
    parts = ["// Generated by gemm_defer_gen.py -- do not edit.  K-step bodies of the",
             "// deferred-epilogue grouped GEMM (kernels_gemm_defer.hip): dk_<z|a>_d<DMA ops>_<unit>",
             "// (z: accumulators start from zero; a: accumulate), dk_pack_b<block> and dk_bias_add.", "",
             "// every AGPR: the wave's accumulators, named in the asm text", f"#define DK_AGPRS {AGPR_CLOBBERS}", ""]
    for b in range(16):
        parts.append(pack_function(b))
        parts.append("")
    parts.append(bias_add_function())
    parts.append("")
    for epi in (None, "gelu"):
        for zero, ndma in ((True, 4), (False, 0), (False, 4), (False, 8)):
            parts.append(function(zero, ndma, epi))
            parts.append("")
    return "\n".join(parts)


def main():
    with open(os.path.join(HERE, "gemm_defer_kstep.inc"), "w") as f:
        f.write(render())


if __name__ == "__main__":
    main()

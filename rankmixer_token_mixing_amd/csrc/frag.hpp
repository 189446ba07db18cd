// MFMA operand staging shared by the GEMM kernels: LDS rows of eight 16-byte
// chunks, XOR-swizzled so that the 32-row fragment reads of a wave hit
// distinct banks, and the register / address-space types the kernels use.
#pragma once

#include <hip/hip_runtime.h>

namespace rm {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // one MFMA fragment (register operand)
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

constexpr int kCpr = 8;  // 16-byte chunks per LDS operand row

// uint4 index of logical chunk c of row `row`: physical chunk c ^ (row/2 mod 8)
__device__ __forceinline__ int swz(int row, int c) { return row * kCpr + (c ^ ((row >> 1) & 7)); }

// s_waitcnt vmcnt(n) only (expcnt / lgkmcnt untouched); n < 16
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(N | (7 << 4) | (15 << 8));
}

// one LDS DMA op on its own: 64 lanes x 16 bytes from sb + voff (per lane)
// into LDS at m0v (prologues)
__device__ __forceinline__ void dma1(uint32_t m0v, const void* sb, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %[m]\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %[v], %[sb]\n\t"
               :
               : [m] "s"(m0v), [sb] "s"(sb), [v] "v"(voff)
               : "m0");
}

// ---- the k-step of the pipelined products (N-major operands) ---------------
// One 16-wide k-step of a wave's 128 x 64 tile (4 x 2 blocks of 32 x 32) as
// one asm block: eight v_mfma_f32_32x32x16_bf16 on the current fragments,
// with the six 16-byte fragment reads of the next k-step (A blocks at la +
// 4096 i, W blocks at lb + 4096 j, the row-swizzled layout above) behind the
// first six MFMAs, in the order the next block consumes them, and a wait for
// them at the end, so no LDS load result outlives the statement.  The
// weight fragment is the first operand, so a lane's accumulator registers
// hold 4 consecutive output columns.  Shared by the GEMM kernels and the
// k-step probe.

struct Frags {
  u32x4 a0, a1, a2, a3, b0, b1;
};

#define RM_MF(c, b, a) "v_mfma_f32_32x32x16_bf16 %[" #c "], %[" #b "], %[" #a "], %[" #c "]\n\t"
#define RM_RD(dst, addr, off) "ds_read_b128 %[" #dst "], %[" #addr "] offset:" #off "\n\t"
#define RM_KSTEP                                                                                               \
  RM_MF(c00, b0, a0) RM_RD(na0, la, 0) RM_MF(c01, b1, a0) RM_RD(nb0, lb, 0) RM_MF(c10, b0, a1) RM_RD(nb1, lb, 4096) \
      RM_MF(c11, b1, a1) RM_RD(na1, la, 4096) RM_MF(c20, b0, a2) RM_RD(na2, la, 8192) RM_MF(c21, b1, a2)           \
          RM_RD(na3, la, 12288) RM_MF(c30, b0, a3) RM_MF(c31, b1, a3) "s_waitcnt lgkmcnt(0)\n\t"

#define RM_KSTEP_ACC                                                                                   \
  [c00] "+v"(acc[0][0]), [c01] "+v"(acc[0][1]), [c10] "+v"(acc[1][0]), [c11] "+v"(acc[1][1]),         \
      [c20] "+v"(acc[2][0]), [c21] "+v"(acc[2][1]), [c30] "+v"(acc[3][0]), [c31] "+v"(acc[3][1]),     \
      [na0] "=&v"(nx.a0), [na1] "=&v"(nx.a1), [na2] "=&v"(nx.a2), [na3] "=&v"(nx.a3), [nb0] "=&v"(nx.b0), \
      [nb1] "=&v"(nx.b1)
#define RM_KSTEP_IN \
  [a0] "v"(cu.a0), [a1] "v"(cu.a1), [a2] "v"(cu.a2), [a3] "v"(cu.a3), [b0] "v"(cu.b0), [b1] "v"(cu.b1), \
      [la] "v"(la), [lb] "v"(lb)

__device__ __forceinline__ void kstep(floatx16 (&acc)[4][2], const Frags& cu, Frags& nx, uint32_t la, uint32_t lb) {
  asm volatile(RM_KSTEP : RM_KSTEP_ACC : RM_KSTEP_IN);
}

// the six fragment reads of one k-step on their own (first k-step of a tile)
__device__ __forceinline__ void read_frags(Frags& nx, uint32_t la, uint32_t lb) {
  asm volatile(RM_RD(na0, la, 0) RM_RD(nb0, lb, 0) RM_RD(nb1, lb, 4096) RM_RD(na1, la, 4096) RM_RD(na2, la, 8192)
                   RM_RD(na3, la, 12288) "s_waitcnt lgkmcnt(0)\n\t"
               : [na0] "=&v"(nx.a0), [na1] "=&v"(nx.a1), [na2] "=&v"(nx.a2), [na3] "=&v"(nx.a3), [nb0] "=&v"(nx.b0),
                 [nb1] "=&v"(nx.b1)
               : [la] "v"(la), [lb] "v"(lb));
}

}  // namespace rm

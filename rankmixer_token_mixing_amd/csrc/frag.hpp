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

}  // namespace rm

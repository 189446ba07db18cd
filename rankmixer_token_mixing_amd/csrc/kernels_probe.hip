// Measurement probes: the ceilings the products and the row kernels are
// compared with, measured on the chip rather than taken from its data sheet.
//
//  * k_mfma_loop: nothing but v_mfma_f32_32x32x16_bf16, the instruction of
//    the grouped products, on random bf16 operands held in registers.  Each
//    wave owns eight 32x32 fp32 accumulators (the products' 128 x 64 wave
//    tile) and sixteen different operand fragments, and every MFMA of a
//    64-MFMA round pairs a different A and B fragment, so the multiplier
//    inputs change from one MFMA to the next as they do when fragments stream
//    from LDS.  Two workgroups of four waves per compute unit: two waves per
//    SIMD, as in the products.
//  * k_kstep_loop: the pipelined products' k-step alone (frag.hpp's kstep):
//    per wave and k-step eight MFMAs on a 128 x 64 tile and the six 16-byte
//    fragment reads of the next k-step from the products' swizzled LDS layout
//    (a 32 KB A slice and a 32 KB W slice of random bf16), eight waves per
//    compute unit as in the products, no DMA and no barriers: the rate the
//    main loop could reach with its operands fed from LDS.
//  * k_copy: a streaming copy of 16-byte chunks, four loads in flight per
//    lane; HBM bandwidth as a kernel sees it (with a cold or warm last-level
//    cache, depending on what the caller ran before).
#include "common.hpp"
#include "frag.hpp"
#include "launch.hpp"

namespace rm {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

// two waves per SIMD, as the products run
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_mfma_loop(
    const uint4* __restrict__ frags, float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  // 16 fragments per wave: 8 for the A side, 8 for the W side
  uint4 f[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) f[i] = frags[(wave % 64) * 16 * 64 + i * 64 + lane];
  floatx16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
    // 8 k-steps of 8 MFMAs (4 x 2 blocks); k-step s pairs A fragment
    // (s + i) % 8 with W fragment 8 + (s + 3 j) % 8
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i * 2 + j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, f[8 + (s + 3 * j) % 8]), __builtin_bit_cast(bf16x8, f[(s + i) % 8]),
              acc[i * 2 + j], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[i][e];
  out[wave * 64 + lane] = sum;
}

// eight waves of the products' 2 x 4 wave grid; the slab is the A slice
// (bytes 0..32K) and the W slice (32K..64K) in the products' LDS layout
__global__ __launch_bounds__(512) void k_kstep_loop(const uint4* __restrict__ slab, float* __restrict__ out,
                                                    int iters) {
  __shared__ uint4 lds[kProbeSlabBytes / 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kProbeSlabBytes / 16; i += 512) lds[i] = slab[i];
  __syncthreads();
  const int wm = wave / 4, wn = wave % 4, lr = lane & 31, lh = lane >> 5;
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t ch = (uint32_t)(((kk * 2 + lh) ^ ((lr >> 1) & 7)) * 16);
    oa[kk] = (uint32_t)(wm * 128 + lr) * 128 + ch;
    ob[kk] = (uint32_t)(wn * 64 + lr) * 128 + ch;
  }
  const uint32_t sA = (uint32_t)(uintptr_t)lds, sW = sA + kProbeSlabBytes / 2;
  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  Frags f0, f1;
  read_frags(f0, sA + oa[0], sW + ob[0]);
  for (int it = 0; it < iters; ++it) {
    kstep(acc, f0, f1, sA + oa[1], sW + ob[1]);
    kstep(acc, f1, f0, sA + oa[2], sW + ob[2]);
    kstep(acc, f0, f1, sA + oa[3], sW + ob[3]);
    kstep(acc, f1, f0, sA + oa[0], sW + ob[0]);
  }
  // the last MFMAs' results are read by ordinary code from here on
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t" ::);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[i][j][e];
  out[(long long)blockIdx.x * 512 + tid] = sum;
}

__global__ __launch_bounds__(256) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

int probe_mfma_waves() { return device_cus() * 8; }

hipError_t launch_probe_mfma(const void* frags, float* out, int iters, hipStream_t s) {
  const int blocks = device_cus() * 2;
  hipLaunchKernelGGL(k_mfma_loop, dim3(blocks), dim3(256), 0, s, (const uint4*)frags, out, iters);
  return hipGetLastError();
}

int probe_kstep_blocks() { return device_cus(); }

hipError_t launch_probe_kstep(const void* slab, float* out, int iters, hipStream_t s) {
  hipLaunchKernelGGL(k_kstep_loop, dim3(probe_kstep_blocks()), dim3(512), 0, s, (const uint4*)slab, out, iters);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, long long n16, hipStream_t s) {
  const int blocks = device_cus() * 8;
  hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, s, (const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError();
}

}  // namespace rm

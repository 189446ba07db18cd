// Pointwise kernels of the block variants of "淘宝闪购-爆品团精排 Scaling Up
// 迭代实践": the SwiGLU per-token FFN (section 3.6) combines the gate and up
// halves of its first product, H = SiLU(G) * U.  HBM-bound.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace rm {

namespace {

// rows of [G | U] (2*Hs wide) -> rows of H (Hs wide), 8 elements per thread
template <typename T>
__global__ __launch_bounds__(256) void k_swiglu_ew(const T* __restrict__ gu, T* __restrict__ h, int64_t rows, int Hs) {
  const int per = Hs / 8;
  const int64_t n = rows * per;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per;
    const int j = (int)(i - r * per) * 8;
    float g[8], u[8], o[8];
    load_f32<T, 8>(gu + r * 2 * Hs + j, g);
    load_f32<T, 8>(gu + r * 2 * Hs + Hs + j, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = g[e] / (1.0f + __expf(-g[e])) * u[e];
    store_from_f32<T, 8>(h + r * Hs + j, o);
  }
}

}  // namespace

hipError_t launch_swiglu_ew(const void* gu, void* h, int64_t rows, int Hs, int dt, hipStream_t s) {
  if (Hs % 8) return hipErrorInvalidValue;
  const int64_t n = rows * (Hs / 8);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536)));
  if (dt == kBF16)
    hipLaunchKernelGGL((k_swiglu_ew<bf16>), grid, dim3(256), 0, s, (const bf16*)gu, (bf16*)h, rows, Hs);
  else
    hipLaunchKernelGGL((k_swiglu_ew<float>), grid, dim3(256), 0, s, (const float*)gu, (float*)h, rows, Hs);
  return hipGetLastError();
}

}  // namespace rm

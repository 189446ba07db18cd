// Row kernels of training the ReLU-routed MoE block with the dense-training /
// sparse-inference routers ("Rankmixer: 硬件效率优化", section "Sparse MoE扩展":
// the training forward routes with h_train, the sparsity loss sums the gates
// of h_infer).  The expert products run densely over every (token, expert)
// group on the grouped GEMM -- dense training activates most experts by
// design -- and a gate of zero contributes zero.  HBM-bound pieces here:
//  * k_moe_combine_dense: v = sum_j G_train[j] * y_j, one row per wave;
//  * k_moe_bwd_rows: per row, dG_j = dV . y_j, dy_j = G_j dV, the training
//    router's dz_j = dG_j [G_j > 0], its input gradient sum_j dz_j Wr_j, and the
//    inference router's mask [G_infer > 0];
//  * k_sum_all: the sparsity loss, a fixed-order sum in two passes.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace rm {

namespace {

constexpr int kRowWaves = 4;

// z[b][t][:] = sum_j G[b][t][j] * y[b][t][j][:]  (y [B][T][E][D] and z in T, fp32 sums)
template <typename T>
__global__ __launch_bounds__(kRowWaves* kWave) void k_moe_combine_dense(const T* __restrict__ y,
                                                                          const float* __restrict__ gate,
                                                                          T* __restrict__ z, int64_t rows, int E,
                                                                          int D) {
  const int64_t row = (int64_t)blockIdx.x * kRowWaves + threadIdx.x / kWave;
  if (row >= rows) return;
  const int lane = lane_id();
  const T* yr = y + row * E * (int64_t)D;
  for (int k = lane * 4; k < D; k += kWave * 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < E; ++j) {
      const float g = gate[row * E + j];
      float v[4];
      load_f32<T, 4>(yr + (int64_t)j * D + k, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(g, v[e], acc[e]);
    }
    store_from_f32<T, 4>(z + row * D + k, acc);
  }
}

struct MoeBwdArgs {
  const void* dv;      // dY2, token-major [T][B][D] (dtype)
  const void* y;       // expert outputs [B][T][E][D] (dtype)
  const float* gt;     // G_train [B][T][E]
  const float* gi;     // G_infer [B][T][E]
  const void* wr;      // training router [T][E][D] (dtype)
  void* dy;            // [T][E][B][D] dtype: G_train * dV, (token, expert)-major
  void* dz;            // [B][T][E] dtype: dL/dz_train
  void* mask;          // [B][T][E] dtype: [G_infer > 0]
  float* dsr;          // [T][B][D] fp32: sum_j dz_j Wr[t][j]
  int64_t B;
  int T, E, D;
};

// one wave per row (b, t); 4 elements per lane-chunk, D % 4 == 0 (checked)
template <typename T>
__global__ __launch_bounds__(kRowWaves* kWave) void k_moe_bwd_rows(MoeBwdArgs a) {
  const int64_t row = (int64_t)blockIdx.x * kRowWaves + threadIdx.x / kWave;
  if (row >= a.B * a.T) return;
  const int lane = lane_id();
  const int64_t b = row / a.T;
  const int t = (int)(row - b * a.T);
  const int D = a.D, E = a.E;
  const T* dvr = (const T*)a.dv + ((int64_t)t * a.B + b) * D;
  const T* yr = (const T*)a.y + row * E * (int64_t)D;
  float my_dz = 0.f;  // lane j keeps dz_j (E <= 32, checked)
  for (int j = 0; j < E; ++j) {
    const float g = a.gt[row * E + j];
    float part = 0.f;
    for (int k = lane * 4; k < D; k += kWave * 4) {
      float dv[4], yv[4], o[4];
      load_f32<T, 4>(dvr + k, dv);
      load_f32<T, 4>(yr + (int64_t)j * D + k, yv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fmaf(dv[e], yv[e], part);
        o[e] = g * dv[e];
      }
      store_from_f32<T, 4>((T*)a.dy + (((int64_t)t * E + j) * a.B + b) * D + k, o);
    }
    const float dg = wave_sum(part);
    if (lane == j) my_dz = g > 0.f ? dg : 0.f;
  }
  if (lane < E) {
    ((T*)a.dz)[row * E + lane] = from_f32<T>(my_dz);
    ((T*)a.mask)[row * E + lane] = from_f32<T>(a.gi[row * E + lane] > 0.f ? 1.f : 0.f);
  }
  const T* wr = (const T*)a.wr + (int64_t)t * E * D;
  float* out = a.dsr + ((int64_t)t * a.B + b) * D;
  // the chunk loop runs the same trip count on every lane, so the broadcast
  // of lane j's dz happens with the whole wave active (lanes past D only skip
  // the memory accesses)
  const int nch = (D + kWave * 4 - 1) / (kWave * 4);
  for (int c = 0; c < nch; ++c) {
    const int k = c * kWave * 4 + lane * 4;
    const bool in = k < D;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < E; ++j) {
      const float dzj = __shfl(my_dz, j, kWave);
      if (in) {
        float w[4];
        load_f32<T, 4>(wr + (int64_t)j * D + k, w);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(dzj, w[e], acc[e]);
      }
    }
    if (in) store_from_f32<float, 4>(out + k, acc);
  }
}

// out[blockIdx.x] = sum of x[blockIdx.x * chunk, min(n, (blockIdx.x + 1) * chunk))
// in a fixed order
__global__ __launch_bounds__(256) void k_sum_all(const float* __restrict__ x, float* __restrict__ out, int64_t n,
                                                 int64_t chunk) {
  __shared__ float red[256];
  const int64_t lo = (int64_t)blockIdx.x * chunk, hi = std::min<int64_t>(n, lo + chunk);
  float s = 0.f;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256) s += x[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = red[0];
}

// x[i] *= s
__global__ __launch_bounds__(256) void k_scale(float* __restrict__ x, int64_t n, float s) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    x[i] *= s;
}

dim3 rows_grid(int64_t rows) { return dim3((unsigned)((rows + kRowWaves - 1) / kRowWaves)); }

}  // namespace

hipError_t launch_moe_combine_dense(const void* y, const float* gate, void* z, int64_t rows, int E, int D, int dt,
                                    hipStream_t s) {
  if (D % 4) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  if (dt == kBF16)
    hipLaunchKernelGGL(k_moe_combine_dense<bf16>, rows_grid(rows), dim3(kRowWaves * kWave), 0, s, (const bf16*)y,
                       gate, (bf16*)z, rows, E, D);
  else
    hipLaunchKernelGGL(k_moe_combine_dense<float>, rows_grid(rows), dim3(kRowWaves * kWave), 0, s, (const float*)y,
                       gate, (float*)z, rows, E, D);
  return hipGetLastError();
}

hipError_t launch_moe_bwd_rows(const void* dv, const void* y, const float* gt, const float* gi, const void* wr,
                               void* dy, void* dz, void* mask, float* dsr, int64_t B, int T, int E, int D, int dt,
                               hipStream_t s) {
  if (D % 4 || E < 1 || E > 32) return hipErrorInvalidValue;
  if (B == 0) return hipSuccess;
  MoeBwdArgs a{dv, y, gt, gi, wr, dy, dz, mask, dsr, B, T, E, D};
  if (dt == kBF16)
    hipLaunchKernelGGL(k_moe_bwd_rows<bf16>, rows_grid(B * T), dim3(kRowWaves * kWave), 0, s, a);
  else
    hipLaunchKernelGGL(k_moe_bwd_rows<float>, rows_grid(B * T), dim3(kRowWaves * kWave), 0, s, a);
  return hipGetLastError();
}

int sum_all_parts(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>(kSumParts, (n + 4095) / 4096)); }

hipError_t launch_sum_all(const float* x, float* out, int64_t n, float* part, hipStream_t s) {
  // pass 1: up to kSumParts workgroups over contiguous chunks; pass 2: one
  // workgroup over the partial sums
  const int np = sum_all_parts(n);
  const int64_t chunk = (n + np - 1) / np;
  hipLaunchKernelGGL(k_sum_all, dim3(np), dim3(256), 0, s, x, part, n, std::max<int64_t>(chunk, 1));
  hipLaunchKernelGGL(k_sum_all, dim3(1), dim3(256), 0, s, part, out, (int64_t)np, (int64_t)np);
  return hipGetLastError();
}

hipError_t launch_scale(float* x, int64_t n, float scale, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536)));
  hipLaunchKernelGGL(k_scale, grid, dim3(256), 0, s, x, n, scale);
  return hipGetLastError();
}

}  // namespace rm

// Device helpers shared by the RankMixer HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rm {

constexpr int kWave = 64;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// scalar conversions

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float -> bf16, round to nearest even (gfx950 converts in hardware)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// ---------------------------------------------------------------------------
// vector loads / stores of N consecutive elements, converted to / from float.
// N * sizeof(T) is 2, 4, 8, 16 or 32 bytes; the address is aligned to
// min(16, N * sizeof(T)) bytes.

template <int BYTES> struct RawVec;
template <> struct RawVec<2> { typedef uint16_t type; };
template <> struct RawVec<4> { typedef uint32_t type; };
template <> struct RawVec<8> { typedef uint2 type; };
template <> struct RawVec<16> { typedef uint4 type; };
struct Raw32 { uint4 lo, hi; };
template <> struct RawVec<32> { typedef Raw32 type; };

template <typename T, int N>
struct Vec {
  static constexpr int kBytes = N * (int)sizeof(T);
  typedef typename RawVec<kBytes>::type raw_t;
  union {
    raw_t raw;
    T e[N];
  };
};

template <typename T, int N>
__device__ __forceinline__ void load_f32(const T* p, float (&out)[N]) {
  Vec<T, N> v;
  v.raw = *reinterpret_cast<const typename Vec<T, N>::raw_t*>(p);
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = to_f32(v.e[i]);
}

template <typename T, int N>
__device__ __forceinline__ void store_from_f32(T* p, const float (&in)[N]) {
  Vec<T, N> v;
#pragma unroll
  for (int i = 0; i < N; ++i) v.e[i] = from_f32<T>(in[i]);
  *reinterpret_cast<typename Vec<T, N>::raw_t*>(p) = v.raw;
}

// ---------------------------------------------------------------------------
// wave-level reductions (all 64 lanes get the result)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// ---------------------------------------------------------------------------
// GELU, exact form x * Phi(x) with Phi the standard normal CDF, written as
//   GELU(x) = max(x, 0) - |x| Phi(-|x|)
// (for x >= 0, x Phi(x) = x - x Phi(-x); for x < 0 it is x Phi(-|x|)).  The
// tail is Phi(-a) = exp2(P(min(a, 6.5))), P a degree-6 polynomial fitted to
// log2 Phi(-a) on [0, 6.5] by weighted least squares (gelu_fit.py prints the
// coefficients and the error); the Gaussian's -log2(e) a^2 / 2 is P's square
// term.  In fp32 the result is within 2.5e-7 of the exact GELU for |x| <= 9
// (|x| * 4e-11 beyond, the clamped tail) and within 1.3e-5 relative wherever
// |GELU| > 1e-3, at nine ALU ops and one transcendental (exp2).

__device__ __forceinline__ float phi_tail_log2(float ac) {
  float p = fmaf(3.4358014090685174e-05f, ac, -0.000775179301854223f);
  p = fmaf(p, ac, 0.008079172112047672f);
  p = fmaf(p, ac, -0.05336913466453552f);
  p = fmaf(p, ac, -0.4588397741317749f);
  p = fmaf(p, ac, -1.1511653661727905f);
  return fmaf(p, ac, -0.9999982714653015f);
}

// The clamps take their operand as it is -- v_med3_f32 for min(a, 6.5) and an
// integer max for max(x, 0) (a float's bits ordered as a signed integer put
// every negative value below +0) -- where fminf / fmaxf would first
// canonicalize a value that comes straight out of an MFMA (one more
// instruction per value in a product's epilogue).
__device__ __forceinline__ float gelu_erf(float x) {
  const float a = fabsf(x);
  const float tail = __builtin_amdgcn_exp2f(phi_tail_log2(__builtin_amdgcn_fmed3f(a, 0.0f, 6.5f)));  // Phi(-a)
  return fmaf(-a, tail, __int_as_float(max(__float_as_int(x), 0)));
}

// GELU(x) as gelu_erf and its derivative Phi(x) + x phi(x) from the same tail:
// Phi(x) = 1 - Phi(-a) for x >= 0, Phi(-a) otherwise, and
// phi(x) = exp2(-log2(e) x^2 / 2) / sqrt(2 pi).  In fp32 the derivative is
// within 7e-7 of the exact one.
__device__ __forceinline__ void gelu_and_grad(float x, float& g, float& dg) {
  const float a = fabsf(x);
  const float tail = __builtin_amdgcn_exp2f(phi_tail_log2(fminf(a, 6.5f)));  // Phi(-a)
  g = fmaf(-a, tail, fmaxf(x, 0.0f));
  const float cdf = x >= 0.0f ? 1.0f - tail : tail;
  dg = fmaf(x, 0.3989422804014327f * __builtin_amdgcn_exp2f(x * -0.7213475204444817f * x), cdf);
}

// ---------------------------------------------------------------------------
// Workgroup ids are handed to the 8 XCDs round-robin (id % 8).  Map the ids
// of one XCD to a contiguous range of logical tiles so that tiles sharing
// operand panels run under the same L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int id, int n) {
  constexpr int kXcd = 8;
  const int q = n / kXcd, r = n % kXcd;
  const int x = id % kXcd, local = id / kXcd;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

}  // namespace rm

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
// GELU, exact form x * Phi(x) with Phi the standard normal CDF.  Written as
//   GELU(x) = max(x, 0) - |x| Phi(-|x|)
// (for x >= 0, x Phi(x) = x - x Phi(-x); for x < 0 it is x Phi(-|x|)), with the
// tail Phi(-a) = erfc(a / sqrt 2) / 2 from Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26:
//   erfc(z) = (c1 t + c2 t^2 + c3 t^3 + c4 t^4 + c5 t^5) exp(-z^2),
//   t = 1 / (1 + p z),  z >= 0,  |error| <= 1.5e-7.
// The coefficients below are c_i / 2 and p / sqrt 2; exp(-a^2 / 2) is
// exp2(-a^2 log2(e) / 2).  Eleven ALU ops and two transcendental ones.

__device__ __forceinline__ float gelu_erf(float x) {
  const float a = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(a, 0.23164188826636f, 1.0f));  // p / sqrt 2, p = 0.3275911
  float y = fmaf(0.5307027145f, t, -0.7265760135f);
  y = fmaf(y, t, 0.7107068705f);
  y = fmaf(y, t, -0.142248368f);
  y = fmaf(y, t, 0.127414796f);  // Phi(-a) = t y e
  const float e = __builtin_amdgcn_exp2f((x * x) * -0.7213475204444817f);
  return fmaf(-(a * t) * y, e, fmaxf(x, 0.0f));
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

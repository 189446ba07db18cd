// Row kernels of the RankMixer forward: pad-split tokenizer, token mixing,
// the fused token-mix + residual + LayerNorm that produces S, a LayerNorm
// over fp32 rows, and mean pooling with the logit head.  All are bound by
// HBM bandwidth; each wave owns one [D] row and keeps it in registers.
#include "common.hpp"
#include "launch.hpp"

namespace rm {

namespace {

constexpr int kRowsPerBlock = 4;  // waves (rows) per workgroup
__device__ __forceinline__ float ln_eps() { return 1e-5f; }

// largest chunk (elements) that divides `d`, is at most 16 bytes and keeps the
// address aligned
int chunk_elems(int d, int elem_bytes) {
  const int max_e = 16 / elem_bytes;
  for (int v = max_e; v > 1; v >>= 1)
    if (d % v == 0) return v;
  return 1;
}

// register slots per lane for a row of `chunks` chunks (0: row too wide)
int pick_maxi(int chunks) {
  const int need = (chunks + kWave - 1) / kWave;
  if (need <= 1) return 1;
  if (need <= 2) return 2;
  if (need <= 4) return 4;
  if (need <= 8) return 8;
  if (need <= 16) return 16;
  return 0;
}

// as pick_maxi, but exactly 3 slots where a row needs 3 (rows of 129-192
// chunks, e.g. D = 1536 in 16-byte chunks): the block-boundary pass holds two
// rows per lane and then needs 108 registers instead of 128
int pick_maxi3(int chunks) { return (chunks + kWave - 1) / kWave == 3 ? 3 : pick_maxi(chunks); }

// ---------------------------------------------------------------------------
// pad-split tokenizer: x0[b][i] = i < F ? cast(emb[b][i]) : 0, i < T*D.
// Each thread writes 4 consecutive outputs of one sample.

template <typename T>
__global__ __launch_bounds__(256) void k_tokenize(const float* __restrict__ emb, T* __restrict__ x0,
                                                  int64_t B, int64_t F, int64_t TD) {
  const int64_t per_row = TD / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * per_row) return;
  const int64_t b = idx / per_row;
  const int64_t i = (idx - b * per_row) * 4;
  const float* src = emb + b * F;
  float v[4];
  if (i + 4 <= F && (F & 3) == 0) {
    const float4 q = *reinterpret_cast<const float4*>(src + i);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (i + e < F) ? src[i + e] : 0.0f;
  }
  store_from_f32<T, 4>(x0 + b * TD + i, v);
}

// odd T*D: one element per thread
template <typename T>
__global__ __launch_bounds__(256) void k_tokenize1(const float* __restrict__ emb, T* __restrict__ x0,
                                                   int64_t B, int64_t F, int64_t TD) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * TD) return;
  const int64_t b = idx / TD, i = idx - b * TD;
  x0[idx] = from_f32<T>(i < F ? emb[b * F + i] : 0.0f);
}

// ---------------------------------------------------------------------------
// token mixing, H = T: y[b][h][t*d + j] = x[b][t][h*d + j].  One wave per
// output row (b, h); VEC-element chunks never straddle a head.

template <int EB, int VEC>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void k_token_mix(const void* __restrict__ xv,
                                                                     void* __restrict__ yv,
                                                                     int64_t B, int T, int D) {
  typedef typename RawVec<EB * VEC>::type raw_t;
  typedef typename RawVec<EB>::type elem_t;
  // the T rows of one sample read the same [T][D] block: keep them on one XCD
  const int64_t row = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= B * T) return;
  const int lane = lane_id();
  const int64_t b = row / T;
  const int h = (int)(row - b * T);
  const int d = D / T;
  const elem_t* xb = reinterpret_cast<const elem_t*>(xv) + b * (int64_t)T * D;
  elem_t* yr = reinterpret_cast<elem_t*>(yv) + row * (int64_t)D;
  const int nch = D / VEC;
  for (int c = lane; c < nch; c += kWave) {
    const int k = c * VEC;
    const int t = k / d, j = k - t * d;
    *reinterpret_cast<raw_t*>(yr + k) = *reinterpret_cast<const raw_t*>(xb + (int64_t)t * D + h * d + j);
  }
}

// ---------------------------------------------------------------------------
// S[b,t,:] = LN(TokenMix(X)[b,t,:] + X[b,t,:]) * g + beta.  One wave per row.
// Element k of mixed token t is element t*d + (k mod d) of token k / d.
// Rows move in 16-byte chunks (OV elements); the gather takes each chunk in
// pieces of VEC elements (VEC divides the head width d, so a piece never
// crosses a head).

template <typename T, int VEC, int MAXI>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void k_mix_ln(const T* __restrict__ x, T* __restrict__ s,
                                                                  const float* __restrict__ g,
                                                                  const float* __restrict__ beta,
                                                                  int64_t B, int T_, int D, int token_major) {
  constexpr int OV = 16 / (int)sizeof(T), PV = OV / VEC;
  static_assert(OV % VEC == 0, "pieces of a chunk");
  // the T rows of one sample gather from the same [T][D] block: keep them on
  // one XCD so the second read of each element hits its L2
  const int64_t row = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= B * T_) return;
  const int lane = lane_id();
  const int64_t b = row / T_;
  const int t = (int)(row - b * T_);
  const int d = D / T_;
  const T* xb = x + b * (int64_t)T_ * D;
  const int nch = D / OV;
  float v[MAXI][OV];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
      const int k = c * OV;
      float m[OV], r[OV];
#pragma unroll
      for (int pc = 0; pc < PV; ++pc) {
        const int kp = k + pc * VEC;
        const int tp = kp / d, j = kp - tp * d;
        float piece[VEC];
        load_f32<T, VEC>(xb + (int64_t)tp * D + t * d + j, piece);
#pragma unroll
        for (int e = 0; e < VEC; ++e) m[pc * VEC + e] = piece[e];
      }
      load_f32<T, OV>(xb + (int64_t)t * D + k, r);
#pragma unroll
      for (int e = 0; e < OV; ++e) {
        v[i][e] = m[e] + r[e];
        sum += v[i][e];
      }
    }
  }
  const float mean = wave_sum(sum) / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < OV; ++e) {
        const float q = v[i][e] - mean;
        sq += q * q;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + ln_eps());
  // S row (b, t) at [b][t] or, token-major, at [t][b]
  T* sr = s + (token_major ? ((int64_t)t * B + b) : row) * (int64_t)D;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
      const int k = c * OV;
      float o[OV];
#pragma unroll
      for (int e = 0; e < OV; ++e) o[e] = (v[i][e] - mean) * rstd * g[k + e] + beta[k + e];
      store_from_f32<T, OV>(sr + k, o);
    }
  }
}

// ---------------------------------------------------------------------------
// The same S computed straight from the pad-split tokenizer's input: element
// (t, k) of sample b's X0 is emb[b][t*D + k] cast to T (0 past F), read where
// it lies, so X0 is never written.  F % 4 == 0 keeps every sample's row
// 16-byte aligned; a piece that straddles F is read element by element.

template <typename T, int N>
__device__ __forceinline__ void load_emb(const float* __restrict__ er, int idx, int F, float (&out)[N]) {
  if (idx + N <= F) {
    float f[N];
    load_f32<float, N>(er + idx, f);
#pragma unroll
    for (int e = 0; e < N; ++e) out[e] = to_f32(from_f32<T>(f[e]));
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) out[e] = idx + e < F ? to_f32(from_f32<T>(er[idx + e])) : 0.f;
  }
}

template <typename T, int VEC, int MAXI>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void k_mix_ln_emb(const float* __restrict__ emb, int F,
                                                                      T* __restrict__ s, const float* __restrict__ g,
                                                                      const float* __restrict__ beta, int64_t B,
                                                                      int T_, int D) {
  constexpr int OV = 16 / (int)sizeof(T), PV = OV / VEC;
  static_assert(OV % VEC == 0, "pieces of a chunk");
  const int64_t row = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= B * T_) return;
  const int lane = lane_id();
  const int64_t b = row / T_;
  const int t = (int)(row - b * T_);
  const int d = D / T_;
  const float* er = emb + b * (int64_t)F;
  const int nch = D / OV;
  float v[MAXI][OV];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
      const int k = c * OV;
      float m[OV], r[OV];
#pragma unroll
      for (int pc = 0; pc < PV; ++pc) {
        const int kp = k + pc * VEC;
        const int tp = kp / d, j = kp - tp * d;
        float piece[VEC];
        load_emb<T, VEC>(er, tp * D + t * d + j, F, piece);
#pragma unroll
        for (int e = 0; e < VEC; ++e) m[pc * VEC + e] = piece[e];
      }
      load_emb<T, OV>(er, t * D + k, F, r);
#pragma unroll
      for (int e = 0; e < OV; ++e) {
        v[i][e] = m[e] + r[e];
        sum += v[i][e];
      }
    }
  }
  const float mean = wave_sum(sum) / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < OV; ++e) {
        const float q = v[i][e] - mean;
        sq += q * q;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + ln_eps());
  // token-major S row (b, t) at [t][b]
  T* sr = s + ((int64_t)t * B + b) * (int64_t)D;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
      const int k = c * OV;
      float o[OV];
#pragma unroll
      for (int e = 0; e < OV; ++e) o[e] = (v[i][e] - mean) * rstd * g[k + e] + beta[k + e];
      store_from_f32<T, OV>(sr + k, o);
    }
  }
}

// ---------------------------------------------------------------------------
// out[r,:] = LN(z[r,:] + res[r,:]) * g + beta over rows of D (D % 8 == 0), 8
// elements per lane-chunk, fp32 arithmetic.  Row r = b * Tn + t; the residual
// (optional) of row r starts at res + b * res_bs + t * res_ts, so a
// token-major residual is read in place.

template <typename T, int MAXI>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void k_ln_rows(const T* __restrict__ z,
                                                                   const T* __restrict__ res, int64_t res_bs,
                                                                   int64_t res_ts, int Tn, T* __restrict__ out,
                                                                   const float* __restrict__ g,
                                                                   const float* __restrict__ beta,
                                                                   int64_t rows, int D) {
  constexpr int VEC = 8;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= rows) return;
  const int lane = lane_id();
  const int nch = D / VEC;
  const T* zr = z + row * (int64_t)D;
  const T* rr = res ? res + (row / Tn) * res_bs + (row % Tn) * res_ts : nullptr;
  float v[MAXI][VEC];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
      load_f32<T, VEC>(zr + c * VEC, v[i]);
      if (rr) {
        float r[VEC];
        load_f32<T, VEC>(rr + c * VEC, r);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[i][e] += r[e];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) sum += v[i][e];
    }
  }
  const float mean = wave_sum(sum) / (float)D;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float q = v[i][e] - mean;
        sq += q * q;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + ln_eps());
  T* orow = out + row * (int64_t)D;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
      const int k = c * VEC;
      float o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = (v[i][e] - mean) * rstd * g[k + e] + beta[k + e];
      store_from_f32<T, VEC>(orow + k, o);
    }
  }
}

// ---------------------------------------------------------------------------
// Block boundary: the LN2 of one block and the mix + LN1 of the next, per
// sample in one workgroup.  Phase 1: X'[t] = LN2(Z[b][t] + S[t][b]) for every
// token t of sample b, rounded to the activation type as the block output is,
// into LDS (row pitch D plus one head, so the gathers of phase 2 walk the
// banks).  Phase 2: S'[h][b] = LN1(TM(X')[h] + X'[h]) from LDS, written over
// S (token-major; only this workgroup touches sample b's rows, and every
// read of them happens before the barrier).  X' never goes to HBM.
constexpr int kBndThreads = 1024;
constexpr int kBndLdsMax = 128 * 1024;

template <typename T, int VEC, int MAXI, int R>
__global__ __launch_bounds__(R == 2 ? kBndThreads : kBndThreads / 2) void k_ln_mix_ln(const T* __restrict__ z, T* s,
                                                           const float* __restrict__ g2,
                                                           const float* __restrict__ be2,
                                                           const float* __restrict__ g1,
                                                           const float* __restrict__ be1, int64_t B, int T_,
                                                           int D, int pitch) {
  constexpr int OV = 16 / (int)sizeof(T), PV = OV / VEC;  // 16-byte chunks, gathered in pieces of VEC
  static_assert(OV % VEC == 0, "pieces of a chunk");
  extern __shared__ uint4 bnd_lds[];
  T* xl = reinterpret_cast<T*>(bnd_lds);
  const int NW = blockDim.x / kWave;  // T/R waves (at most 16): R rows each
  const int64_t b = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int d = D / T_, nch = D / OV;
  // phase 1, R rows per wave at a time (rows t0, t0 + NW, ...): every load of
  // those rows is issued before any is used (a row index past T re-reads row
  // t0 and is skipped; chunk indices past the row re-read its last chunk and
  // are left out of the sums and stores)
  for (int t0 = wave; t0 < T_; t0 += R * NW) {
    int tr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) tr[r] = t0 + r * NW < T_ ? t0 + r * NW : t0;
    float v[R][MAXI][OV], q[R][MAXI][OV];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const T* zr = z + (b * T_ + tr[r]) * (int64_t)D;
      const T* sr = s + ((int64_t)tr[r] * B + b) * D;
#pragma unroll
      for (int i = 0; i < MAXI; ++i) {
        const int c = min(lane + i * kWave, nch - 1);
        load_f32<T, OV>(zr + c * OV, v[r][i]);
        load_f32<T, OV>(sr + c * OV, q[r][i]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r > 0 && t0 + r * NW >= T_) break;
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < MAXI; ++i) {
        const bool in = lane + i * kWave < nch;
#pragma unroll
        for (int e = 0; e < OV; ++e) {
          v[r][i][e] += q[r][i][e];
          sum += in ? v[r][i][e] : 0.f;
        }
      }
      const float mean = wave_sum(sum) / (float)D;
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < MAXI; ++i) {
        const bool in = lane + i * kWave < nch;
#pragma unroll
        for (int e = 0; e < OV; ++e) {
          const float dv = v[r][i][e] - mean;
          sq += in ? dv * dv : 0.f;
        }
      }
      const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + ln_eps());
#pragma unroll
      for (int i = 0; i < MAXI; ++i) {
        const int c = lane + i * kWave;
        if (c < nch) {
          const int k = c * OV;
          float o[OV];
#pragma unroll
          for (int e = 0; e < OV; ++e) o[e] = (v[r][i][e] - mean) * rstd * g2[k + e] + be2[k + e];
          store_from_f32<T, OV>(xl + tr[r] * pitch + k, o);
        }
      }
    }
  }
  __syncthreads();
  for (int h = wave; h < T_; h += NW) {
    float v[MAXI][OV];
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      if (c < nch) {
        const int k = c * OV;
        float m[OV], r[OV];
#pragma unroll
        for (int pc = 0; pc < PV; ++pc) {
          const int kp = k + pc * VEC;
          const int tp = kp / d, j = kp - tp * d;
          float piece[VEC];
          load_f32<T, VEC>(xl + tp * pitch + h * d + j, piece);
#pragma unroll
          for (int e = 0; e < VEC; ++e) m[pc * VEC + e] = piece[e];
        }
        load_f32<T, OV>(xl + h * pitch + k, r);
#pragma unroll
        for (int e = 0; e < OV; ++e) {
          v[i][e] = m[e] + r[e];
          sum += v[i][e];
        }
      }
    }
    const float mean = wave_sum(sum) / (float)D;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      if (c < nch) {
#pragma unroll
        for (int e = 0; e < OV; ++e) {
          const float q = v[i][e] - mean;
          sq += q * q;
        }
      }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + ln_eps());
    T* orow = s + ((int64_t)h * B + b) * D;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      if (c < nch) {
        const int k = c * OV;
        float o[OV];
#pragma unroll
        for (int e = 0; e < OV; ++e) o[e] = (v[i][e] - mean) * rstd * g1[k + e] + be1[k + e];
        store_from_f32<T, OV>(orow + k, o);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// pooled[b,k] = (1/T) sum_t x[b,t,k];  logit[b] = sum_k w[k] pooled[b,k] + c

template <typename T, int VEC>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void k_pool_logit(const T* __restrict__ x,
                                                                      const float* __restrict__ w, float c0,
                                                                      float* __restrict__ pooled,
                                                                      float* __restrict__ logits,
                                                                      int64_t B, int T_, int D) {
  const int64_t b = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  if (b >= B) return;
  const int lane = lane_id();
  const T* xb = x + b * (int64_t)T_ * D;
  const float inv_t = 1.0f / (float)T_;
  float dot = 0.f;
  for (int c = lane; c < D / VEC; c += kWave) {
    const int k = c * VEC;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
    for (int t = 0; t < T_; ++t) {
      float q[VEC];
      load_f32<T, VEC>(xb + (int64_t)t * D + k, q);
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[e] += q[e];
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      acc[e] *= inv_t;
      if (w) dot += acc[e] * w[k + e];
    }
    if (pooled) store_from_f32<float, VEC>(pooled + b * D + k, acc);
  }
  dot = wave_sum(dot);
  if (logits && lane == 0) logits[b] = dot + c0;
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers

hipError_t launch_tokenize_padsplit(const float* emb, int64_t B, int64_t F, int T, int D, int dt,
                                    void* x0, hipStream_t s) {
  const int64_t TD = (int64_t)T * D;
  if (TD % 4 == 0) {
    const int64_t n = B * (TD / 4);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dt == kBF16)
      hipLaunchKernelGGL(k_tokenize<bf16>, grid, dim3(256), 0, s, emb, (bf16*)x0, B, F, TD);
    else
      hipLaunchKernelGGL(k_tokenize<float>, grid, dim3(256), 0, s, emb, (float*)x0, B, F, TD);
  } else {
    const int64_t n = B * TD;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (dt == kBF16)
      hipLaunchKernelGGL(k_tokenize1<bf16>, grid, dim3(256), 0, s, emb, (bf16*)x0, B, F, TD);
    else
      hipLaunchKernelGGL(k_tokenize1<float>, grid, dim3(256), 0, s, emb, (float*)x0, B, F, TD);
  }
  return hipGetLastError();
}

namespace {
template <int EB>
hipError_t token_mix_eb(const void* x, void* y, int64_t B, int T, int D, int vec, hipStream_t s) {
  const dim3 grid((unsigned)((B * T + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * kWave);
  switch (vec) {
    case 1: hipLaunchKernelGGL((k_token_mix<EB, 1>), grid, block, 0, s, x, y, B, T, D); break;
    case 2: hipLaunchKernelGGL((k_token_mix<EB, 2>), grid, block, 0, s, x, y, B, T, D); break;
    case 4: hipLaunchKernelGGL((k_token_mix<EB, 4>), grid, block, 0, s, x, y, B, T, D); break;
    default:
      if constexpr (EB == 2) hipLaunchKernelGGL((k_token_mix<EB, 8>), grid, block, 0, s, x, y, B, T, D);
      break;
  }
  return hipGetLastError();
}

template <typename T, int VEC>
hipError_t mix_ln_vec(const void* x, void* so, const float* g, const float* b, int64_t B, int T_, int D, int tm,
                      hipStream_t s) {
  const dim3 grid((unsigned)((B * T_ + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * kWave);
  const T* xx = (const T*)x;
  T* ss = (T*)so;
  switch (pick_maxi(D / (16 / (int)sizeof(T)))) {
    case 0: return hipErrorInvalidValue;
    case 1: hipLaunchKernelGGL((k_mix_ln<T, VEC, 1>), grid, block, 0, s, xx, ss, g, b, B, T_, D, tm); break;
    case 2: hipLaunchKernelGGL((k_mix_ln<T, VEC, 2>), grid, block, 0, s, xx, ss, g, b, B, T_, D, tm); break;
    case 4: hipLaunchKernelGGL((k_mix_ln<T, VEC, 4>), grid, block, 0, s, xx, ss, g, b, B, T_, D, tm); break;
    case 8: hipLaunchKernelGGL((k_mix_ln<T, VEC, 8>), grid, block, 0, s, xx, ss, g, b, B, T_, D, tm); break;
    default: hipLaunchKernelGGL((k_mix_ln<T, VEC, 16>), grid, block, 0, s, xx, ss, g, b, B, T_, D, tm); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t ln_rows_t(const void* zv, const void* res, int64_t rbs, int64_t rts, int Tn, void* out, const float* g,
                     const float* b, int64_t rows, int D, hipStream_t s) {
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * kWave);
  const T* z = (const T*)zv;
  T* o = (T*)out;
  const T* r = (const T*)res;
  if (Tn <= 0) Tn = 1;
  switch (pick_maxi(D / 8)) {
    case 0: return hipErrorInvalidValue;
    case 1: hipLaunchKernelGGL((k_ln_rows<T, 1>), grid, block, 0, s, z, r, rbs, rts, Tn, o, g, b, rows, D); break;
    case 2: hipLaunchKernelGGL((k_ln_rows<T, 2>), grid, block, 0, s, z, r, rbs, rts, Tn, o, g, b, rows, D); break;
    case 4: hipLaunchKernelGGL((k_ln_rows<T, 4>), grid, block, 0, s, z, r, rbs, rts, Tn, o, g, b, rows, D); break;
    case 8: hipLaunchKernelGGL((k_ln_rows<T, 8>), grid, block, 0, s, z, r, rbs, rts, Tn, o, g, b, rows, D); break;
    default: hipLaunchKernelGGL((k_ln_rows<T, 16>), grid, block, 0, s, z, r, rbs, rts, Tn, o, g, b, rows, D); break;
  }
  return hipGetLastError();
}
}  // namespace

bool row_width_supported(int T, int D, int dt) {
  const int eb = dt == kBF16 ? 2 : 4;
  if (T <= 0 || D <= 0 || D % T || D % 8) return false;
  return pick_maxi(D / chunk_elems(D / T, eb)) != 0 && pick_maxi(D / 8) != 0;
}

hipError_t launch_token_mix(const void* x, void* y, int64_t B, int T, int D, int dt, hipStream_t s) {
  const int eb = dt == kBF16 ? 2 : 4;
  const int vec = chunk_elems(D / T, eb);
  return eb == 2 ? token_mix_eb<2>(x, y, B, T, D, vec, s) : token_mix_eb<4>(x, y, B, T, D, vec, s);
}

hipError_t launch_mix_ln(const void* x, void* so, const float* g, const float* b, int64_t B, int T,
                         int D, int dt, bool token_major, hipStream_t s) {
  const int tm = token_major ? 1 : 0;
  const int d = D / T;
  if (dt == kBF16) {
    switch (chunk_elems(d, 2)) {
      case 8: return mix_ln_vec<bf16, 8>(x, so, g, b, B, T, D, tm, s);
      case 4: return mix_ln_vec<bf16, 4>(x, so, g, b, B, T, D, tm, s);
      case 2: return mix_ln_vec<bf16, 2>(x, so, g, b, B, T, D, tm, s);
      default: return mix_ln_vec<bf16, 1>(x, so, g, b, B, T, D, tm, s);
    }
  }
  switch (chunk_elems(d, 4)) {
    case 4: return mix_ln_vec<float, 4>(x, so, g, b, B, T, D, tm, s);
    case 2: return mix_ln_vec<float, 2>(x, so, g, b, B, T, D, tm, s);
    default: return mix_ln_vec<float, 1>(x, so, g, b, B, T, D, tm, s);
  }
}

template <typename T, int VEC>
hipError_t mix_ln_emb_vec(const float* emb, int F, void* so, const float* g, const float* b, int64_t B, int T_,
                          int D, hipStream_t s) {
  const dim3 grid((unsigned)((B * T_ + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * kWave);
  T* ss = (T*)so;
  switch (pick_maxi(D / (16 / (int)sizeof(T)))) {
    case 0: return hipErrorInvalidValue;
    case 1: hipLaunchKernelGGL((k_mix_ln_emb<T, VEC, 1>), grid, block, 0, s, emb, F, ss, g, b, B, T_, D); break;
    case 2: hipLaunchKernelGGL((k_mix_ln_emb<T, VEC, 2>), grid, block, 0, s, emb, F, ss, g, b, B, T_, D); break;
    case 4: hipLaunchKernelGGL((k_mix_ln_emb<T, VEC, 4>), grid, block, 0, s, emb, F, ss, g, b, B, T_, D); break;
    case 8: hipLaunchKernelGGL((k_mix_ln_emb<T, VEC, 8>), grid, block, 0, s, emb, F, ss, g, b, B, T_, D); break;
    default: hipLaunchKernelGGL((k_mix_ln_emb<T, VEC, 16>), grid, block, 0, s, emb, F, ss, g, b, B, T_, D); break;
  }
  return hipGetLastError();
}

bool mix_ln_emb_supported(int T, int D, int64_t F, int dt) {
  return F > 0 && F % 4 == 0 && F <= (int64_t)T * D && row_width_supported(T, D, dt);
}

hipError_t launch_mix_ln_emb(const float* emb, int64_t F, void* so, const float* g, const float* b, int64_t B, int T,
                             int D, int dt, hipStream_t s) {
  if (!mix_ln_emb_supported(T, D, F, dt)) return hipErrorInvalidValue;
  const int d = D / T;
  if (dt == kBF16) {
    switch (chunk_elems(d, 2)) {
      case 8: return mix_ln_emb_vec<bf16, 8>(emb, (int)F, so, g, b, B, T, D, s);
      case 4: return mix_ln_emb_vec<bf16, 4>(emb, (int)F, so, g, b, B, T, D, s);
      case 2: return mix_ln_emb_vec<bf16, 2>(emb, (int)F, so, g, b, B, T, D, s);
      default: return mix_ln_emb_vec<bf16, 1>(emb, (int)F, so, g, b, B, T, D, s);
    }
  }
  switch (chunk_elems(d, 4)) {
    case 4: return mix_ln_emb_vec<float, 4>(emb, (int)F, so, g, b, B, T, D, s);
    case 2: return mix_ln_emb_vec<float, 2>(emb, (int)F, so, g, b, B, T, D, s);
    default: return mix_ln_emb_vec<float, 1>(emb, (int)F, so, g, b, B, T, D, s);
  }
}

namespace {
// LDS row pitch of the boundary kernel in elements: D plus one head rounded
// up to 16 bytes
int bnd_pitch(int T, int D, int eb) { return D + ((D / T * eb + 15) / 16 * 16) / eb; }

template <typename T, int VEC, int R>
hipError_t ln_mix_ln_rows(const void* z, void* s, const float* g2, const float* b2, const float* g1,
                          const float* b1, int64_t B, int T_, int D, hipStream_t st) {
  const int pitch = bnd_pitch(T_, D, (int)sizeof(T));
  const size_t lds = (size_t)T_ * pitch * sizeof(T);
  const int nw = std::min(kBndThreads / kWave, std::max(1, (T_ + R - 1) / R));
  const dim3 grid((unsigned)B), block(nw * kWave);
  const T* zz = (const T*)z;
  T* ss = (T*)s;
  const int maxi = pick_maxi3(D / (16 / (int)sizeof(T)));
  if constexpr (R == 4) {  // rows of two chunks per lane only
    if (maxi != 2) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_ln_mix_ln<T, VEC, 2, R>), grid, block, lds, st, zz, ss, g2, b2, g1, b1, B, T_, D, pitch);
    return hipGetLastError();
  }
  switch (maxi) {
    case 0: return hipErrorInvalidValue;
    case 3: hipLaunchKernelGGL((k_ln_mix_ln<T, VEC, 3, R>), grid, block, lds, st, zz, ss, g2, b2, g1, b1, B, T_, D, pitch); break;
    case 1: hipLaunchKernelGGL((k_ln_mix_ln<T, VEC, 1, R>), grid, block, lds, st, zz, ss, g2, b2, g1, b1, B, T_, D, pitch); break;
    case 2: hipLaunchKernelGGL((k_ln_mix_ln<T, VEC, 2, R>), grid, block, lds, st, zz, ss, g2, b2, g1, b1, B, T_, D, pitch); break;
    case 4: hipLaunchKernelGGL((k_ln_mix_ln<T, VEC, 4, R>), grid, block, lds, st, zz, ss, g2, b2, g1, b1, B, T_, D, pitch); break;
    default: return hipErrorInvalidValue;  // wider rows: see ln_mix_ln_supported
  }
  return hipGetLastError();
}

template <typename T, int VEC>
hipError_t ln_mix_ln_vec(const void* z, void* s, const float* g2, const float* b2, const float* g1,
                         const float* b1, int64_t B, int T_, int D, hipStream_t st) {
  // rows of two chunks per lane (D of 1024 bf16 or 512 fp32 at most): four rows per wave,
  // so twice the samples fit on a compute unit (rows of D = 768 with T = 16:
  // 53.2-53.8 against 56.5-56.7 us per pass); one-chunk rows (D = 320, T = 16)
  // measured slower that way (49-50 against 45 us) and keep two
  const int maxi = pick_maxi3(D / (16 / (int)sizeof(T)));
  if (maxi == 2 && T_ <= 32) return ln_mix_ln_rows<T, VEC, 4>(z, s, g2, b2, g1, b1, B, T_, D, st);
  return ln_mix_ln_rows<T, VEC, 2>(z, s, g2, b2, g1, b1, B, T_, D, st);
}
}  // namespace

bool ln_mix_ln_supported(int T, int D, int dt) {
  // the sample's rows fit in LDS, and a row is at most 4 chunks per lane (the
  // 16 waves of a workgroup hold two rows each in 128 registers)
  const int eb = dt == kBF16 ? 2 : 4;
  return row_width_supported(T, D, dt) && (size_t)T * bnd_pitch(T, D, eb) * eb <= (size_t)kBndLdsMax &&
         pick_maxi(D / chunk_elems(D / T, eb)) <= 4;
}

hipError_t launch_ln_mix_ln(const void* z, void* s, const float* g2, const float* b2, const float* g1,
                            const float* b1, int64_t B, int T, int D, int dt, hipStream_t st) {
  if (!ln_mix_ln_supported(T, D, dt)) return hipErrorInvalidValue;
  if (B == 0) return hipSuccess;
  const int d = D / T;
  if (dt == kBF16) {
    switch (chunk_elems(d, 2)) {
      case 8: return ln_mix_ln_vec<bf16, 8>(z, s, g2, b2, g1, b1, B, T, D, st);
      case 4: return ln_mix_ln_vec<bf16, 4>(z, s, g2, b2, g1, b1, B, T, D, st);
      case 2: return ln_mix_ln_vec<bf16, 2>(z, s, g2, b2, g1, b1, B, T, D, st);
      default: return ln_mix_ln_vec<bf16, 1>(z, s, g2, b2, g1, b1, B, T, D, st);
    }
  }
  switch (chunk_elems(d, 4)) {
    case 4: return ln_mix_ln_vec<float, 4>(z, s, g2, b2, g1, b1, B, T, D, st);
    case 2: return ln_mix_ln_vec<float, 2>(z, s, g2, b2, g1, b1, B, T, D, st);
    default: return ln_mix_ln_vec<float, 1>(z, s, g2, b2, g1, b1, B, T, D, st);
  }
}

hipError_t launch_ln_rows(const void* z, const void* res, int64_t res_bs, int64_t res_ts, int Tn, void* out,
                          const float* g, const float* b, int64_t rows, int D, int dt, hipStream_t s) {
  return dt == kBF16 ? ln_rows_t<bf16>(z, res, res_bs, res_ts, Tn, out, g, b, rows, D, s)
                     : ln_rows_t<float>(z, res, res_bs, res_ts, Tn, out, g, b, rows, D, s);
}

hipError_t launch_pool_logit(const void* x, const float* w, float c, float* pooled, float* logits,
                             int64_t B, int T, int D, int dt, hipStream_t s) {
  const dim3 grid((unsigned)((B + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * kWave);
  if (dt == kBF16) {
    if (D % 8 == 0)
      hipLaunchKernelGGL((k_pool_logit<bf16, 8>), grid, block, 0, s, (const bf16*)x, w, c, pooled, logits, B, T, D);
    else
      hipLaunchKernelGGL((k_pool_logit<bf16, 4>), grid, block, 0, s, (const bf16*)x, w, c, pooled, logits, B, T, D);
  } else {
    hipLaunchKernelGGL((k_pool_logit<float, 4>), grid, block, 0, s, (const float*)x, w, c, pooled, logits, B, T, D);
  }
  return hipGetLastError();
}

}  // namespace rm

// Kernels of the dense block backward (the chain rule through the block of
// "Rankmixer: 硬件效率优化", section "RankMixer整体架构"; the pages print no
// backward).  The four gradient products run on the grouped GEMM; these are
// the HBM-bound pieces around them:
//  * k_ln_bwd: LayerNorm backward, one row per wave, fp32 math, with the
//    gamma / beta gradients accumulated per workgroup in a fixed order;
//  * k_transpose: [G][R][C] -> [G][C][ldo] through a 64 x 64 LDS tile, with an
//    elementwise op on the way (GELU, or the GELU derivative times an upstream
//    gradient), an optional untransposed copy of the result and optional
//    per-tile column sums (the bias gradients);
//  * k_tm_add: dX = dY1 + TM(dY1), the token mix being its own transpose;
//  * k_sum_parts: fixed-order sums of the per-workgroup / per-tile partials;
//  * k_gelu_ew: H = GELU(U) for the training forward, which keeps U.
// No floating-point atomics: every sum has one fixed order, so results are
// bitwise reproducible.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace rm {

namespace {

constexpr int kLnWaves = 4;       // rows (waves) per workgroup of k_ln_bwd
constexpr int kLnBwdDmax = 4096;  // widest row: the waves' gamma/beta partials live in LDS (128 KB)
__device__ __forceinline__ float ln_eps_b() { return 1e-5f; }

struct LnBwdArgs {
  const void* dout;    // mode 0: dL/dX' rows [B][T][D]
  const void* dres;    // mode 1: dY2, token-major [T][B][D]
  const float* dres32; // mode 1: the W1-branch gradient of S, token-major fp32
  const float* dres32b; // mode 1, optional: a further fp32 addend, token-major
  const void* z;       // mode 0: Z (W2 product + b2) [B][T][D];  mode 1: X [B][T][D]
  const void* res;     // mode 0: S, token-major
  const float* gamma;
  void* dy;            // mode 0: dY2 token-major (dtype);  mode 1: dY1 [B][T][D] fp32
  float* part;         // [gridDim.x][2][D]: sum of dout * xhat, sum of dout
  int64_t B;
  int T, D;
};

// LayerNorm backward.  Mode 0 (LN2): Y = Z + S, upstream dX'.  Mode 1 (LN1):
// Y = TM(X) + X gathered as the forward does, upstream dY2 + dS_ffn.  With
// xhat = (Y - mean) * rstd and g = upstream * gamma:
//   dY = (g - mean(g) - xhat * mean(g * xhat)) * rstd.
// Element k of mixed token t is element t*d + (k mod d) of token k / d.
// The gamma / beta partials of each wave accumulate in its own LDS region
// [2][D] (dynamic LDS, kLnWaves * 2 * D floats), so registers hold only the
// row being processed.  Inside a region, element c * VEC + e (chunk c, lane
// c mod 64) sits at e * nch + c, so the 64 lanes of one update touch 64
// consecutive floats (with the row's element order, lane L's eight floats
// would share a bank with lanes L + 4, L + 8, ...).
template <typename T, int VEC, int MAXI, int MODE>
__global__ __launch_bounds__(kLnWaves* kWave) void k_ln_bwd(LnBwdArgs a) {
  extern __shared__ float wpart[];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int D = a.D, T_ = a.T, d = D / T_;
  const int nch = D / VEC;
  const int64_t rows = a.B * T_;
  for (int k = threadIdx.x; k < kLnWaves * 2 * D; k += kLnWaves * kWave) wpart[k] = 0.f;
  __syncthreads();
  float* pg = wpart + wave * 2 * D;
  float* pb = pg + D;

  // LN2 rows of at most three chunks per lane: the next row's chunks are
  // loaded while this one is reduced (3 * MAXI raw registers; the gamma /
  // beta partials already hold occupancy at three workgroups per CU)
  constexpr bool PF = MODE == 0 && MAXI <= 3;
  typedef typename RawVec<(int)sizeof(T) * VEC>::type raw_t;
  raw_t nz[PF ? MAXI : 1], nr[PF ? MAXI : 1], nd[PF ? MAXI : 1];
  const int64_t stride = (int64_t)gridDim.x * kLnWaves;
  auto fetch = [&](int64_t rw) {
    if constexpr (PF) {
      const int64_t bb = rw / T_;
      const int64_t tmm = (rw - bb * T_) * a.B + bb;
#pragma unroll
      for (int i = 0; i < MAXI; ++i) {
        const int k = min(lane + i * kWave, nch - 1) * VEC;  // past the row: its last chunk, unused
        nz[i] = *reinterpret_cast<const raw_t*>((const T*)a.z + rw * D + k);
        nr[i] = *reinterpret_cast<const raw_t*>((const T*)a.res + tmm * D + k);
        nd[i] = *reinterpret_cast<const raw_t*>((const T*)a.dout + rw * D + k);
      }
    }
  };
  if (PF && (int64_t)blockIdx.x * kLnWaves + wave < rows) fetch((int64_t)blockIdx.x * kLnWaves + wave);

  for (int64_t row = (int64_t)blockIdx.x * kLnWaves + wave; row < rows; row += stride) {
    const int64_t b = row / T_;
    const int t = (int)(row - b * T_);
    const int64_t tm = (int64_t)t * a.B + b;  // token-major row index
    float y[MAXI][VEC], up[MAXI][VEC];
    float sum = 0.f;
    if constexpr (PF) {
#pragma unroll
      for (int i = 0; i < MAXI; ++i) {
        Vec<T, VEC> vz, vr, vd;
        vz.raw = nz[i];
        vr.raw = nr[i];
        vd.raw = nd[i];
        const bool in = lane + i * kWave < nch;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          y[i][e] = to_f32(vz.e[e]) + to_f32(vr.e[e]);
          up[i][e] = to_f32(vd.e[e]);
          sum += in ? y[i][e] : 0.f;
        }
      }
      if (row + stride < rows) fetch(row + stride);
    }
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      if (!PF && c < nch) {
        const int k = c * VEC;
        float p[VEC], q[VEC];
        if constexpr (MODE == 0) {
          load_f32<T, VEC>((const T*)a.z + row * D + k, p);
          load_f32<T, VEC>((const T*)a.res + tm * D + k, q);
          load_f32<T, VEC>((const T*)a.dout + row * D + k, up[i]);
        } else {
          const T* xb = (const T*)a.z + b * (int64_t)T_ * D;
          const int tp = k / d, j = k - tp * d;
          load_f32<T, VEC>(xb + (int64_t)tp * D + t * d + j, p);
          load_f32<T, VEC>(xb + (int64_t)t * D + k, q);
          float r[VEC];
          load_f32<T, VEC>((const T*)a.dres + tm * D + k, up[i]);
          load_f32<float, VEC>(a.dres32 + tm * D + k, r);
#pragma unroll
          for (int e = 0; e < VEC; ++e) up[i][e] += r[e];
          if (a.dres32b) {
            load_f32<float, VEC>(a.dres32b + tm * D + k, r);
#pragma unroll
            for (int e = 0; e < VEC; ++e) up[i][e] += r[e];
          }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          y[i][e] = p[e] + q[e];
          sum += y[i][e];
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
        for (int e = 0; e < VEC; ++e) {
          const float q = y[i][e] - mean;
          sq += q * q;
        }
      }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + ln_eps_b());
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      if (c < nch) {
        const int k = c * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          y[i][e] = (y[i][e] - mean) * rstd;  // xhat from here on
          const float g = up[i][e] * a.gamma[k + e];
          sg += g;
          sgx += g * y[i][e];
          pg[e * nch + c] += up[i][e] * y[i][e];
          pb[e * nch + c] += up[i][e];
        }
      }
    }
    const float mg = wave_sum(sg) / (float)D, mgx = wave_sum(sgx) / (float)D;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      if (c < nch) {
        const int k = c * VEC;
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = (up[i][e] * a.gamma[k + e] - mg - y[i][e] * mgx) * rstd;
        if constexpr (MODE == 0)
          store_from_f32<T, VEC>((T*)a.dy + tm * D + k, o);
        else
          store_from_f32<float, VEC>((float*)a.dy + row * D + k, o);
      }
    }
  }
  // workgroup partials: the waves' regions added in a fixed order, back in
  // the row's element order
  __syncthreads();
  float* out = a.part + (int64_t)blockIdx.x * 2 * D;
  for (int k = threadIdx.x; k < 2 * D; k += kLnWaves * kWave) {
    const int h = k >= D ? 1 : 0, kk = k - h * D;
    const int src = h * D + (kk % VEC) * nch + kk / VEC;
    float v = wpart[src];
#pragma unroll
    for (int w = 1; w < kLnWaves; ++w) v += wpart[w * 2 * D + src];
    out[k] = v;
  }
}

// 64-row tiles covering max(R, ldo) rows (the column-sum partials)
__host__ __device__ __forceinline__ int transpose_row_tiles_dev(int64_t R, int64_t ldo) {
  return (int)(((R > ldo ? R : ldo) + 63) / 64);
}

struct TrArgs {
  const void* in;   // [G][R][C]: element (g, r, c) at g * in_gs + r * in_rs + c
  const void* aux;  // op 2: U, same layout as in
  void* out;        // [G][C][ldo]: out[g][c][r] = op(in[g][r][c]), zero for R <= r < rows covered
  void* direct;     // op 2, optional: op(in), element (g, r, c) at g * dir_gs + r * dir_rs + c
  void* out2;       // op 2, optional: GELU(aux) transposed like out
  float* colsum;    // optional [G][row tiles][C]: per 64-row tile sums of op(in) over r
  int64_t R, C, ldo, in_gs, in_rs, dir_gs, dir_rs;
};

// op 0: x;  op 1: GELU(x);  op 2: x * GELU'(aux)
template <typename T, int OP>
__global__ __launch_bounds__(256) void k_transpose(TrArgs a) {
  __shared__ float tile[64][65];
  __shared__ float tile2[OP == 2 ? 64 : 1][65];
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const T* in = (const T*)a.in + g * a.in_gs;
  {
    const int rl = tid >> 2, cl = (tid & 3) * 16;
    const int64_t r = r0 + rl;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t c = c0 + cl + 8 * h;
      float v[8];
      if (r < a.R && c < a.C) {
        load_f32<T, 8>(in + r * a.in_rs + c, v);
        if constexpr (OP == 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e]);
        } else if constexpr (OP == 2) {
          float u[8];
          load_f32<T, 8>((const T*)a.aux + g * a.in_gs + r * a.in_rs + c, u);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float gu, dgu;
            gelu_and_grad(u[e], gu, dgu);
            v[e] *= dgu;
            u[e] = gu;
          }
          if (a.direct) store_from_f32<T, 8>((T*)a.direct + g * a.dir_gs + r * a.dir_rs + c, v);
          if (a.out2)
#pragma unroll
            for (int e = 0; e < 8; ++e) tile2[rl][cl + 8 * h + e] = u[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
        if constexpr (OP == 2)
          if (a.out2)
#pragma unroll
            for (int e = 0; e < 8; ++e) tile2[rl][cl + 8 * h + e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[rl][cl + 8 * h + e] = v[e];
    }
  }
  __syncthreads();
  {
    const int cl = tid >> 2, rl = (tid & 3) * 16;
    const int64_t c = c0 + cl;
    float s = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t r = r0 + rl + 8 * h;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = tile[rl + 8 * h + e][cl];
        s += v[e];
      }
      if (c < a.C && r < a.ldo) store_from_f32<T, 8>((T*)a.out + g * a.C * a.ldo + c * a.ldo + r, v);
      if constexpr (OP == 2) {
        if (a.out2 && c < a.C && r < a.ldo) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = tile2[rl + 8 * h + e][cl];
          store_from_f32<T, 8>((T*)a.out2 + g * a.C * a.ldo + c * a.ldo + r, v);
        }
      }
    }
    if (a.colsum) {
      s += __shfl_xor(s, 1, kWave);
      s += __shfl_xor(s, 2, kWave);
      if ((tid & 3) == 0 && c < a.C) a.colsum[(g * gridDim.y + blockIdx.y) * a.C + c] = s;
    }
  }
}

// The GELU-derivative pass (op 2) in bf16, 128 x 128 tiles (256-byte row
// segments on both sides).  Phase 1: each thread loads 8 chunks of 8 elements
// of dH and U (rows tid/16 + 16i, columns (tid%16)*8), forms dU = dH GELU'(U),
// stores it directly (direct), keeps GELU(U) in registers and writes dU as
// bf16 into an LDS tile of row pitch 136.  Phase 2: each thread reads 32 rows
// of two adjacent columns (one 32-bit LDS read per row) and writes two
// 64-byte pieces of output rows; the per-64-row column sums come from the
// rounded values.  With out2, phase 2 runs a second time over GELU(U).  The 16-byte chunks of a row are
// XOR-swizzled by 4 x (row / 32 mod 4), so the four 32-row blocks a wave reads
// in phase 2 fall on disjoint banks.
constexpr int kTr = 128;       // tile edge
constexpr int kTrPitch = 136;  // LDS row pitch (elements)

// LDS element index of (row, column) in the swizzled tile
__device__ __forceinline__ int tr_lds(int row, int col) {
  return row * kTrPitch + (((col >> 3) ^ (((row >> 5) & 3) << 2)) << 3) + (col & 7);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(lo)) |
         ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(hi)) << 16);
}

__global__ __launch_bounds__(256) void k_gelu_bwd_t128(TrArgs a) {
  __shared__ __align__(16) bf16 tile[kTr * kTrPitch];
  const int tid = threadIdx.x;
  const int64_t g = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kTr, c0 = (int64_t)blockIdx.x * kTr;
  const bf16* in = (const bf16*)a.in + g * a.in_gs;
  const int ch = tid % 16;                 // column chunk of phase 1
  const int64_t cc = c0 + ch * 8;
  uint4 keep[8];                           // GELU(aux) of the 8 chunks, packed
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rl = tid / 16 + 16 * i;
    const int64_t r = r0 + rl;
    float v[8];
    const bool ok = r < a.R && cc < a.C;
    if (ok) {
      float u[8];
      load_f32<bf16, 8>(in + r * a.in_rs + cc, v);
      load_f32<bf16, 8>((const bf16*)a.aux + g * a.in_gs + r * a.in_rs + cc, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float gu, dgu;
        gelu_and_grad(u[e], gu, dgu);
        v[e] *= dgu;
        u[e] = gu;
      }
      if (a.direct) store_from_f32<bf16, 8>((bf16*)a.direct + g * a.dir_gs + r * a.dir_rs + cc, v);
      keep[i] = make_uint4(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]), pack_bf16x2(u[4], u[5]),
                           pack_bf16x2(u[6], u[7]));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
      keep[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    *reinterpret_cast<uint4*>(tile + tr_lds(rl, ch * 8)) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7]));
  }
  __syncthreads();
  // phase 2: columns cl, cl + 1 of the tile, rows q*32 .. q*32 + 31
  const int cl = (tid / 4) * 2, q = tid % 4;
  const int nrt = transpose_row_tiles_dev(a.R, a.ldo);
  auto out_pass = [&](bf16* out, bool sums) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(tile + tr_lds(q * 32 + k * 8 + e, cl));
        lo[e] = __uint_as_float(w << 16);
        hi[e] = __uint_as_float(w & 0xffff0000u);
        s0 += lo[e];
        s1 += hi[e];
      }
      const int64_t r = r0 + q * 32 + k * 8;
      if (r < a.ldo) {
        if (c0 + cl < a.C) store_from_f32<bf16, 8>(out + g * a.C * a.ldo + (c0 + cl) * a.ldo + r, lo);
        if (c0 + cl + 1 < a.C) store_from_f32<bf16, 8>(out + g * a.C * a.ldo + (c0 + cl + 1) * a.ldo + r, hi);
      }
    }
    if (sums) {
      // the two threads of one 64-row half are adjacent lanes
      s0 += __shfl_xor(s0, 1, kWave);
      s1 += __shfl_xor(s1, 1, kWave);
      const int half = (int)(blockIdx.y * 2) + q / 2;
      if ((q & 1) == 0 && half < nrt) {
        float* cs = a.colsum + (g * nrt + half) * a.C;
        if (c0 + cl < a.C) cs[c0 + cl] = s0;
        if (c0 + cl + 1 < a.C) cs[c0 + cl + 1] = s1;
      }
    }
  };
  out_pass((bf16*)a.out, a.colsum != nullptr);
  if (a.out2) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rl = tid / 16 + 16 * i;
      *reinterpret_cast<uint4*>(tile + tr_lds(rl, ch * 8)) = keep[i];
    }
    __syncthreads();
    out_pass((bf16*)a.out2, false);
  }
}

// dX[b,t,k] = dY1[b,t,k] + dY1[b, k/d, t*d + k%d]; VEC elements per thread
// never straddle a head
template <typename T, int VEC>
__global__ __launch_bounds__(256) void k_tm_add(const float* __restrict__ dy, T* __restrict__ dx, int64_t B, int T_,
                                                int D) {
  const int64_t n = B * T_ * (int64_t)D / VEC;
  const int d = D / T_;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = i * VEC;
    const int64_t b = e0 / ((int64_t)T_ * D);
    const int rem = (int)(e0 - b * T_ * (int64_t)D);
    const int t = rem / D, k = rem - t * D;
    const int tp = k / d, j = k - tp * d;
    float p[VEC], q[VEC];
    load_f32<float, VEC>(dy + e0, p);
    load_f32<float, VEC>(dy + b * T_ * (int64_t)D + (int64_t)tp * D + t * d + j, q);
#pragma unroll
    for (int e = 0; e < VEC; ++e) p[e] += q[e];
    store_from_f32<T, VEC>(dx + e0, p);
  }
}

// out[g][c] = sum over p < P of part[(g * P + p) * C + c]; columns c < split
// go to out0[g * split + c], the rest to out1[g * (C - split) + c - split].
// A workgroup owns 64 columns of one g: lane group q < S sums p = q, q + S,
// ... in order, then the group sums are added in order -- a fixed order
// throughout (S = 16 for many partials, 4 for few).
template <int S>
__global__ __launch_bounds__(64 * S) void k_sum_parts(const float* __restrict__ part, float* __restrict__ out0,
                                                      float* __restrict__ out1, int P, int64_t C, int64_t split,
                                                      float scale) {
  __shared__ float acc[S][64];
  const int cl = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t g = blockIdx.y, c = (int64_t)blockIdx.x * 64 + cl;
  float s = 0.f;
  if (c < C) {
    const float* p = part + g * P * C + c;
    int i = q;
    for (; i + 3 * S < P; i += 4 * S) {
      const float a0 = p[(int64_t)i * C], a1 = p[(int64_t)(i + S) * C], a2 = p[(int64_t)(i + 2 * S) * C],
                  a3 = p[(int64_t)(i + 3 * S) * C];
      s += a0;
      s += a1;
      s += a2;
      s += a3;
    }
    for (; i < P; i += S) s += p[(int64_t)i * C];
  }
  acc[q][cl] = s;
  __syncthreads();
  if (q == 0 && c < C) {
    float v = acc[0][cl];
#pragma unroll
    for (int k = 1; k < S; ++k) v += acc[k][cl];
    v *= scale;
    if (c < split)
      out0[g * split + c] = v;
    else
      out1[g * (C - split) + c - split] = v;
  }
}

// H = GELU(U), 8 elements per thread
template <typename T>
__global__ __launch_bounds__(256) void k_gelu_ew(const T* __restrict__ u, T* __restrict__ h, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    load_f32<T, 8>(u + i * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e]);
    store_from_f32<T, 8>(h + i * 8, v);
  }
}

int ln_slots(int chunks) {
  const int need = (chunks + kWave - 1) / kWave;
  if (need <= 1) return 1;
  if (need <= 2) return 2;
  if (need <= 4) return 4;
  if (need <= 8) return 8;
  if (need <= 16) return 16;
  return 0;
}

int chunk_of(int d, int eb) {
  const int max_e = 16 / eb;
  for (int v = max_e; v > 1; v >>= 1)
    if (d % v == 0) return v;
  return 1;
}

template <typename T, int VEC, int MODE>
hipError_t ln_bwd_vec(const LnBwdArgs& a, int grid, hipStream_t s) {
  const dim3 block(kLnWaves * kWave);
  const size_t lds = (size_t)kLnWaves * 2 * a.D * sizeof(float);
  const int need = (a.D / VEC + kWave - 1) / kWave;
  switch (MODE == 0 && need == 3 ? 3 : ln_slots(a.D / VEC)) {
    case 1: hipLaunchKernelGGL((k_ln_bwd<T, VEC, 1, MODE>), dim3(grid), block, lds, s, a); break;
    case 3: hipLaunchKernelGGL((k_ln_bwd<T, VEC, 3, MODE>), dim3(grid), block, lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_ln_bwd<T, VEC, 2, MODE>), dim3(grid), block, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_ln_bwd<T, VEC, 4, MODE>), dim3(grid), block, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_ln_bwd<T, VEC, 8, MODE>), dim3(grid), block, lds, s, a); break;
    case 16: hipLaunchKernelGGL((k_ln_bwd<T, VEC, 16, MODE>), dim3(grid), block, lds, s, a); break;
    default: return hipErrorInvalidValue;  // a row wider than 1024 chunks
  }
  return hipGetLastError();
}

template <typename T, int MODE>
hipError_t ln_bwd_t(const LnBwdArgs& a, int grid, hipStream_t s) {
  // mode 1 gathers within heads: chunks must not straddle one
  const int vec = MODE == 0 ? 8 : chunk_of(a.D / a.T, (int)sizeof(T));
  switch (vec) {
    case 8: return ln_bwd_vec<T, 8, MODE>(a, grid, s);
    case 4: return ln_bwd_vec<T, 4, MODE>(a, grid, s);
    case 2: return ln_bwd_vec<T, 2, MODE>(a, grid, s);
    default: return ln_bwd_vec<T, 1, MODE>(a, grid, s);
  }
}

}  // namespace

int ln_bwd_grid(int64_t B, int T, int D) {
  // as many workgroups as fit on every CU at once (their per-wave gamma /
  // beta partials take kLnWaves * 2 * D floats of LDS; at most 8 per CU),
  // but at least ~8 rows per wave
  const int64_t rows = B * T;
  const int64_t lds = (int64_t)kLnWaves * 2 * std::max(D, 8) * 4;
  const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(8, (160 * 1024) / lds));
  const int64_t want = (rows + kLnWaves * 8 - 1) / (kLnWaves * 8);
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, per_cu * (int64_t)device_cus()));
}

int ln_bwd_max_width() { return kLnBwdDmax; }

hipError_t launch_ln_bwd(int mode, const void* dout, const void* dres, const float* dres32, const void* z,
                         const void* res, const float* gamma, void* dy, float* part, int64_t B, int T, int D, int dt,
                         hipStream_t s, const float* dres32b) {
  if (D > kLnBwdDmax || D % 8 || D % T) return hipErrorInvalidValue;
  LnBwdArgs a{dout, dres, dres32, dres32b, z, res, gamma, dy, part, B, T, D};
  const int grid = ln_bwd_grid(B, T, D);
  if (dt == kBF16)
    return mode == 0 ? ln_bwd_t<bf16, 0>(a, grid, s) : ln_bwd_t<bf16, 1>(a, grid, s);
  return mode == 0 ? ln_bwd_t<float, 0>(a, grid, s) : ln_bwd_t<float, 1>(a, grid, s);
}

int transpose_row_tiles(int64_t R, int64_t ldo) { return (int)((std::max(R, ldo) + 63) / 64); }

hipError_t launch_transpose(int op, const void* in, const void* aux, void* out, void* direct, void* out2,
                            float* colsum, int G, int64_t R, int64_t C, int64_t ldo, int dt, hipStream_t s,
                            int64_t in_gs, int64_t in_rs, int64_t dir_gs, int64_t dir_rs) {
  if (C % 8 || ldo % 8 || ldo < R || G <= 0) return hipErrorInvalidValue;
  if (in_rs < 0) in_rs = C;
  if (in_gs < 0) in_gs = R * in_rs;
  if (in_rs % 8 || in_gs % 8 || in_rs < C) return hipErrorInvalidValue;
  if (dir_rs < 0) dir_rs = in_rs;
  if (dir_gs < 0) dir_gs = in_gs;
  if (dir_rs % 8 || dir_gs % 8 || dir_rs < C) return hipErrorInvalidValue;
  if (R == 0 && ldo == 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)transpose_row_tiles(R, ldo), (unsigned)G);
  TrArgs a{in, aux, out, direct, out2, colsum, R, C, ldo, in_gs, in_rs, dir_gs, dir_rs};
  const dim3 block(256);
  if (dt == kBF16) {
    // the GELU-derivative pass (two inputs, up to three outputs) runs faster in
    // 128 x 128 tiles; plain transposes in 64 x 64 ones (measured)
    const dim3 g128((unsigned)((C + kTr - 1) / kTr), (unsigned)((std::max(R, ldo) + kTr - 1) / kTr), (unsigned)G);
    switch (op) {
      case 0: hipLaunchKernelGGL((k_transpose<bf16, 0>), grid, block, 0, s, a); break;
      case 1: hipLaunchKernelGGL((k_transpose<bf16, 1>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL(k_gelu_bwd_t128, g128, block, 0, s, a); break;
    }
  } else {
    switch (op) {
      case 0: hipLaunchKernelGGL((k_transpose<float, 0>), grid, block, 0, s, a); break;
      case 1: hipLaunchKernelGGL((k_transpose<float, 1>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((k_transpose<float, 2>), grid, block, 0, s, a); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_tm_add(const float* dy, void* dx, int64_t B, int T, int D, int dt, hipStream_t s) {
  const int vec = chunk_of(D / T, 4);  // fp32 input: at most 4 elements per 16 bytes
  const int64_t n = B * T * (int64_t)D / vec;
  const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536)));
  if (dt == kBF16) {
    switch (vec) {
      case 4: hipLaunchKernelGGL((k_tm_add<bf16, 4>), grid, dim3(256), 0, s, dy, (bf16*)dx, B, T, D); break;
      case 2: hipLaunchKernelGGL((k_tm_add<bf16, 2>), grid, dim3(256), 0, s, dy, (bf16*)dx, B, T, D); break;
      default: hipLaunchKernelGGL((k_tm_add<bf16, 1>), grid, dim3(256), 0, s, dy, (bf16*)dx, B, T, D); break;
    }
  } else {
    switch (vec) {
      case 4: hipLaunchKernelGGL((k_tm_add<float, 4>), grid, dim3(256), 0, s, dy, (float*)dx, B, T, D); break;
      case 2: hipLaunchKernelGGL((k_tm_add<float, 2>), grid, dim3(256), 0, s, dy, (float*)dx, B, T, D); break;
      default: hipLaunchKernelGGL((k_tm_add<float, 1>), grid, dim3(256), 0, s, dy, (float*)dx, B, T, D); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_sum_parts(const float* part, float* out0, float* out1, int G, int P, int64_t C, int64_t split,
                            hipStream_t s, float scale) {
  if ((int64_t)G * C == 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)G);
  if (P >= 64)
    hipLaunchKernelGGL(k_sum_parts<16>, grid, dim3(64 * 16), 0, s, part, out0, out1, P, C, split, scale);
  else
    hipLaunchKernelGGL(k_sum_parts<4>, grid, dim3(64 * 4), 0, s, part, out0, out1, P, C, split, scale);
  return hipGetLastError();
}

// part[g][b][c] = the sum of in[g][r][c] over rows r = 64 b .. 64 b + 63 (< R):
// one thread per 16-byte chunk of columns, rows in order
template <typename T>
__global__ __launch_bounds__(256) void k_colsum64(const T* __restrict__ in, float* __restrict__ part, int64_t R,
                                                  int64_t C, int P) {
  const int64_t g = blockIdx.z, b = blockIdx.y;
  const int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (c >= C) return;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t r0 = b * 64, r1 = min(R, r0 + 64);
  const T* src = in + g * R * C + c;
#pragma unroll 8
  for (int64_t r = r0; r < r1; ++r) {
    float v[8];
    load_f32<T, 8>(src + r * C, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] += v[e];
  }
  float* dst = part + (g * P + b) * C + c;
  *reinterpret_cast<float4*>(dst) = make_float4(s[0], s[1], s[2], s[3]);
  *reinterpret_cast<float4*>(dst + 4) = make_float4(s[4], s[5], s[6], s[7]);
}

int colsum64_parts(int64_t R) { return (int)((R + 63) / 64); }

hipError_t launch_colsum64(const void* in, float* part, int G, int64_t R, int64_t C, int dt, hipStream_t s) {
  if (C % 8) return hipErrorInvalidValue;
  if (G == 0 || R == 0 || C == 0) return hipSuccess;
  const int P = colsum64_parts(R);
  const dim3 grid((unsigned)((C / 8 + 255) / 256), (unsigned)P, (unsigned)G);
  if (dt == kBF16)
    hipLaunchKernelGGL((k_colsum64<bf16>), grid, dim3(256), 0, s, (const bf16*)in, part, R, C, P);
  else
    hipLaunchKernelGGL((k_colsum64<float>), grid, dim3(256), 0, s, (const float*)in, part, R, C, P);
  return hipGetLastError();
}

hipError_t launch_gelu_ew(const void* u, void* h, int64_t n, int dt, hipStream_t s) {
  if (n % 8) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>((n8 + 255) / 256, 65536)));
  if (dt == kBF16)
    hipLaunchKernelGGL((k_gelu_ew<bf16>), grid, dim3(256), 0, s, (const bf16*)u, (bf16*)h, n8);
  else
    hipLaunchKernelGGL((k_gelu_ew<float>), grid, dim3(256), 0, s, (const float*)u, (float*)h, n8);
  return hipGetLastError();
}

}  // namespace rm

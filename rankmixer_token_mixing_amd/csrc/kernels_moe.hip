// ReLU-gated per-token MoE around the grouped GEMMs: the router, the
// compaction of active (sample, token, expert) rows into per-(token, expert)
// lists, and the deterministic combine (+ residual + LayerNorm).
//
// Routing follows the ReLU router of "Rankmixer: 硬件效率优化", section
// "Sparse MoE扩展": G = ReLU(h(s)), expert j of token t runs only where its
// gate is positive.  Lists are built without any host round trip: counts,
// an exclusive scan and a stable scatter, all on the device.
#include "common.hpp"
#include "launch.hpp"

namespace rm {

namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kMaxGroups = 4096;  // T * E

int pick_slots(int chunks) {
  const int need = (chunks + kWave - 1) / kWave;
  if (need <= 1) return 1;
  if (need <= 2) return 2;
  if (need <= 4) return 4;
  if (need <= 8) return 8;
  if (need <= 16) return 16;
  return 0;
}

// gates[b,t,j] = max(0, Wr[t,j,:] . s[b,t,:] + br[t,j]); one wave per (b, t),
// the waves walking the samples of one token together so that token's router
// rows stay in the near caches
template <typename T, int VEC, int MAXI>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void k_router(const T* __restrict__ s, int64_t sb, int64_t st,
                                                                  const T* __restrict__ wr,
                                                                  const float* __restrict__ br,
                                                                  float* __restrict__ gates, int64_t B, int T_,
                                                                  int D, int E) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= B * T_) return;
  const int lane = lane_id();
  const int t = (int)(row / B);
  const int64_t b = row - (int64_t)t * B;
  const int nch = D / VEC;
  const T* sr = s + b * sb + t * st;
  float v[MAXI][VEC];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) load_f32<T, VEC>(sr + c * VEC, v[i]);
  }
  for (int j = 0; j < E; ++j) {
    const T* w = wr + ((int64_t)t * E + j) * D;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      if (c < nch) {
        float q[VEC];
        load_f32<T, VEC>(w + c * VEC, q);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc += v[i][e] * q[e];
      }
    }
    const float z = wave_sum(acc) + br[t * E + j];
    if (lane == j % kWave) gates[(b * T_ + t) * E + j] = z > 0.f ? z : 0.f;
  }
}

// The same gates for E <= 8 experts with the token's router rows staged in
// LDS: workgroup (x, t) takes samples [16x, 16x + 16) of token t, a wave four
// of them, whose S rows it loads at once (clamped addresses, so the loads
// issue back to back).  Each lane forms its partial dot products for all
// experts and rows; per row a butterfly that halves the experts per lane at
// each of the first three exchange steps (32, 16, 8 lanes apart) and then sums
// across the remaining 8 lanes reduces the 8 partial sums in 6 exchanges.
constexpr int kRouterRowsPerWave = 4;
constexpr int kRouterRows = 4 * kRouterRowsPerWave;  // samples per workgroup (4 waves)
constexpr int kRouterMaxE = 8;
constexpr int kRouterLds = 65536;  // bytes of router rows staged per workgroup

template <typename T, int VEC, int MAXI>
__global__ __launch_bounds__(256) void k_router_lds(const T* __restrict__ s, int64_t sb, int64_t st,
                                                    const T* __restrict__ wr, const float* __restrict__ br,
                                                    float* __restrict__ gates, int64_t B, int T_, int D, int E) {
  constexpr int R = kRouterRowsPerWave;
  extern __shared__ uint4 wl_raw[];
  const T* wl = reinterpret_cast<const T*>(wl_raw);
  const int t = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  {
    const uint4* src = reinterpret_cast<const uint4*>(wr + (int64_t)t * E * D);
    const int n16 = E * D * (int)sizeof(T) / 16;
    for (int i = threadIdx.x; i < n16; i += 256) wl_raw[i] = src[i];
  }
  const int nch = D / VEC;
  const int64_t b0 = (int64_t)blockIdx.x * kRouterRows + wave * R;
  float v[R][MAXI][VEC];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t b = b0 + r < B ? b0 + r : B - 1;
    const T* sr = s + b * sb + t * st;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      load_f32<T, VEC>(sr + (c < nch ? c : nch - 1) * VEC, v[r][i]);
    }
  }
  __syncthreads();
  float acc[R][kRouterMaxE];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < kRouterMaxE; ++j) acc[r][j] = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
#pragma unroll
      for (int j = 0; j < kRouterMaxE; ++j) {
        if (j < E) {
          float q[VEC];
          load_f32<T, VEC>(wl + j * D + c * VEC, q);
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[r][j] = fmaf(v[r][i][e], q[e], acc[r][j]);
        }
      }
    }
  }
  const int e_of = ((lane >> 5) & 1) * 4 + ((lane >> 4) & 1) * 2 + ((lane >> 3) & 1);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // 8 -> 4 -> 2 -> 1 experts per lane, then the sum over 8 lanes
    float* a = acc[r];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool hi = lane & 32;
      const float keep = hi ? a[k + 4] : a[k], give = hi ? a[k] : a[k + 4];
      a[k] = keep + __shfl_xor(give, 32, kWave);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const bool hi = lane & 16;
      const float keep = hi ? a[k + 2] : a[k], give = hi ? a[k] : a[k + 2];
      a[k] = keep + __shfl_xor(give, 16, kWave);
    }
    {
      const bool hi = lane & 8;
      const float keep = hi ? a[1] : a[0], give = hi ? a[0] : a[1];
      a[0] = keep + __shfl_xor(give, 8, kWave);
    }
    float z = a[0];
    z += __shfl_xor(z, 1, kWave);
    z += __shfl_xor(z, 2, kWave);
    z += __shfl_xor(z, 4, kWave);
    const int64_t b = b0 + r;
    if ((lane & 7) == 0 && e_of < E && b < B) {
      z += br[t * E + e_of];
      gates[(b * T_ + t) * E + e_of] = z > 0.f ? z : 0.f;
    }
  }
}

// threads per workgroup of the count and the scatter: one workgroup per
// (token, expert) group walks the batch in strides of this many samples
constexpr int kCompactThreads = 1024;

// counts[g] = #{b : gates[b, g] > 0}, g = t*E + j; one workgroup per group
__global__ __launch_bounds__(kCompactThreads) void k_moe_count(const float* __restrict__ gates,
                                                               int* __restrict__ counts, int64_t B, int G) {
  constexpr int NW = kCompactThreads / kWave;
  const int g = blockIdx.x;
  int c = 0;
  for (int64_t b = threadIdx.x; b < B; b += blockDim.x) c += gates[b * G + g] > 0.f ? 1 : 0;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, kWave);
  __shared__ int part[NW];
  if (lane_id() == 0) part[threadIdx.x / kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) n += part[w];
    counts[g] = n;
  }
}

// offsets = exclusive scan of counts; tile list of (g, m0) pairs with bm rows
// per tile; ntiles = its length.  One workgroup of 256 threads; thread i
// owns groups [i*per, (i+1)*per).
__global__ __launch_bounds__(256) void k_moe_scan(const int* __restrict__ counts, int* __restrict__ offsets,
                                                  int* __restrict__ tiles, int* __restrict__ ntiles, int G,
                                                  int bm) {
  __shared__ int s_rows[256], s_tiles[256];
  const int per = (G + 255) / 256;
  const int g0 = threadIdx.x * per;
  int my_rows = 0, my_tiles = 0;
  for (int g = g0; g < g0 + per && g < G; ++g) {
    my_rows += counts[g];
    my_tiles += (counts[g] + bm - 1) / bm;
  }
  s_rows[threadIdx.x] = my_rows;
  s_tiles[threadIdx.x] = my_tiles;
  __syncthreads();
  // inclusive Hillis-Steele scan over the 256 partial sums
  for (int off = 1; off < 256; off <<= 1) {
    const int r = threadIdx.x >= off ? s_rows[threadIdx.x - off] : 0;
    const int q = threadIdx.x >= off ? s_tiles[threadIdx.x - off] : 0;
    __syncthreads();
    s_rows[threadIdx.x] += r;
    s_tiles[threadIdx.x] += q;
    __syncthreads();
  }
  int o = s_rows[threadIdx.x] - my_rows;
  int to = s_tiles[threadIdx.x] - my_tiles;
  for (int g = g0; g < g0 + per && g < G; ++g) {
    const int c = counts[g];
    offsets[g] = o;
    const int nt = (c + bm - 1) / bm;
    for (int i = 0; i < nt; ++i) {
      tiles[2 * (to + i)] = g;
      tiles[2 * (to + i) + 1] = i * bm;
    }
    o += c;
    to += nt;
  }
  if (threadIdx.x == 255) {
    offsets[G] = s_rows[255];
    *ntiles = s_tiles[255];
  }
}

// stable scatter: entry offsets[g] + rank of each active b (in increasing b)
__global__ __launch_bounds__(kCompactThreads) void k_moe_scatter(const float* __restrict__ gates,
                                                                 const int* __restrict__ offsets,
                                                                 int* __restrict__ rows, float* __restrict__ gatec,
                                                                 int* __restrict__ pos, int64_t B, int G) {
  constexpr int NW = kCompactThreads / kWave;
  const int g = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  __shared__ int wtot[NW];
  int running = offsets[g];
  for (int64_t base = 0; base < B; base += blockDim.x) {
    const int64_t b = base + threadIdx.x;
    const float gv = b < B ? gates[b * G + g] : 0.f;
    const bool on = gv > 0.f;
    const unsigned long long mask = __ballot(on);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[wave] = __popcll(mask);
    __syncthreads();
    int wbase = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      wbase += w < wave ? wtot[w] : 0;
      total += wtot[w];
    }
    if (b < B) {
      if (on) {
        const int idx = running + wbase + before;
        rows[idx] = (int)b;
        gatec[idx] = gv;
        pos[b * G + g] = idx;
      } else {
        pos[b * G + g] = -1;
      }
    }
    running += total;
    __syncthreads();
  }
}

// v = sum_j y[pos[b,t,j]] (fixed j order); out = ln ? LN(v + s) : v
template <typename T, int VEC, int MAXI>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void k_moe_combine(const T* __restrict__ y,
                                                                       const int* __restrict__ pos,
                                                                       const T* __restrict__ s, int64_t sb,
                                                                       int64_t st, int T_,
                                                                       const float* __restrict__ g,
                                                                       const float* __restrict__ beta,
                                                                       T* __restrict__ out, int64_t rows_n,
                                                                       int D, int E, int ln) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= rows_n) return;
  const int lane = lane_id();
  const int nch = D / VEC;
  float v[MAXI][VEC];
#pragma unroll
  for (int i = 0; i < MAXI; ++i)
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[i][e] = 0.f;
  // the row's active experts as a wave-uniform bit mask (lane j < E holds
  // pos[row][j]); two rows of y are loaded per step, both issued before
  // either is added, and added in expert order
  const int pj = lane < E ? pos[row * E + lane] : -1;
  // the residual row, loaded ahead of the expert rows
  float r[MAXI][VEC];
  if (ln) {
    const T* sr = s + (row / T_) * sb + (row % T_) * st;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) load_f32<T, VEC>(sr + min(lane + i * kWave, nch - 1) * VEC, r[i]);
  }
  unsigned long long act = __ballot(pj >= 0);
  while (act) {
    const int j0 = __builtin_ctzll(act);
    act &= act - 1;
    const int p0 = __shfl(pj, j0, kWave);
    int p1 = -1;
    if (act) {
      const int j1 = __builtin_ctzll(act);
      act &= act - 1;
      p1 = __shfl(pj, j1, kWave);
    }
    const T* y0 = y + (int64_t)p0 * D;
    const T* y1 = y + (int64_t)(p1 >= 0 ? p1 : p0) * D;
    float q0[MAXI][VEC], q1[MAXI][VEC];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = min(lane + i * kWave, nch - 1);
      load_f32<T, VEC>(y0 + c * VEC, q0[i]);
      load_f32<T, VEC>(y1 + c * VEC, q1[i]);
    }
#pragma unroll
    for (int i = 0; i < MAXI; ++i)
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[i][e] += q0[i][e];
    if (p1 >= 0) {
#pragma unroll
      for (int i = 0; i < MAXI; ++i)
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[i][e] += q1[i][e];
    }
  }
  T* orow = out + row * (int64_t)D;
  if (!ln) {
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int c = lane + i * kWave;
      if (c < nch) store_from_f32<T, VEC>(orow + c * VEC, v[i]);
    }
    return;
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + i * kWave;
    if (c < nch) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        v[i][e] += r[i][e];
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
      for (int e = 0; e < VEC; ++e) {
        const float q = v[i][e] - mean;
        sq += q * q;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) / (float)D + 1e-5f);
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

template <typename T, int VEC>
hipError_t router_t(const void* s, int64_t sb, int64_t sT, const void* wr, const float* br, float* gates,
                    int64_t B, int T_, int D, int E, hipStream_t st) {
  const dim3 grid((unsigned)((B * T_ + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * kWave);
  const T* ss = (const T*)s;
  const T* ww = (const T*)wr;
  switch (pick_slots(D / VEC)) {
    case 0: return hipErrorInvalidValue;
    case 1: hipLaunchKernelGGL((k_router<T, VEC, 1>), grid, block, 0, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
    case 2: hipLaunchKernelGGL((k_router<T, VEC, 2>), grid, block, 0, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
    case 4: hipLaunchKernelGGL((k_router<T, VEC, 4>), grid, block, 0, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
    case 8: hipLaunchKernelGGL((k_router<T, VEC, 8>), grid, block, 0, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
    default: hipLaunchKernelGGL((k_router<T, VEC, 16>), grid, block, 0, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
  }
  return hipGetLastError();
}

template <typename T, int VEC>
hipError_t router_lds_t(const void* s, int64_t sb, int64_t sT, const void* wr, const float* br, float* gates,
                        int64_t B, int T_, int D, int E, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)((B + kRouterRows - 1) / kRouterRows), (unsigned)T_), block(256);
  const size_t lds = (size_t)E * D * sizeof(T);
  const T* ss = (const T*)s;
  const T* ww = (const T*)wr;
  switch (pick_slots(D / VEC)) {
    case 0: return hipErrorInvalidValue;
    case 1: hipLaunchKernelGGL((k_router_lds<T, VEC, 1>), grid, block, lds, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
    case 2: hipLaunchKernelGGL((k_router_lds<T, VEC, 2>), grid, block, lds, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
    case 4: hipLaunchKernelGGL((k_router_lds<T, VEC, 4>), grid, block, lds, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
    case 8: hipLaunchKernelGGL((k_router_lds<T, VEC, 8>), grid, block, lds, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
    default: hipLaunchKernelGGL((k_router_lds<T, VEC, 16>), grid, block, lds, st, ss, sb, sT, ww, br, gates, B, T_, D, E); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t combine_t(const void* yv, const int* pos, const void* s, int64_t sb, int64_t sT, const float* g,
                     const float* b, void* out, int64_t B, int T_, int D, int E, bool ln, hipStream_t st) {
  const int64_t rows = B * T_;
  const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), block(kRowsPerBlock * kWave);
  const T* ss = (const T*)s;
  const T* y = (const T*)yv;
  T* oo = (T*)out;
  const int l = ln ? 1 : 0;
  constexpr int VEC = sizeof(T) == 2 ? 8 : 4;  // 16-byte chunks
  switch (pick_slots(D / VEC)) {
    case 0: return hipErrorInvalidValue;
    case 1: hipLaunchKernelGGL((k_moe_combine<T, VEC, 1>), grid, block, 0, st, y, pos, ss, sb, sT, T_, g, b, oo, rows, D, E, l); break;
    case 2: hipLaunchKernelGGL((k_moe_combine<T, VEC, 2>), grid, block, 0, st, y, pos, ss, sb, sT, T_, g, b, oo, rows, D, E, l); break;
    case 4: hipLaunchKernelGGL((k_moe_combine<T, VEC, 4>), grid, block, 0, st, y, pos, ss, sb, sT, T_, g, b, oo, rows, D, E, l); break;
    case 8: hipLaunchKernelGGL((k_moe_combine<T, VEC, 8>), grid, block, 0, st, y, pos, ss, sb, sT, T_, g, b, oo, rows, D, E, l); break;
    default: hipLaunchKernelGGL((k_moe_combine<T, VEC, 16>), grid, block, 0, st, y, pos, ss, sb, sT, T_, g, b, oo, rows, D, E, l); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe_router(const void* s, int64_t sb, int64_t sT, const void* wr, const float* br, float* gates,
                             int64_t B, int T, int D, int E, int dt, hipStream_t st) {
  // the staged kernel keeps four S rows per lane in registers: up to four
  // 16-byte chunks of each
  const int eb = dt == kBF16 ? 2 : 4;
  if (E <= kRouterMaxE && (int64_t)E * D * eb <= kRouterLds && D * eb <= 4 * kWave * 16) {
    if (dt == kBF16) return router_lds_t<bf16, 8>(s, sb, sT, wr, br, gates, B, T, D, E, st);
    return router_lds_t<float, 4>(s, sb, sT, wr, br, gates, B, T, D, E, st);
  }
  if (dt == kBF16) return router_t<bf16, 8>(s, sb, sT, wr, br, gates, B, T, D, E, st);
  return router_t<float, 4>(s, sb, sT, wr, br, gates, B, T, D, E, st);
}

hipError_t launch_moe_compact(const MoeWork& w, int64_t B, int T, int E, int bm, hipStream_t st) {
  const int G = T * E;
  if (G > kMaxGroups) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_moe_count, dim3(G), dim3(kCompactThreads), 0, st, w.gates, w.counts, B, G);
  hipLaunchKernelGGL(k_moe_scan, dim3(1), dim3(256), 0, st, w.counts, w.offsets, w.tiles, w.ntiles, G, bm);
  hipLaunchKernelGGL(k_moe_scatter, dim3(G), dim3(kCompactThreads), 0, st, w.gates, w.offsets, w.rows, w.gatec,
                     w.pos, B, G);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const void* y, const int* pos, const void* s, int64_t sb, int64_t sT, const float* g,
                              const float* b, void* out, int64_t B, int T, int D, int E, bool ln, int dt,
                              hipStream_t st) {
  if (dt == kBF16) return combine_t<bf16>(y, pos, s, sb, sT, g, b, out, B, T, D, E, ln, st);
  return combine_t<float>(y, pos, s, sb, sT, g, b, out, B, T, D, E, ln, st);
}

}  // namespace rm

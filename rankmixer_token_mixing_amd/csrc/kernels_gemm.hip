// Grouped MFMA GEMM with fused epilogues: the two products of the per-token
// FFN ("Rankmixer: 硬件效率优化", section "Per-Token FFN": T independent
// FFNs, run as one grouped [T,B,d] x [T,d,h] product as in section 3.2 of
// "重新理解 RankMixer：扩参为什么有效，又为什么划算？") and the ragged
// per-(token, expert) products of the ReLU MoE.
//
// C_g[m][n] = sum_k A_g[m][k] W_g[n][k]: both operands are read along k
// (weights stored [out][in]).  One workgroup computes a BM x BN tile of one
// group.  Operand k-slices stream straight from global memory into LDS with
// global_load_lds_dwordx4 (no VGPR staging); LDS rows are 8 chunks of 16
// bytes, XOR-swizzled (chunk ^ (row/2 mod 8)) so the 32-row fragment reads of
// a wave hit distinct banks, and the DMA writes 1 KB contiguous per
// instruction with each lane fetching the global chunk that belongs at its
// swizzled slot.  Each wave multiplies an FM x FN grid of 32x32 blocks with
// v_mfma_f32_32x32x16_bf16 (fp32 data: 4 x v_mfma_f32_32x32x2f32), fp32
// accumulators in registers, the weight fragment as first MFMA operand so a
// lane ends up holding 4 consecutive output columns of one row.
//
// Two main loops:
//  * ring (bf16, K a multiple of 64): k-slices of 64 (one full 128-byte cache
//    line per row), five LDS slots of max(BM,BN) rows each; stage k reads
//    slots 2k%5 (A) and (2k+1)%5 (W) and, once every wave has passed the
//    stage barrier, refills the two slots stage k-1 used with W_{k+1} and
//    A_{k+2}.  Three k-slices (96 KB for 256x256) are always in flight, which
//    is what the L2 -> LDS path needs to stream full lines at rate; the slots
//    are separate LDS objects and the loop is unrolled by 5 so the compiler's
//    DMA wait tracking sees which slot each read touches.
//  * generic (fp32, or K not a multiple of 64): two LDS stages, chunks past K
//    fetched from a 16-byte zero block.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"
#include "frag.hpp"
#include "launch.hpp"

namespace rm {

namespace {


struct KParams {
  const void* A;
  long long a_gs, a_rs;
  int a_gdiv;
  const int* a_rowidx;
  const void* W;
  long long b_gs;
  int b_gdiv;
  void* C;
  long long c_gs, c_rs;
  void* C2;  // kEpiBiasGeluDual: GELU(C), same layout as C
  const void* aux;  // kEpiGeluBwd: the pre-activation, group g row m at g * aux_gs + m * aux_rs
  long long aux_gs, aux_rs;
  float* colsum;    // kEpiGeluBwd: partial column sums
  const float* bias;
  long long bias_gs;
  const float* rowscale;
  const int* row_off;
  const int* tiles;
  const int* ntiles;
  int M, N, K, G, tiles_m, tiles_n;
  int n_fast;  // dense: consecutive tiles walk the N tiles of one M row (else the M tiles of one N column)
};

// 16 zero bytes: the source of every chunk that lies past K
__device__ __align__(16) uint4 g_zero_chunk = {0, 0, 0, 0};

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  // 2 chunks (lane halves) x 8 bf16 = 16 k per MFMA
  static __device__ __forceinline__ void run(floatx16& c, const uint4& a, const uint4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                0, 0, 0);
  }
};

template <> struct Mma<float> {
  // 2 chunks x 4 fp32 = 8 k: element e of every lane's chunk is the k-slice of
  // MFMA e, the same slice in both operands
  static __device__ __forceinline__ void run(floatx16& c, const uint4& a, const uint4& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};


template <int EPI, typename T>
struct OutType {
  typedef typename std::conditional<EPI == kEpiBiasGelu || EPI == kEpiBias || EPI == kEpiBiasScale ||
                                        EPI == kEpiBiasGeluDual || EPI == kEpiGeluBwd,
                                    T, float>::type type;
};

// which tile this workgroup owns
struct TileId {
  int g, m0, n0, Mg;
  long long row_base;
};

template <bool RAGGED, int BM, int BN>
__device__ __forceinline__ bool tile_id(const KParams& p, TileId& t) {
  if constexpr (RAGGED) {
    const int nv = (*p.ntiles) * p.tiles_n;
    if ((int)blockIdx.x >= nv) return false;
    const int lid = xcd_remap(blockIdx.x, nv);
    const int slot = lid / p.tiles_n;
    t.n0 = (lid - slot * p.tiles_n) * BN;
    t.g = p.tiles[2 * slot];
    t.m0 = p.tiles[2 * slot + 1];
    t.row_base = p.row_off[t.g];
    t.Mg = p.row_off[t.g + 1] - (int)t.row_base;
  } else {
    // consecutive ids (one XCD after xcd_remap) walk the M tiles of one N
    // column first (or, n_fast, the N tiles of one M row), so concurrently
    // running tiles share W panels and A panels
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int per = p.tiles_m * p.tiles_n;
    t.g = lid / per;
    const int r = lid - t.g * per;
    const int tn = p.n_fast ? r % p.tiles_n : r / p.tiles_m;
    const int tm = p.n_fast ? r / p.tiles_n : r - tn * p.tiles_m;
    t.m0 = tm * BM;
    t.n0 = tn * BN;
    t.row_base = 0;
    t.Mg = p.M;
  }
  return true;
}

// epilogue math on 4 consecutive columns of one row
template <int EPI, typename T>
__device__ __forceinline__ void epi4(const KParams& p, const TileId& t, int m, int n, float scale, float (&v)[4]) {
  if constexpr (EPI == kEpiBiasGelu) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = gelu_erf(v[e]);
  }
  if constexpr (EPI == kEpiBiasScale) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= scale;
  }
}

// direct epilogue: block (i, j), register 4q+e holds row m0 + wm*FM*32 + i*32 + lr,
// column n0 + wn*FN*32 + j*32 + 8q + 4lh + e
template <typename T, int FM, int FN, int EPI>
__device__ __forceinline__ void store_direct(const KParams& p, const TileId& t, const floatx16 (&acc)[FM][FN], int wm,
                                             int wn, int lr, int lh) {
  typedef typename OutType<EPI, T>::type TO;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = t.m0 + wm * FM * 32 + i * 32 + lr;
    if (m >= t.Mg) continue;
    const long long orow = (t.row_base + m) * p.c_rs + (long long)t.g * p.c_gs;
    float scale = 1.f;
    if constexpr (EPI == kEpiBiasScale) scale = p.rowscale[t.row_base + m];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = t.n0 + wn * FN * 32 + j * 32 + 8 * q + 4 * lh;
        if (n >= p.N) continue;
        float4 bias = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.bias) bias = *reinterpret_cast<const float4*>(p.bias + (long long)t.g * p.bias_gs + n);
        float v[4] = {acc[i][j][4 * q + 0] + bias.x, acc[i][j][4 * q + 1] + bias.y, acc[i][j][4 * q + 2] + bias.z,
                      acc[i][j][4 * q + 3] + bias.w};
        epi4<EPI, T>(p, t, m, n, scale, v);
        store_from_f32<TO, 4>((TO*)p.C + orow + n, v);
      }
    }
  }
}

// ===========================================================================
// generic main loop: two LDS stages, any K (multiple of the chunk), bf16/fp32

template <typename T, int NWM, int NWN, int FM, int FN>
struct Tile {
  static constexpr int NW = NWM * NWN;
  static constexpr int NT = NW * kWave;
  static constexpr int BM = NWM * FM * 32, BN = NWN * FN * 32;
  static constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
  static constexpr int BK = kCpr * EPC;             // k per stage
  static constexpr int A_DMA = BM / 8 / NW;         // 1 KB DMA blocks per wave
  static constexpr int B_DMA = BN / 8 / NW;
  static constexpr int STAGE = (BM + BN) * kCpr;    // uint4 per stage
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile rows must split into 1 KB blocks per wave");
};

template <typename T, int NWM, int NWN, int FM, int FN, int EPI, bool RAGGED, bool AIDX>
__global__ __launch_bounds__(NWM* NWN* kWave) void k_gemm_generic(KParams p) {
  typedef Tile<T, NWM, NWN, FM, FN> TL;
  constexpr int BM = TL::BM, BN = TL::BN, EPC = TL::EPC, BK = TL::BK;
  constexpr int A_DMA = TL::A_DMA, B_DMA = TL::B_DMA;

  __shared__ uint4 lds0[TL::STAGE];
  __shared__ uint4 lds1[TL::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  TileId t;
  if (!tile_id<RAGGED, BM, BN>(p, t)) return;

  // DMA sources: wave w fills 1 KB blocks w, w+NW, ... of each operand tile;
  // block b holds tile rows 8b..8b+7, lane L its slot L (row 8b + L/8,
  // physical chunk L%8, logical chunk (L%8) ^ (row/2 mod 8)).
  const int K = p.K;
  const T* asrc[A_DMA];
  const T* bsrc[B_DMA];
  int a_chunk[A_DMA], b_chunk[B_DMA];
  {
    const T* Ab = (const T*)p.A + (long long)(t.g / p.a_gdiv) * p.a_gs;
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
      const int row = 8 * (wave + i * TL::NW) + (lane >> 3);
      const int m = min(t.m0 + row, t.Mg - 1);  // rows past the end re-read the last row
      const long long r = AIDX ? (long long)p.a_rowidx[t.row_base + m] : t.row_base + m;
      a_chunk[i] = ((lane & 7) ^ ((row >> 1) & 7)) * EPC;
      asrc[i] = Ab + r * p.a_rs + a_chunk[i];
    }
    const T* Bb = (const T*)p.W + (long long)(t.g / p.b_gdiv) * p.b_gs;
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
      const int row = 8 * (wave + i * TL::NW) + (lane >> 3);
      const int n = min(t.n0 + row, p.N - 1);
      b_chunk[i] = ((lane & 7) ^ ((row >> 1) & 7)) * EPC;
      bsrc[i] = Bb + (long long)n * K + b_chunk[i];
    }
  }

  auto issue = [&](uint4* st, int kt) {
    const int koff = kt * BK;
    const bool full = koff + BK <= K;
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
      const void* src = (full || koff + a_chunk[i] < K) ? (const void*)(asrc[i] + koff) : (const void*)&g_zero_chunk;
      __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)(st + (wave + i * TL::NW) * 64), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
      const void* src = (full || koff + b_chunk[i] < K) ? (const void*)(bsrc[i] + koff) : (const void*)&g_zero_chunk;
      __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)(st + BM * kCpr + (wave + i * TL::NW) * 64),
                                       16, 0, 0);
    }
  };

  const int wm = wave / NWN, wn = wave % NWN;
  const int lr = lane & 31, lh = lane >> 5;
  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](const uint4* st) {
    const uint4* As = st;
    const uint4* Bs = st + BM * kCpr;
#pragma unroll
    for (int kk = 0; kk < kCpr / 2; ++kk) {
      uint4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = As[swz(wm * FM * 32 + i * 32 + lr, kk * 2 + lh)];
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = Bs[swz(wn * FN * 32 + j * 32 + lr, kk * 2 + lh)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mma<T>::run(acc[i][j], bfr[j], af[i]);
    }
  };

  // two stages, the k loop unrolled by 2 so each half names its stage
  const int nk = (K + BK - 1) / BK;
  issue(lds0, 0);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    __syncthreads();  // stage 0 landed (each wave waits for its DMA before the barrier); stage 1 free
    issue(lds1, kt + 1);
    compute(lds0);
    __syncthreads();  // stage 1 landed; stage 0 free
    if (kt + 2 < nk) issue(lds0, kt + 2);
    compute(lds1);
  }
  if (kt < nk) {
    __syncthreads();
    compute(lds0);
  }
  store_direct<T, FM, FN, EPI>(p, t, acc, wm, wn, lr, lh);
}

// Epilogue of the ring kernels.  bf16 output is staged through LDS (orow(ml)
// = the LDS row that holds output row ml, BN*2 bytes, 16-byte chunks
// XOR-swizzled by row) so every global store writes whole row segments; fp32
// output goes straight from the accumulators.  Every DMA has landed and every
// wave is past its last operand read when this runs.
template <int NWM, int NWN, int FM, int FN, int EPI, typename ORow>
__device__ __forceinline__ void ring_epilogue(const KParams& p, const TileId& t, const floatx16 (&acc)[FM][FN],
                                              int wave, int lane, ORow orow) {
  constexpr int BM = NWM * FM * 32, BN = NWN * FN * 32, NT = NWM * NWN * kWave;
  typedef typename OutType<EPI, bf16>::type TO;
  const int wm = wave / NWN, wn = wave % NWN;
  const int lr = lane & 31, lh = lane >> 5;
  const int tid = threadIdx.x;
  if constexpr (EPI == kEpiBiasGelu || EPI == kEpiBias) {
    constexpr int OCH = BN / 8;  // 16-byte chunks per output row
    __syncthreads();             // every wave is done reading operand slots
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * FN * 32 + j * 32 + 8 * q + 4 * lh;
        float4 bias = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.bias && t.n0 + nl < p.N)
          bias = *reinterpret_cast<const float4*>(p.bias + (long long)t.g * p.bias_gs + t.n0 + nl);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int ml = wm * FM * 32 + i * 32 + lr;
          float v[4] = {acc[i][j][4 * q + 0] + bias.x, acc[i][j][4 * q + 1] + bias.y, acc[i][j][4 * q + 2] + bias.z,
                        acc[i][j][4 * q + 3] + bias.w};
          epi4<EPI, bf16>(p, t, 0, 0, 1.f, v);
          const int phys = (nl >> 3) ^ (ml & (OCH - 1));
          store_from_f32<bf16, 4>(reinterpret_cast<bf16*>(orow(ml) + phys * 16 + (nl & 7) * 2), v);
        }
      }
    }
    __syncthreads();
    constexpr int RPP = NT / OCH;  // output rows per pass
#pragma unroll 4
    for (int pass = 0; pass < BM / RPP; ++pass) {
      const int ml = pass * RPP + tid / OCH;
      const int c = tid % OCH;
      const uint4 val = *reinterpret_cast<const uint4*>(orow(ml) + ((c ^ (ml & (OCH - 1))) * 16));
      const int m = t.m0 + ml;
      if (m < t.Mg && t.n0 + c * 8 < p.N)
        *reinterpret_cast<uint4*>((TO*)p.C + (t.row_base + m) * p.c_rs + (long long)t.g * p.c_gs + t.n0 + c * 8) = val;
    }
  } else if constexpr (EPI == kEpiGeluBwd) {
    static_assert(BM == 256 && BN == 256, "GELU backward epilogue: 256 x 256 tiles");
    constexpr int OCH = BN / 8;    // 16-byte chunks per output row
    constexpr int RPP = NT / OCH;  // rows per pass (16)
    const bf16* U = (const bf16*)p.aux + (long long)t.g * p.aux_gs;
    __syncthreads();  // every wave is done reading operand slots
    // the tile's pre-activations into the LDS rows (whole row segments),
    // every load of a thread in flight at once: rows and columns past the
    // end re-read the last ones (their results are neither stored nor summed)
    {
      const int c = tid % OCH;
      const int n = min(t.n0 + c * 8, p.N - 8);
      uint4 u[BM / RPP];
#pragma unroll
      for (int pass = 0; pass < BM / RPP; ++pass) {
        const int m = min(t.m0 + pass * RPP + tid / OCH, t.Mg - 1);
        u[pass] = *reinterpret_cast<const uint4*>(U + (t.row_base + m) * p.aux_rs + n);
      }
#pragma unroll
      for (int pass = 0; pass < BM / RPP; ++pass) {
        const int ml = pass * RPP + tid / OCH;
        *reinterpret_cast<uint4*>(orow(ml) + ((c ^ (ml & (OCH - 1))) * 16)) = u[pass];
      }
    }
    __syncthreads();
    // in place: C = acc * GELU'(U), rounded to bf16
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = wn * FN * 32 + j * 32 + 8 * q + 4 * lh;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int ml = wm * FM * 32 + i * 32 + lr;
          const int phys = (nl >> 3) ^ (ml & (OCH - 1));
          bf16* cell = reinterpret_cast<bf16*>(orow(ml) + phys * 16 + (nl & 7) * 2);
          float u[4], v[4];
          load_f32<bf16, 4>(cell, u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float gu, dgu;
            gelu_and_grad(u[e], gu, dgu);
            v[e] = acc[i][j][4 * q + e] * dgu;
          }
          store_from_f32<bf16, 4>(cell, v);
        }
      }
    }
    __syncthreads();
    // whole row segments out; each thread also sums its 8 columns over the
    // rows it stores (rows tid / OCH + 16 r of the tile)
    float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int c = tid % OCH;
    const int n = t.n0 + c * 8;
#pragma unroll 4
    for (int pass = 0; pass < BM / RPP; ++pass) {
      const int ml = pass * RPP + tid / OCH;
      const uint4 val = *reinterpret_cast<const uint4*>(orow(ml) + ((c ^ (ml & (OCH - 1))) * 16));
      const int m = t.m0 + ml;
      if (m < t.Mg && n < p.N) {
        *reinterpret_cast<uint4*>((bf16*)p.C + (t.row_base + m) * p.c_rs + (long long)t.g * p.c_gs + n) = val;
        float f[8];
        load_f32<bf16, 8>(reinterpret_cast<const bf16*>(&val), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] += f[e];
      }
    }
    if (n < p.N) {
      float* dst = p.colsum + ((long long)(t.g * p.tiles_m + t.m0 / BM) * RPP + tid / OCH) * p.N + n;
      *reinterpret_cast<float4*>(dst) = make_float4(cs[0], cs[1], cs[2], cs[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(cs[4], cs[5], cs[6], cs[7]);
    }
  } else {
    store_direct<bf16, FM, FN, EPI>(p, t, acc, wm, wn, lr, lh);
  }
}

// ===========================================================================
// ring main loop (bf16, K % 64 == 0)

template <int NWM, int NWN, int FM, int FN>
struct Ring {
  static constexpr int NW = NWM * NWN;
  static constexpr int NT = NW * kWave;
  static constexpr int BM = NWM * FM * 32, BN = NWN * FN * 32;
  static constexpr int BK = 64;
  static constexpr int SR = BM > BN ? BM : BN;  // rows per LDS slot
  static constexpr int SLOT = SR * kCpr;        // uint4 per slot
  static constexpr int A_DMA = BM / 8 / NW;     // 1 KB DMA blocks per wave per operand slice
  static constexpr int B_DMA = BN / 8 / NW;
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile rows must split into 1 KB blocks per wave");
  static_assert(A_DMA < 16, "vmcnt field");
};

// W panel stored K-major (WT): the 64 k-rows of a stage hold BN elements
// each, their 16-byte chunks XOR-swizzled by wt_swz(row) (multiples of four
// chunks), so the four 4-row x 16-column blocks a transposed fragment read
// takes from rows k, k + 8 (two lane groups each) fall on disjoint banks.
__device__ __forceinline__ int wt_swz(int r) { return 4 * ((r & 3) | (((r >> 3) & 1) << 2)); }

typedef short short4v __attribute__((ext_vector_type(4)));
// 4 bf16 of one column over 4 rows (ds_read_b64_tr_b16): within each group of
// 16 lanes, lane i receives element i % 4 of the chunks lanes i/4, 4 + i/4,
// 8 + i/4 and 12 + i/4 point at -- with lanes 4e..4e+3 pointing at the four
// 4-element pieces of row e, column i of the 4 x 16 block
__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(const_cast<char*>(p)));
  return __builtin_bit_cast(uint2, r);
}

template <int NWM, int NWN, int FM, int FN, int EPI, bool RAGGED, bool AIDX, bool WT = false, bool AT = false>
__global__ __launch_bounds__(NWM* NWN* kWave) void k_gemm_ring(KParams p) {
  typedef Ring<NWM, NWN, FM, FN> RG;
  static_assert(!WT || (RG::BN == 256 && !RAGGED), "K-major W: 256-column tiles, dense");
  static_assert(!AT || (WT && RG::BM == 256 && !AIDX), "K-major A: with K-major W, 256-row tiles");
  constexpr int BM = RG::BM, BN = RG::BN, BK = RG::BK, NW = RG::NW;
  constexpr int A_DMA = RG::A_DMA, B_DMA = RG::B_DMA;

  __shared__ uint4 r0[RG::SLOT];
  __shared__ uint4 r1[RG::SLOT];
  __shared__ uint4 r2[RG::SLOT];
  __shared__ uint4 r3[RG::SLOT];
  __shared__ uint4 r4[RG::SLOT];
  auto slot = [&](auto ic) -> uint4* {
    constexpr int i = decltype(ic)::value % 5;
    if constexpr (i == 0) return r0;
    else if constexpr (i == 1) return r1;
    else if constexpr (i == 2) return r2;
    else if constexpr (i == 3) return r3;
    else return r4;
  };

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  TileId t;
  if (!tile_id<RAGGED, BM, BN>(p, t)) return;

  const int K = p.K;
  const bf16* Ab = (const bf16*)p.A + (long long)(t.g / p.a_gdiv) * p.a_gs;
  const bf16* Bb = (const bf16*)p.W + (long long)(t.g / p.b_gdiv) * p.b_gs;
  const bf16* asrc[A_DMA];
  const bf16* bsrc[B_DMA];
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) {
    if constexpr (AT) {
      // as the K-major W below: k-row r of the [64][BM] panel, columns past
      // M re-read the row's last chunk
      const int q = (wave + i * NW) * 64 + lane;
      const int r = q / (BM / 8), c = q % (BM / 8);
      const int m = min(t.m0 + ((c ^ wt_swz(r)) * 8), p.M - 8);
      asrc[i] = Ab + (long long)r * p.a_rs + m;
    } else {
      const int row = 8 * (wave + i * NW) + (lane >> 3);
      const int m = min(t.m0 + row, t.Mg - 1);  // rows past the end re-read the last row
      const long long r = AIDX ? (long long)p.a_rowidx[t.row_base + m] : t.row_base + m;
      asrc[i] = Ab + r * p.a_rs + ((lane & 7) ^ ((row >> 1) & 7)) * 8;
    }
  }
#pragma unroll
  for (int i = 0; i < B_DMA; ++i) {
    if constexpr (WT) {
      // 1 KB block (wave + i*NW) of the [64][BN] panel: k-row r, chunk c of
      // the LDS row holds the row's global chunk c ^ wt_swz(r); columns past
      // N re-read the row's last chunk
      const int q = (wave + i * NW) * 64 + lane;
      const int r = q / (BN / 8), c = q % (BN / 8);
      const int n = min(t.n0 + ((c ^ wt_swz(r)) * 8), p.N - 8);
      bsrc[i] = Bb + (long long)r * p.N + n;
    } else {
      const int row = 8 * (wave + i * NW) + (lane >> 3);
      const int n = min(t.n0 + row, p.N - 1);
      bsrc[i] = Bb + (long long)n * K + ((lane & 7) ^ ((row >> 1) & 7)) * 8;
    }
  }
  const int nk_real = K / BK;
  // k-slices past the end re-read the last slice; they land in slots no
  // compute reads again
  auto issueA = [&](uint4* dst, int kt) {
    const long long koff = (long long)min(kt, nk_real - 1) * BK * (AT ? p.a_rs : 1);
#pragma unroll
    for (int i = 0; i < A_DMA; ++i)
      __builtin_amdgcn_global_load_lds((global_cvoid*)(asrc[i] + koff), (lds_void*)(dst + (wave + i * NW) * 64), 16,
                                       0, 0);
  };
  auto issueB = [&](uint4* dst, int kt) {
    const long long koff = (long long)min(kt, nk_real - 1) * BK * (WT ? p.N : 1);
#pragma unroll
    for (int i = 0; i < B_DMA; ++i)
      __builtin_amdgcn_global_load_lds((global_cvoid*)(bsrc[i] + koff), (lds_void*)(dst + (wave + i * NW) * 64), 16,
                                       0, 0);
  };

  const int wm = wave / NWN, wn = wave % NWN;
  const int lr = lane & 31, lh = lane >> 5;
  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragments of k-step kk (16 k) double-buffered in registers
  auto compute = [&](const uint4* As, const uint4* Bs) {
    uint4 af[2][FM], bfr[2][FN];
    // a fragment from a K-major panel of `width` columns: lane group g4 =
    // lane/16 takes k rows 8*(g4/2) .. +7 of this k-step, columns 16*(g4%2)
    // .. +15 of the 32-column block at col0; lane i16 addresses row i16/4 of
    // each 4-row block, columns 4*(i16%4) .. +3
    auto frag_tr = [&](const uint4* S, int width, int col0, int kk) {
      const int g4 = lane >> 4, i16 = lane & 15;
      const int col = col0 + (g4 & 1) * 16 + 4 * (i16 & 3);
      uint2 h[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = kk * 16 + (g4 >> 1) * 8 + hh * 4 + (i16 >> 2);
        h[hh] = lds_read_tr16(reinterpret_cast<const char*>(S) + r * (width * 2) + (((col >> 3) ^ wt_swz(r)) << 4) +
                              (col & 7) * 2);
      }
      return make_uint4(h[0].x, h[0].y, h[1].x, h[1].y);
    };
    auto ld = [&](int kk, int b) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (AT)
          af[b][i] = frag_tr(As, BM, wm * FM * 32 + i * 32, kk);
        else
          af[b][i] = As[swz(wm * FM * 32 + i * 32 + lr, kk * 2 + lh)];
      }
      if constexpr (WT) {
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[b][j] = frag_tr(Bs, BN, wn * FN * 32 + j * 32, kk);
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[b][j] = Bs[swz(wn * FN * 32 + j * 32 + lr, kk * 2 + lh)];
      }
    };
    auto mm = [&](int b) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mma<bf16>::run(acc[i][j], bfr[b][j], af[b][i]);
    };
    ld(0, 0);
    ld(1, 1);
    mm(0);
    ld(2, 0);
    mm(1);
    ld(3, 1);
    mm(0);
    mm(1);
    if constexpr (AT) {
      // keep the double buffering: left alone, the scheduler moves each
      // fragment read next to its first MFMA and waits for it there; pinned
      // as k-step 0's reads, then each k-step's MFMAs with the next k-step's
      // reads spread between them, the reads' latency hides under MFMAs.
      // (With both operands transposed the fragments take few registers; on
      // the other forms the extra live fragments spill.)
      constexpr int NR = 2 * FM + 2 * FN;  // transposed LDS reads per k-step
      constexpr int NM = FM * FN;          // MFMAs per k-step
      static_assert(NM > 1, "the K-major A form has 4 x 2 blocks per wave");
      constexpr int PER = (NR + NM - 2) / (NM - 1);
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (kk < 3 && i < NM - 1) __builtin_amdgcn_sched_group_barrier(0x100, PER, 0);
        }
      }
    }
  };

  // prologue: A_0 -> slot 0, W_0 -> slot 1, A_1 -> slot 2
  issueA(slot(std::integral_constant<int, 0>()), 0);
  issueB(slot(std::integral_constant<int, 1>()), 0);
  issueA(slot(std::integral_constant<int, 2>()), 1);
  auto step = [&](auto ic, int k) {
    constexpr int s5 = decltype(ic)::value;  // k mod 5
    // A_k and W_k landed: the only newer DMA of this wave is A_{k+1}
    wait_vmcnt<A_DMA>();
    __builtin_amdgcn_s_barrier();
    // every wave is past stage k-1: refill its slots with W_{k+1}, A_{k+2}
    issueB(slot(std::integral_constant<int, 2 * s5 + 3>()), k + 1);
    issueA(slot(std::integral_constant<int, 2 * s5 + 4>()), k + 2);
    if (k < nk_real) compute(slot(std::integral_constant<int, 2 * s5>()), slot(std::integral_constant<int, 2 * s5 + 1>()));
  };
  const int nk = (nk_real + 4) / 5 * 5;
  for (int kt = 0; kt < nk; kt += 5) {
    step(std::integral_constant<int, 0>(), kt);
    step(std::integral_constant<int, 1>(), kt + 1);
    step(std::integral_constant<int, 2>(), kt + 2);
    step(std::integral_constant<int, 3>(), kt + 3);
    step(std::integral_constant<int, 4>(), kt + 4);
  }
  wait_vmcnt<0>();  // no DMA may land in LDS after this point

  ring_epilogue<NWM, NWN, FM, FN, EPI>(p, t, acc, wave, lane, [&](int ml) -> char* {
    constexpr int RPS = RG::SLOT * 16 / (BN * 2);  // output rows per slot
    const int s = ml / RPS;
    char* base = s == 0 ? (char*)r0 : s == 1 ? (char*)r1 : s == 2 ? (char*)r2 : (char*)r3;
    return base + (ml - s * RPS) * (BN * 2);
  });
}


// ===========================================================================
// pipelined ring (bf16, K % 64 == 0, dense, 128 x 64 per wave: the 256 x 256
// and 256 x 128 tiles).  Same five slots and slot assignment as k_gemm_ring
// (A_j in slot 2j mod 5, W_j in slot 2j+1 mod 5), scheduled by hand:
//  * a stage is four k-steps of 16.  Each k-step is one asm block: its eight
//    MFMAs, the six fragment reads of the next k-step in the order the next
//    block consumes them (A_0, W_0, W_1, A_1, A_2, A_3) behind the first six
//    MFMAs, and up to four DMA ops behind its last MFMA; the block waits for
//    its own reads at its end, so no LDS load result outlives the statement
//    that issued it.
//  * the stage barrier sits before the last k-step.  By then every wave has
//    read all of stage k's fragments (the last k-step's were read by the
//    third block), so after it stage k's slots take W_{k+2} (first block
//    after the barrier) and the last k-step already reads stage k+1's first
//    fragments.  A_{k+2} goes into the slot of W_{k-1} in the first block(s)
//    of stage k.
//  * DMA and fragment reads are plain asm, invisible to the compiler's wait
//    tracking; the waits are explicit: before barrier k, everything but the
//    A_{k+2} ops (the newest A_DMA) has landed, i.e. A_{k+1} and W_{k+1}.
//  * wave priority falls by one with each k-step block a wave issues after a
//    stage barrier (3, 2, 1, 0).  Left to age order, the older wave of each
//    SIMD issues its MFMAs first, finishes the stage early and waits at the
//    barrier while the younger one runs alone; with the priority the wave
//    that is behind goes first (0.2-1.3 % on the forward products).
// Spread over the stage this way, the eight waves' DMA ops no longer arrive
// in one burst that stalls each wave's MFMA issue behind the vector-memory
// queue, and no fragment read latency is exposed at a stage boundary.

#define RM_DMA(v) "global_load_lds_dwordx4 %[" #v "], %[sb]\n\t"
#define RM_M0NEXT "s_add_u32 m0, m0, %[ms]\n\t"

// the four DMA ops of a k-step: voff v0..v3 against the 64-bit base sb, LDS
// destinations mb, mb + ms, mb + 2ms, mb + 3ms (M0 is written one
// instruction before each DMA that reads it: the s_nop is that wait state)
#define RM_DMA4 \
  RM_DMA(v0) RM_M0NEXT "s_nop 0\n\t" RM_DMA(v1) RM_M0NEXT "s_nop 0\n\t" RM_DMA(v2) RM_M0NEXT "s_nop 0\n\t" RM_DMA(v3)
#define RM_IN_DMA4 \
  [mb] "s"(mb), [sb] "s"(sb), [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]), [v3] "v"(v[3]), [ms] "n"(MS)

// one k-step with four DMA ops, issued behind its eight MFMAs: a DMA op
// whose issue waits for room in the vector-memory queue then holds up no
// MFMA of the block (between the MFMAs it cost 1-2.5 % of a product)
#define RM_KSTEP_DMA                                                                                          \
  "s_mov_b32 m0, %[mb]\n\t" RM_MF(c00, b0, a0) RM_RD(na0, la, 0) RM_MF(c01, b1, a0) RM_RD(nb0, lb, 0)         \
      RM_MF(c10, b0, a1) RM_RD(nb1, lb, 4096) RM_MF(c11, b1, a1) RM_RD(na1, la, 4096) RM_MF(c20, b0, a2)        \
          RM_RD(na2, la, 8192) RM_MF(c21, b1, a2) RM_RD(na3, la, 12288) RM_MF(c30, b0, a3) RM_MF(c31, b1, a3)    \
              RM_DMA4 "s_waitcnt lgkmcnt(0)\n\t"
// a k-step's four DMA ops alone: the share of the slice loads of a wave
// whose rows of the tile are all past the end (it issues no MFMAs)
template <int MS>
__device__ __forceinline__ void dma4(uint32_t mb, const void* sb, const uint32_t* v) {
  asm volatile("s_mov_b32 m0, %[mb]\n\ts_nop 0\n\t" RM_DMA4 "\n\t"
               :
               : RM_IN_DMA4
               : "m0", "scc");
}

template <int MS>
__device__ __forceinline__ void kstep_dma(floatx16 (&acc)[4][2], const Frags& cu, Frags& nx, uint32_t la,
                                          uint32_t lb, uint32_t mb, const void* sb, const uint32_t* v) {
  asm volatile(RM_KSTEP_DMA
               : RM_KSTEP_ACC
               : RM_KSTEP_IN, RM_IN_DMA4
               : "m0", "scc");
}

// ---- K-major operands (the backward products) ----------------------------
// A K-major operand's stage slice is [64 k][256] in LDS (512-byte rows,
// chunks swizzled by wt_swz), and each of its fragments is two transposed
// 64-bit reads (rows +0..3 and +4..7 of the lane group's 8 k-rows, 2048
// bytes apart), whose halves the compiler places side by side as the MFMA
// operand.  WT: W K-major, A as above (four A reads of 16 bytes, four W
// reads of 8 per k-step); KK: both K-major (twelve reads of 8 per k-step,
// two behind each of the first six MFMAs).  Addresses: la (or la0..la3, one
// per A block) and lb0, lb1 (one per W block) for the next k-step.

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
struct FragsWT {
  u32x4 a0, a1, a2, a3;
  u32x2 b0l, b0h, b1l, b1h;
};
struct FragsKK {
  u32x2 a0l, a0h, a1l, a1h, a2l, a2h, a3l, a3h, b0l, b0h, b1l, b1h;
};
__device__ __forceinline__ u32x4 cat2(u32x2 lo, u32x2 hi) { return u32x4{lo.x, lo.y, hi.x, hi.y}; }

// fragment addresses of one k-step: a[0] (N-major A) or a[0..3] (K-major A,
// one per row block), b[0] (N-major W) or b[0..1] (K-major W)
struct PAddr {
  uint32_t a[4];
  uint32_t b[2];
};

// the two halves of a transposed fragment: rows +0..3 at offset o0 (k-step
// KI's 16 rows further down the slice), rows +4..7 at o1 = o0 + 2048
#define RM_TR(dst, addr, h) "ds_read_b64_tr_b16 %[" #dst "], %[" #addr "] offset:%[o" #h "]\n\t"

#define RM_KSTEP_WT_BODY(TAIL)                                                                              \
  RM_MF(c00, b0, a0) RM_RD(na0, la, 0) RM_TR(nb0l, lb0, 0) RM_MF(c01, b1, a0) RM_TR(nb0h, lb0, 1) RM_TR(nb1l, lb1, 0) \
      RM_MF(c10, b0, a1) RM_TR(nb1h, lb1, 1) RM_MF(c11, b1, a1) RM_RD(na1, la, 4096) RM_MF(c20, b0, a2)              \
          RM_RD(na2, la, 8192) RM_MF(c21, b1, a2) RM_RD(na3, la, 12288) RM_MF(c30, b0, a3) RM_MF(c31, b1, a3) TAIL   \
              "s_waitcnt lgkmcnt(0)\n\t"
#define RM_KSTEP_KK_BODY(D0, D1, D2, D3)                                                                       \
  RM_MF(c00, b0, a0) RM_TR(na0l, la0, 0) RM_TR(na0h, la0, 1) D0 RM_MF(c01, b1, a0) RM_TR(nb0l, lb0, 0)         \
      RM_TR(nb0h, lb0, 1) RM_MF(c10, b0, a1) RM_TR(nb1l, lb1, 0) RM_TR(nb1h, lb1, 1) D1 RM_MF(c11, b1, a1)     \
          RM_TR(na1l, la1, 0) RM_TR(na1h, la1, 1) RM_MF(c20, b0, a2) RM_TR(na2l, la2, 0) RM_TR(na2h, la2, 1)  \
              D2 RM_MF(c21, b1, a2) RM_TR(na3l, la3, 0) RM_TR(na3h, la3, 1) RM_MF(c30, b0, a3) D3             \
                  RM_MF(c31, b1, a3) "s_waitcnt lgkmcnt(0)\n\t"
// the KK form keeps its DMA ops between its MFMAs (behind them it measured
// 1-2 % slower, unlike the other forms)
#define RM_D(v) RM_DMA(v) RM_M0NEXT

#define RM_ACC8                                                                                \
  [c00] "+v"(acc[0][0]), [c01] "+v"(acc[0][1]), [c10] "+v"(acc[1][0]), [c11] "+v"(acc[1][1]), \
      [c20] "+v"(acc[2][0]), [c21] "+v"(acc[2][1]), [c30] "+v"(acc[3][0]), [c31] "+v"(acc[3][1])
#define RM_OUT_WT                                                                                      \
  RM_ACC8, [na0] "=&v"(nx.a0), [na1] "=&v"(nx.a1), [na2] "=&v"(nx.a2), [na3] "=&v"(nx.a3),             \
      [nb0l] "=&v"(nx.b0l), [nb0h] "=&v"(nx.b0h), [nb1l] "=&v"(nx.b1l), [nb1h] "=&v"(nx.b1h)
#define RM_OUT_KK                                                                                         \
  RM_ACC8, [na0l] "=&v"(nx.a0l), [na0h] "=&v"(nx.a0h), [na1l] "=&v"(nx.a1l), [na1h] "=&v"(nx.a1h),         \
      [na2l] "=&v"(nx.a2l), [na2h] "=&v"(nx.a2h), [na3l] "=&v"(nx.a3l), [na3h] "=&v"(nx.a3h),             \
      [nb0l] "=&v"(nx.b0l), [nb0h] "=&v"(nx.b0h), [nb1l] "=&v"(nx.b1l), [nb1h] "=&v"(nx.b1h)
#define RM_IN_FR [a0] "v"(a0), [a1] "v"(a1), [a2] "v"(a2), [a3] "v"(a3), [b0] "v"(b0), [b1] "v"(b1)
#define RM_IN_OFF [o0] "n"(KI * 8192), [o1] "n"(KI * 8192 + 2048)
#define RM_IN_WT_ADDR [la] "v"(ad.a[0]), [lb0] "v"(ad.b[0]), [lb1] "v"(ad.b[1])
#define RM_IN_KK_ADDR \
  [la0] "v"(ad.a[0]), [la1] "v"(ad.a[1]), [la2] "v"(ad.a[2]), [la3] "v"(ad.a[3]), [lb0] "v"(ad.b[0]), [lb1] "v"(ad.b[1])

// k-step KI (0..3) of a stage; K-major addresses are the stage's, N-major
// ones already the k-step's
template <int KI>
__device__ __forceinline__ void kstep(floatx16 (&acc)[4][2], const FragsWT& cu, FragsWT& nx, const PAddr& ad) {
  const u32x4 a0 = cu.a0, a1 = cu.a1, a2 = cu.a2, a3 = cu.a3, b0 = cat2(cu.b0l, cu.b0h), b1 = cat2(cu.b1l, cu.b1h);
  asm volatile(RM_KSTEP_WT_BODY("") : RM_OUT_WT : RM_IN_FR, RM_IN_WT_ADDR, RM_IN_OFF);
}
template <int MS, int KI>
__device__ __forceinline__ void kstep_dma(floatx16 (&acc)[4][2], const FragsWT& cu, FragsWT& nx, const PAddr& ad,
                                          uint32_t mb, const void* sb, const uint32_t* v) {
  const u32x4 a0 = cu.a0, a1 = cu.a1, a2 = cu.a2, a3 = cu.a3, b0 = cat2(cu.b0l, cu.b0h), b1 = cat2(cu.b1l, cu.b1h);
  asm volatile("s_mov_b32 m0, %[mb]\n\t" RM_KSTEP_WT_BODY(RM_DMA4)
               : RM_OUT_WT
               : RM_IN_FR, RM_IN_WT_ADDR, RM_IN_OFF, RM_IN_DMA4
               : "m0", "scc");
}
__device__ __forceinline__ void read_frags(FragsWT& nx, const PAddr& ad) {
  constexpr int KI = 0;
  asm volatile(RM_RD(na0, la, 0) RM_TR(nb0l, lb0, 0) RM_TR(nb0h, lb0, 1) RM_TR(nb1l, lb1, 0) RM_TR(nb1h, lb1, 1)
                   RM_RD(na1, la, 4096) RM_RD(na2, la, 8192) RM_RD(na3, la, 12288) "s_waitcnt lgkmcnt(0)\n\t"
               : [na0] "=&v"(nx.a0), [na1] "=&v"(nx.a1), [na2] "=&v"(nx.a2), [na3] "=&v"(nx.a3),
                 [nb0l] "=&v"(nx.b0l), [nb0h] "=&v"(nx.b0h), [nb1l] "=&v"(nx.b1l), [nb1h] "=&v"(nx.b1h)
               : RM_IN_WT_ADDR, RM_IN_OFF);
}

template <int KI>
__device__ __forceinline__ void kstep(floatx16 (&acc)[4][2], const FragsKK& cu, FragsKK& nx, const PAddr& ad) {
  const u32x4 a0 = cat2(cu.a0l, cu.a0h), a1 = cat2(cu.a1l, cu.a1h), a2 = cat2(cu.a2l, cu.a2h),
              a3 = cat2(cu.a3l, cu.a3h), b0 = cat2(cu.b0l, cu.b0h), b1 = cat2(cu.b1l, cu.b1h);
  asm volatile(RM_KSTEP_KK_BODY("", "", "", "") : RM_OUT_KK : RM_IN_FR, RM_IN_KK_ADDR, RM_IN_OFF);
}
template <int MS, int KI>
__device__ __forceinline__ void kstep_dma(floatx16 (&acc)[4][2], const FragsKK& cu, FragsKK& nx, const PAddr& ad,
                                          uint32_t mb, const void* sb, const uint32_t* v) {
  const u32x4 a0 = cat2(cu.a0l, cu.a0h), a1 = cat2(cu.a1l, cu.a1h), a2 = cat2(cu.a2l, cu.a2h),
              a3 = cat2(cu.a3l, cu.a3h), b0 = cat2(cu.b0l, cu.b0h), b1 = cat2(cu.b1l, cu.b1h);
  asm volatile("s_mov_b32 m0, %[mb]\n\t" RM_KSTEP_KK_BODY(RM_D(v0), RM_D(v1), RM_D(v2), RM_DMA(v3))
               : RM_OUT_KK
               : RM_IN_FR, RM_IN_KK_ADDR, RM_IN_OFF, RM_IN_DMA4
               : "m0", "scc");
}
__device__ __forceinline__ void read_frags(FragsKK& nx, const PAddr& ad) {
  constexpr int KI = 0;
  asm volatile(RM_TR(na0l, la0, 0) RM_TR(na0h, la0, 1) RM_TR(nb0l, lb0, 0) RM_TR(nb0h, lb0, 1) RM_TR(nb1l, lb1, 0)
                   RM_TR(nb1h, lb1, 1) RM_TR(na1l, la1, 0) RM_TR(na1h, la1, 1) RM_TR(na2l, la2, 0)
                       RM_TR(na2h, la2, 1) RM_TR(na3l, la3, 0) RM_TR(na3h, la3, 1) "s_waitcnt lgkmcnt(0)\n\t"
               : [na0l] "=&v"(nx.a0l), [na0h] "=&v"(nx.a0h), [na1l] "=&v"(nx.a1l), [na1h] "=&v"(nx.a1h),
                 [na2l] "=&v"(nx.a2l), [na2h] "=&v"(nx.a2h), [na3l] "=&v"(nx.a3l), [na3h] "=&v"(nx.a3h),
                 [nb0l] "=&v"(nx.b0l), [nb0h] "=&v"(nx.b0h), [nb1l] "=&v"(nx.b1l), [nb1h] "=&v"(nx.b1h)
               : RM_IN_KK_ADDR, RM_IN_OFF);
}

// the N-major form through the same interface
template <int KI>
__device__ __forceinline__ void kstep(floatx16 (&acc)[4][2], const Frags& cu, Frags& nx, const PAddr& ad) {
  kstep(acc, cu, nx, ad.a[0], ad.b[0]);
}
template <int MS, int KI>
__device__ __forceinline__ void kstep_dma(floatx16 (&acc)[4][2], const Frags& cu, Frags& nx, const PAddr& ad,
                                          uint32_t mb, const void* sb, const uint32_t* v) {
  kstep_dma<MS>(acc, cu, nx, ad.a[0], ad.b[0], mb, sb, v);
}
__device__ __forceinline__ void read_frags(Frags& nx, const PAddr& ad) { read_frags(nx, ad.a[0], ad.b[0]); }

// Start value of the pipelined kernel's accumulators: the bias of each
// accumulator's column (zero without bias), so the epilogue adds nothing.
// Register 4q+e of block (i, j) holds column wn*FN*32 + j*32 + 8q + 4lh + e
// for every i; each block gets its own load (volatile: no shared load plus
// register copies), 4 * FN 16-byte loads per row block and lane.
template <int NWN, int FN, int EPI>
__device__ __forceinline__ void pipe_acc_bias(const KParams& p, const TileId& t, floatx16 (&acc)[4][FN], int wave,
                                              int lane) {
  constexpr int BN = NWN * FN * 32;
  const int wn = wave % NWN, lh = lane >> 5;
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = wn * FN * 32 + j * 32 + 8 * q + 4 * lh;
      int n = t.n0 + nl;
      bool ok = n < p.N;
      if constexpr (EPI == kEpiSwiglu) {  // the tile's column -> gate / up row, as the W operand
        const int hs = p.N / 2, h = t.n0 / 2 + (nl & (BN / 2 - 1));
        n = nl < BN / 2 ? h : hs + h;
        ok = h < hs;
      }
      // columns past N and products without bias read the zero block
      const volatile float4* src = reinterpret_cast<const volatile float4*>(
          p.bias && ok ? (const void*)(p.bias + (long long)t.g * p.bias_gs + n) : (const void*)&g_zero_chunk);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 b;
        b.x = src->x; b.y = src->y; b.z = src->z; b.w = src->w;
        acc[i][j][4 * q + 0] = b.x;
        acc[i][j][4 * q + 1] = b.y;
        acc[i][j][4 * q + 2] = b.z;
        acc[i][j][4 * q + 3] = b.w;
      }
    }
}

// bf16 epilogue of the persistent pipelined ring, in two halves through
// slots 3 and 4 (the next tile's first slices are already landing in slots
// 0-2): half h holds accumulator rows i = 2h, 2h+1 of every wave, i.e. tile
// rows wm*128 + 64h .. +63, at staging row wm*64 + (i-2h)*32 + lr.
template <int NWM, int NWN, int FN, int EPI, typename Init>
__device__ __forceinline__ void pipe_epilogue_bf16(const KParams& p, const TileId& t, const floatx16 (&acc)[4][FN],
                                                   int wave, int lane, char* stage, Init& init_next) {
  constexpr int BN = NWN * FN * 32, NT = NWM * NWN * kWave;
  constexpr int OCH = BN / 8;       // 16-byte chunks per output row
  constexpr int RPP = NT / OCH;     // staging rows per store pass
  constexpr int SROWS = NWM * 64;   // staging rows per half
  const int wm = wave / NWN, wn = wave % NWN;
  const int lr = lane & 31, lh = lane >> 5;
  const int tid = threadIdx.x;
  // kEpiBiasScale: the gate of each accumulator row block's row (rows past
  // the group's end read its last row and are never stored)
  float scale[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (EPI == kEpiBiasScale) {
#pragma unroll
    for (int i = 0; i < 4; ++i) scale[i] = p.rowscale[t.row_base + min(t.m0 + wm * 128 + i * 32 + lr, t.Mg - 1)];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * h + ii;
      const int sr = wm * 64 + ii * 32 + lr;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * FN * 32 + j * 32 + 8 * q + 4 * lh;
          float v[4] = {acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          epi4<EPI, bf16>(p, t, 0, 0, scale[i], v);
          const int phys = (nl >> 3) ^ (sr & (OCH - 1));
          store_from_f32<bf16, 4>(reinterpret_cast<bf16*>(stage + sr * (BN * 2) + phys * 16 + (nl & 7) * 2), v);
        }
    }
    if (h == 1) init_next();  // the accumulators are read for the last time above
    __syncthreads();
    if constexpr (EPI == kEpiSwiglu) {
      // output chunk c of a row: SiLU(gate chunk c) * (up chunk c + OCH/2), the
      // row half the tile wide, so a pass covers twice the rows
#pragma unroll
      for (int pass = 0; pass < SROWS / (2 * RPP); ++pass) {
        const int sr = pass * 2 * RPP + tid / (OCH / 2);
        const int c = tid % (OCH / 2);
        const int m = t.m0 + (sr / 64) * 128 + h * 64 + (sr % 64);
        const int hcol = t.n0 / 2 + c * 8;
        float g[8], u[8];
        load_f32<bf16, 8>(reinterpret_cast<const bf16*>(stage + sr * (BN * 2) + ((c ^ (sr & (OCH - 1))) * 16)), g);
        load_f32<bf16, 8>(
            reinterpret_cast<const bf16*>(stage + sr * (BN * 2) + (((c + OCH / 2) ^ (sr & (OCH - 1))) * 16)), u);
#pragma unroll
        for (int e = 0; e < 8; ++e) g[e] = g[e] / (1.0f + __expf(-g[e])) * u[e];
        if (m < t.Mg && hcol < p.N / 2)
          store_from_f32<bf16, 8>((bf16*)p.C + (t.row_base + m) * p.c_rs + (long long)t.g * p.c_gs + hcol, g);
      }
    } else {
#pragma unroll
      for (int pass = 0; pass < SROWS / RPP; ++pass) {
        const int sr = pass * RPP + tid / OCH;
        const int c = tid % OCH;
        const int m = t.m0 + (sr / 64) * 128 + h * 64 + (sr % 64);
        const uint4 val = *reinterpret_cast<const uint4*>(stage + sr * (BN * 2) + ((c ^ (sr & (OCH - 1))) * 16));
        if (m < t.Mg && t.n0 + c * 8 < p.N) {
          const long long off = (t.row_base + m) * p.c_rs + (long long)t.g * p.c_gs + t.n0 + c * 8;
          *reinterpret_cast<uint4*>((bf16*)p.C + off) = val;
          if constexpr (EPI == kEpiBiasGeluDual) {
            // GELU of the stored (rounded) pre-activation, as a separate pass would
            float u[8];
            load_f32<bf16, 8>(reinterpret_cast<const bf16*>(&val), u);
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = gelu_erf(u[e]);
            store_from_f32<bf16, 8>((bf16*)p.C2 + off, u);
          }
        }
      }
    }
    __syncthreads();  // staging is free again
  }
}

// GELU-backward epilogue of the persistent pipelined ring (256 x 256 tiles):
// C = acc * GELU'(U), rounded to bf16, in the halves of the bf16 epilogue.
// Per half: the half's 128 rows of U into the staging slots (whole row
// segments, every load of a thread in flight at once; rows and columns past
// the end re-read the last ones, their results neither stored nor summed),
// C computed in place, then stored.  Each thread also sums its 8 columns over
// the rows it stores -- the tile rows congruent to tid / 32 mod 16 -- into
// colsum[(g * tiles_m + m0 / 256) * 16 + tid / 32][N].
template <int NWM, int NWN, int FN, typename Init>
__device__ __forceinline__ void pipe_epilogue_gelubwd(const KParams& p, const TileId& t,
                                                      const floatx16 (&acc)[4][FN], int wave, int lane, char* stage,
                                                      Init& init_next) {
  constexpr int BN = NWN * FN * 32, NT = NWM * NWN * kWave;
  constexpr int OCH = BN / 8;      // 16-byte chunks per output row
  constexpr int RPP = NT / OCH;    // staging rows per store pass (16)
  constexpr int SROWS = NWM * 64;  // staging rows per half
  static_assert(NWM * 128 == 256 && BN == 256 && RPP == 16, "GELU backward epilogue: 256 x 256 tiles");
  const int wm = wave / NWN, wn = wave % NWN;
  const int lr = lane & 31, lh = lane >> 5;
  const int tid = threadIdx.x;
  const bf16* U = (const bf16*)p.aux + (long long)t.g * p.aux_gs;
  const int c = tid % OCH;
  const int n = t.n0 + c * 8;
  float cs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // staging row sr of half h holds tile row (sr / 64) * 128 + 64 h + sr % 64
  auto tile_row = [&](int sr, int h) { return (sr / 64) * 128 + h * 64 + (sr % 64); };
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    {
      const int nu = min(n, p.N - 8);
      uint4 u[SROWS / RPP];
#pragma unroll
      for (int pass = 0; pass < SROWS / RPP; ++pass) {
        const int m = min(t.m0 + tile_row(pass * RPP + tid / OCH, h), t.Mg - 1);
        u[pass] = *reinterpret_cast<const uint4*>(U + (t.row_base + m) * p.aux_rs + nu);
      }
#pragma unroll
      for (int pass = 0; pass < SROWS / RPP; ++pass) {
        const int sr = pass * RPP + tid / OCH;
        *reinterpret_cast<uint4*>(stage + sr * (BN * 2) + ((c ^ (sr & (OCH - 1))) * 16)) = u[pass];
      }
    }
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * h + ii;
      const int sr = wm * 64 + ii * 32 + lr;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nl = wn * FN * 32 + j * 32 + 8 * q + 4 * lh;
          const int phys = (nl >> 3) ^ (sr & (OCH - 1));
          bf16* cell = reinterpret_cast<bf16*>(stage + sr * (BN * 2) + phys * 16 + (nl & 7) * 2);
          float u[4], v[4];
          load_f32<bf16, 4>(cell, u);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float gu, dgu;
            gelu_and_grad(u[e], gu, dgu);
            v[e] = acc[i][j][4 * q + e] * dgu;
          }
          store_from_f32<bf16, 4>(cell, v);
        }
    }
    if (h == 1) init_next();  // the accumulators are read for the last time above
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < SROWS / RPP; ++pass) {
      const int sr = pass * RPP + tid / OCH;
      const int m = t.m0 + tile_row(sr, h);
      const uint4 val = *reinterpret_cast<const uint4*>(stage + sr * (BN * 2) + ((c ^ (sr & (OCH - 1))) * 16));
      if (m < t.Mg && n < p.N) {
        *reinterpret_cast<uint4*>((bf16*)p.C + (t.row_base + m) * p.c_rs + (long long)t.g * p.c_gs + n) = val;
        float f[8];
        load_f32<bf16, 8>(reinterpret_cast<const bf16*>(&val), f);
#pragma unroll
        for (int e = 0; e < 8; ++e) cs[e] += f[e];
      }
    }
    __syncthreads();  // staging is free again
  }
  if (n < p.N) {
    float* dst = p.colsum + ((long long)(t.g * p.tiles_m + t.m0 / 256) * RPP + tid / OCH) * p.N + n;
    *reinterpret_cast<float4*>(dst) = make_float4(cs[0], cs[1], cs[2], cs[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(cs[4], cs[5], cs[6], cs[7]);
  }
}

// fp32 epilogue of the persistent pipelined ring, in four quarters through
// slots 3 and 4: quarter i holds accumulator row block i of every wave, tile
// rows wm*128 + 32i + lr at staging row wm*32 + lr, BN*4 bytes per row in
// 16-byte chunks XOR-swizzled by (row mod 16); each store writes a whole row.
template <int NWM, int NWN, int FN, int EPI, typename Init>
__device__ __forceinline__ void pipe_epilogue_f32(const KParams& p, const TileId& t, const floatx16 (&acc)[4][FN],
                                                  int wave, int lane, char* stage, Init& init_next) {
  constexpr int FM = 4, BN = NWN * FN * 32, NT = NWM * NWN * kWave;
  constexpr int OCH = BN / 4;      // 16-byte chunks per output row
  constexpr int RPP = NT / OCH;    // staging rows per store pass
  constexpr int SROWS = NWM * 32;  // staging rows per quarter
  static_assert(SROWS % RPP == 0, "store passes");
  const int wm = wave / NWN, wn = wave % NWN;
  const int lr = lane & 31, lh = lane >> 5;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int sr = wm * 32 + lr;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cix = (wn * FN * 32 + j * 32 + 8 * q + 4 * lh) >> 2;
        const float4 v = make_float4(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                     acc[i][j][4 * q + 3]);
        *reinterpret_cast<float4*>(stage + sr * (BN * 4) + ((cix ^ (sr & 15)) * 16)) = v;
      }
    if (i == FM - 1) init_next();  // the accumulators are read for the last time above
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < SROWS / RPP; ++pass) {
      const int r = pass * RPP + tid / OCH;
      const int c = tid % OCH;
      const uint4 val = *reinterpret_cast<const uint4*>(stage + r * (BN * 4) + ((c ^ (r & 15)) * 16));
      const int m = t.m0 + (r / 32) * 128 + i * 32 + (r % 32);
      if (m < t.Mg && t.n0 + c * 4 < p.N)
        *reinterpret_cast<uint4*>((float*)p.C + (t.row_base + m) * p.c_rs + (long long)t.g * p.c_gs + t.n0 + c * 4) =
            val;
    }
    __syncthreads();  // staging is free again
  }
}

// Persistent: each workgroup walks tiles v = blockIdx.x, + gridDim.x, ...
// (gridDim.x a multiple of 8, so every tile of a workgroup runs on its XCD,
// and at any time the workgroups of one XCD hold consecutive logical tiles).
// The next tile's A_0, W_0, A_1 are issued before this tile's epilogue, so
// they land while it runs; its W_1 follows once the staging slot is free.
// RAGGED: the tiles are the device-side (group, m0) list times the N tiles,
// group g's rows start at row_off[g]; AIDX: A row m of group g is row
// a_rowidx[row_off[g] + m] of that group's A.
template <int NWM, int NWN, int EPI, bool RAGGED, bool AIDX, bool WT = false, bool AT = false>
__global__ __launch_bounds__(NWM* NWN* kWave) void k_gemm_pipe(KParams p) {
  constexpr int FM = 4, FN = 2;
  typedef Ring<NWM, NWN, FM, FN> RG;
  constexpr int BM = RG::BM, BN = RG::BN, NW = RG::NW;
  constexpr int A_DMA = RG::A_DMA, B_DMA = RG::B_DMA;
  constexpr uint32_t SLOTB = RG::SLOT * 16;  // bytes per slot
  static_assert(B_DMA == 4 && (A_DMA == 4 || A_DMA == 8), "DMA ops come in blocks of four");
  static_assert(!WT || (BM == 256 && BN == 256 && !RAGGED && !AIDX), "K-major operands: 256 x 256 tiles, dense");
  static_assert(!AT || WT, "a K-major A comes with a K-major W");
  typedef typename std::conditional<AT, FragsKK, typename std::conditional<WT, FragsWT, Frags>::type>::type FR;
  static_assert(BM / 2 * BN * 2 <= 2 * (int)SLOTB && BM / 4 * BN * 4 <= 2 * (int)SLOTB,
                "a staged part of the output tile must fit in two slots");

  __shared__ uint4 lds[5 * RG::SLOT];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ntile = RAGGED ? (*p.ntiles) * p.tiles_n : p.G * p.tiles_m * p.tiles_n;
  int v = blockIdx.x;
  if (v >= ntile) return;

  // logical tile of virtual id v: consecutive ids of one XCD walk the M tiles
  // of one N column first (dense; n_fast: the N tiles of one M row) or the N
  // tiles of one (group, m0) (ragged), so concurrently running tiles share
  // operand panels
  auto tile_of = [&](int vv, TileId& t) {
    const int lid = xcd_remap(vv, ntile);
    if constexpr (RAGGED) {
      const int slot_ = lid / p.tiles_n;
      t.n0 = (lid - slot_ * p.tiles_n) * BN;
      t.g = p.tiles[2 * slot_];
      t.m0 = p.tiles[2 * slot_ + 1];
      t.row_base = p.row_off[t.g];
      t.Mg = p.row_off[t.g + 1] - (int)t.row_base;
    } else {
      const int per = p.tiles_m * p.tiles_n;
      t.g = lid / per;
      const int r = lid - t.g * per;
      const int tn = p.n_fast ? r % p.tiles_n : r / p.tiles_m;
      const int tm = p.n_fast ? r / p.tiles_n : r - tn * p.tiles_m;
      t.m0 = tm * BM;
      t.n0 = tn * BN;
      t.row_base = 0;
      t.Mg = p.M;
    }
  };

  const int K = p.K;
  const int nk = K / 64;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto slot = [&](int j) -> uint32_t { return lds0 + (uint32_t)(j % 5) * SLOTB; };
  const uint32_t wof = (uint32_t)wave * 1024;

  // per tile: operand bases and, per DMA op, the 32-bit byte offset of this
  // lane's 16-byte chunk (the host checks that every offset fits)
  const char* Ab;
  const char* Bb;
  uint32_t va[A_DMA], vw[B_DMA];
  auto setup = [&](const TileId& t) {
    Ab = (const char*)p.A + (long long)(t.g / p.a_gdiv) * p.a_gs * 2;
    Bb = (const char*)p.W + (long long)(t.g / p.b_gdiv) * p.b_gs * 2;
    if constexpr (AT) {
      // 1 KB block (wave + i*NW) of the [64][BM] slice: k-row r, LDS chunk c
      // holds the row's chunk c ^ wt_swz(r); columns past M re-read the
      // row's last chunk
#pragma unroll
      for (int i = 0; i < A_DMA; ++i) {
        const int q = (wave + i * NW) * 64 + lane;
        const int r = q / (BM / 8), c = q % (BM / 8);
        const int m = min(t.m0 + ((c ^ wt_swz(r)) * 8), p.M - 8);
        va[i] = (uint32_t)(((long long)r * p.a_rs + m) * 2);
      }
    }
    if constexpr (WT) {
#pragma unroll
      for (int i = 0; i < B_DMA; ++i) {
        const int q = (wave + i * NW) * 64 + lane;
        const int r = q / (BN / 8), c = q % (BN / 8);
        const int n = min(t.n0 + ((c ^ wt_swz(r)) * 8), p.N - 8);
        vw[i] = (uint32_t)(((long long)r * p.N + n) * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < (AT ? 0 : A_DMA); ++i) {
      const int row = 8 * (wave + i * NW) + (lane >> 3);
      const int m = min(t.m0 + row, t.Mg - 1);  // rows past the end re-read the last row
      const long long r = AIDX ? (long long)p.a_rowidx[t.row_base + m] : t.row_base + m;
      va[i] = (uint32_t)((r * p.a_rs + ((lane & 7) ^ ((row >> 1) & 7)) * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < (WT ? 0 : B_DMA); ++i) {
      const int row = 8 * (wave + i * NW) + (lane >> 3);
      int n;
      if constexpr (EPI == kEpiSwiglu) {
        // tile columns [0, BN/2) are gate rows h0 + c, [BN/2, BN) the matching
        // up rows Hs + h0 + c (h0 = n0 / 2), so each gate/up pair is in the tile
        const int hs = p.N / 2;
        const int h = min(t.n0 / 2 + (row & (BN / 2 - 1)), hs - 1);
        n = row < BN / 2 ? h : hs + h;
      } else {
        n = min(t.n0 + row, p.N - 1);
      }
      vw[i] = (uint32_t)(((long long)n * K + ((lane & 7) ^ ((row >> 1) & 7)) * 8) * 2);
    }
  };
  // stage kt's slice: 128 bytes further along each row (N-major) or 64 rows
  // further down (K-major); slices past the end re-read the last one
  const long long a_kst = AT ? 128LL * p.a_rs : 128, w_kst = WT ? 128LL * p.N : 128;
  auto kbase = [&](const char* base, long long kst, int kt) -> const void* {
    return base + (long long)min(kt, nk - 1) * kst;
  };
  auto issue_a = [&](int s, int kt) {
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) dma1(slot(s) + wof + i * NW * 1024, kbase(Ab, a_kst, kt), va[i]);
  };
  auto issue_w = [&](int s, int kt) {
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) dma1(slot(s) + wof + i * NW * 1024, kbase(Bb, w_kst, kt), vw[i]);
  };

  // fragment address of lane for k-step kk.  N-major: row * 128 + swizzled
  // chunk, per kk.  K-major: lane group g4 = lane / 16 takes k-rows
  // 8 * (g4 / 2) .. +7 of the k-step and columns 16 * (g4 % 2) .. +15 of the
  // 32-column block, lane i16 row i16 / 4 of each 4-row half and columns
  // 4 * (i16 % 4) .. +3; the swizzle depends on k-row bits the k-step and
  // half do not change, so they are the offsets kk * 16 rows (+ 4 rows)
  const int wm = wave / NWN, wn = wave % NWN;
  const int lr = lane & 31, lh = lane >> 5;
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t ch = (uint32_t)(((kk * 2 + lh) ^ ((lr >> 1) & 7)) * 16);
    oa[kk] = (uint32_t)(wm * FM * 32 + lr) * 128 + ch;
    ob[kk] = (uint32_t)(wn * FN * 32 + lr) * 128 + ch;
  }
  uint32_t ota[4], otb[2];
  {
    const int g4 = lane >> 4, i16 = lane & 15;
    const int r0 = (g4 >> 1) * 8 + (i16 >> 2), sw = wt_swz(r0);
    const int cl = (g4 & 1) * 16 + 4 * (i16 & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = wm * FM * 32 + i * 32 + cl;
      ota[i] = (uint32_t)(r0 * (BM * 2) + (((col >> 3) ^ sw) << 4) + (col & 7) * 2);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = wn * FN * 32 + j * 32 + cl;
      otb[j] = (uint32_t)(r0 * (BN * 2) + (((col >> 3) ^ sw) << 4) + (col & 7) * 2);
    }
  }
  // a K-major operand's addresses are the stage's (the k-step is an
  // immediate offset of the read), an N-major one's the k-step's
  auto paddr = [&](uint32_t sA, uint32_t sW, int kk) {
    PAddr ad;
#pragma unroll
    for (int i = 0; i < 4; ++i) ad.a[i] = AT ? sA + ota[i] : sA + oa[kk];
#pragma unroll
    for (int j = 0; j < 2; ++j) ad.b[j] = WT ? sW + otb[j] : sW + ob[kk];
    return ad;
  };

  TileId t;
  tile_of(v, t);
  setup(t);
  // first tile's A_0 -> 0, W_0 -> 1, A_1 -> 2
  issue_a(0, 0);
  issue_w(1, 0);
  issue_a(2, 1);

  floatx16 acc[FM][FN];
  pipe_acc_bias<NWN, FN, EPI>(p, t, acc, wave, lane);
  for (;;) {
    // W_1 -> 3; then all but W_1 has landed (A_0, W_0, A_1 and any stores)
    issue_w(3, 1);
    wait_vmcnt<B_DMA>();
    __builtin_amdgcn_s_barrier();
    FR f0, f1;
    // a wave whose 128 rows of the tile all lie past the end of the group
    // (the short last tile of a ragged group) issues its share of the slice
    // loads and takes part in every barrier, but no fragment read or MFMA:
    // its SIMD's matrix core then serves only the other wave
    const bool idle = !WT && t.m0 + (wave / NWN) * (FM * 32) >= t.Mg;
    if (idle) {
      for (int k = 0; k < nk; ++k) {
        const uint32_t sA = slot(2 * k);
        const uint32_t dA = slot(2 * k + 4) + wof;
        dma4<NW * 1024>(dA, kbase(Ab, a_kst, k + 2), va);
        if constexpr (A_DMA == 8) dma4<NW * 1024>(dA + 4 * NW * 1024, kbase(Ab, a_kst, k + 2), va + 4);
        wait_vmcnt<A_DMA>();
        __builtin_amdgcn_s_barrier();
        dma4<NW * 1024>(sA + wof, kbase(Bb, w_kst, k + 2), vw);
      }
    } else {
    read_frags(f0, paddr(slot(0), slot(1), 0));

    for (int k = 0; k < nk; ++k) {
      const uint32_t sA = slot(2 * k), sW = slot(2 * k + 1);
      // A_{k+2} into the slot of W_{k-1}
      const uint32_t dA = slot(2 * k + 4) + wof;
      // a wave's priority is 3 minus the k-step blocks it has issued since
      // the last stage barrier: of the two waves of a SIMD, the one behind
      // issues first, so they reach the barrier together
      __builtin_amdgcn_s_setprio(2);
      kstep_dma<NW * 1024, 1>(acc, f0, f1, paddr(sA, sW, 1), dA, kbase(Ab, a_kst, k + 2), va);
      __builtin_amdgcn_s_setprio(1);
      if constexpr (A_DMA == 8)
        kstep_dma<NW * 1024, 2>(acc, f1, f0, paddr(sA, sW, 2), dA + 4 * NW * 1024, kbase(Ab, a_kst, k + 2), va + 4);
      else
        kstep<2>(acc, f1, f0, paddr(sA, sW, 2));
      __builtin_amdgcn_s_setprio(0);
      kstep<3>(acc, f0, f1, paddr(sA, sW, 3));
      // everything but A_{k+2} has landed: A_{k+1} and W_{k+1}
      wait_vmcnt<A_DMA>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_s_setprio(3);
      // stage k's slots are free: W_{k+2} into A_k's; read stage k+1's first fragments
      kstep_dma<NW * 1024, 0>(acc, f1, f0, paddr(slot(2 * k + 2), slot(2 * k + 3), 0), sA + wof,
                           kbase(Bb, w_kst, k + 2), vw);
    }
    }
    __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<0>();  // no DMA may land in LDS after this point
    // the last MFMAs' results are read by ordinary code from here on
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t" ::);
    __syncthreads();  // every wave is past its last operand read

    const TileId cur = t;
    v += gridDim.x;
    const bool more = v < ntile;
    if (more) {
      tile_of(v, t);
      setup(t);
      issue_a(0, 0);
      issue_w(1, 0);
      issue_a(2, 1);
    }
    // the next tile's accumulators start from its bias once this tile's are read
    auto init_next = [&]() {
      if (more) pipe_acc_bias<NWN, FN, EPI>(p, t, acc, wave, lane);
    };
    if constexpr (EPI == kEpiBiasGelu || EPI == kEpiBias || EPI == kEpiSwiglu || EPI == kEpiBiasScale ||
                  EPI == kEpiBiasGeluDual)
      pipe_epilogue_bf16<NWM, NWN, FN, EPI>(p, cur, acc, wave, lane, (char*)lds + 3 * SLOTB, init_next);
    else if constexpr (EPI == kEpiGeluBwd)
      pipe_epilogue_gelubwd<NWM, NWN, FN>(p, cur, acc, wave, lane, (char*)lds + 3 * SLOTB, init_next);
    else
      pipe_epilogue_f32<NWM, NWN, FN, EPI>(p, cur, acc, wave, lane, (char*)lds + 3 * SLOTB, init_next);
    if (!more) break;
  }
}

// ===========================================================================
// host side

struct TileCfg {
  int nwm, nwn, fm, fn;
  int bm() const { return nwm * fm * 32; }
  int bn() const { return nwn * fn * 32; }
};
constexpr TileCfg kCfgs[] = {
    {2, 4, 4, 2},  // 0: 256 x 256, 8 waves of 128 x 64
    {2, 2, 4, 2},  // 1: 256 x 128, 4 waves of 128 x 64
    {2, 2, 2, 2},  // 2: 128 x 128, 4 waves of 64 x 64
    {2, 2, 1, 1},  // 3:  64 x  64, 4 waves of 32 x 32
};
constexpr int kNumCfgs = 4;
constexpr int kMoeCfg = 0;  // ragged expert products: 256 x 256 tiles

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// K-major operands on the pipelined kernel: every DMA offset is 32-bit (the
// N-major A's rows, as for the forward products; a K-major slice spans 64
// rows of its operand)
bool gemm_kmajor_pipe_fits(const GemmArgs& a) {
  const long long lim = 1LL << 32;
  const bool a_fits = a.a_kmajor ? (63LL * a.a_rs + a.M) * 2 < lim : ((long long)(a.M - 1) * a.a_rs + a.K) * 2 < lim;
  return a_fits && (63LL * a.N + a.N) * 2 < lim;
}


int choose_cfg(const GemmArgs& a) {
  if (a.tile_cfg >= 0 && a.tile_cfg < kNumCfgs) return a.tile_cfg;
  if (a.row_off) return kMoeCfg;
  {
    // eight waves on 256 x 256 tiles wherever they fill at least one round of
    // the persistent grid with little padding: a part-filled last round costs
    // less than running every tile on four waves (one per SIMD) of 256 x 128
    // (B = 2048, T = 16, N = 768, K = 3072: 155-158 against 168-169 us)
    const long long tm = ceil_div(a.M, 256), tn = ceil_div(a.N, 256);
    const double eff = (double)a.M * a.N / ((double)tm * 256 * tn * 256);
    if ((long long)a.G * tm * tn >= device_cus() && eff >= 0.8) return 0;
  }
  for (int c = 0; c < kNumCfgs; ++c) {
    const TileCfg& t = kCfgs[c];
    const long long tm = ceil_div(a.M, t.bm()), tn = ceil_div(a.N, t.bn());
    const long long tiles = (long long)a.G * tm * tn;
    const double eff = (double)a.M * a.N / ((double)tm * t.bm() * tn * t.bn());
    if (tiles >= 512 && eff >= 0.8) return c;
  }
  return kNumCfgs - 1;
}

KParams make_params(const GemmArgs& a, int bm, int bn) {
  KParams p;
  p.A = a.A; p.a_gs = a.a_gs; p.a_rs = a.a_rs; p.a_gdiv = a.a_gdiv; p.a_rowidx = a.a_rowidx;
  p.W = a.W; p.b_gs = a.b_gs; p.b_gdiv = a.b_gdiv;
  p.C = a.C; p.c_gs = a.c_gs; p.c_rs = a.c_rs; p.C2 = a.C2;
  p.aux = a.aux; p.colsum = a.colsum;
  p.aux_gs = a.aux_gs >= 0 ? a.aux_gs : a.c_gs;
  p.aux_rs = a.aux_rs >= 0 ? a.aux_rs : a.c_rs;
  p.bias = a.bias; p.bias_gs = a.bias_gs;
  p.rowscale = a.rowscale;
  p.row_off = a.row_off; p.tiles = a.tiles; p.ntiles = a.ntiles;
  p.M = a.M; p.N = a.N; p.K = a.K; p.G = a.G;
  p.tiles_m = ceil_div(a.M, bm);
  p.tiles_n = ceil_div(a.N, bn);
  // tile order: the operand whose panels of one group take less space is the
  // one cycled (kept in L2 across the walk), the other is read once per panel
  const double a_panels = (double)p.tiles_m * bm * a.K, w_panels = (double)p.tiles_n * bn * a.K;
  p.n_fast = !a.row_off && w_panels < a_panels ? 1 : 0;
  return p;
}

template <int NWM, int NWN, int FM, int FN, int EPI, bool RAGGED, bool AIDX>
void launch_one(const GemmArgs& a, const KParams& p, dim3 grid, hipStream_t s, bool ring) {
  const dim3 block(NWM * NWN * kWave);
  if (ring)
    hipLaunchKernelGGL((k_gemm_ring<NWM, NWN, FM, FN, EPI, RAGGED, AIDX>), grid, block, 0, s, p);
  else if (a.dt == kBF16)
    hipLaunchKernelGGL((k_gemm_generic<bf16, NWM, NWN, FM, FN, EPI, RAGGED, AIDX>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm_generic<float, NWM, NWN, FM, FN, EPI, RAGGED, AIDX>), grid, block, 0, s, p);
}

template <int NWM, int NWN, int FM, int FN>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = NWM * FM * 32, BN = NWN * FN * 32;
  const KParams p = make_params(a, BM, BN);
  const bool ring = a.dt == kBF16 && a.K % 64 == 0;
  const bool ragged = a.row_off != nullptr;
  const dim3 grid(ragged ? (unsigned)((long long)a.max_mtiles * p.tiles_n)
                         : (unsigned)((long long)a.G * p.tiles_m * p.tiles_n));
  if (grid.x == 0) return hipSuccess;
  if (ragged && !((a.epi == kEpiBiasGelu && a.a_rowidx) || (a.epi == kEpiBiasScale && !a.a_rowidx)))
    return hipErrorInvalidValue;
  if (a.w_kmajor) {
    // W stored [K][N] per group: the compiler-scheduled ring with transposed
    // fragment reads, 256 x 256 tiles only
    if constexpr (FM == 4 && FN == 2 && NWN == 4) {
      if (!ring || ragged) return hipErrorInvalidValue;
      const dim3 block(NWM * NWN * kWave);
      // the backward products (fp32 result, or GELU backward) on the
      // hand-scheduled persistent form, one workgroup per CU; the forward
      // epilogues on a K-major W stay on the ring
      if (a.pipe != 0 && gemm_kmajor_pipe_fits(a) && (a.epi == kEpiBiasF32 || a.epi == kEpiGeluBwd)) {
        const int cus = device_cus();
        const dim3 grid2(grid.x <= (unsigned)cus ? grid.x : (unsigned)(cus / 8 * 8 > 0 ? cus / 8 * 8 : cus));
        if (a.a_kmajor && a.epi == kEpiBiasF32)
          hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiBiasF32, false, false, true, true>), grid2, block, 0, s, p);
        else if (a.a_kmajor)
          return hipErrorInvalidValue;
        else if (a.epi == kEpiBiasF32)
          hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiBiasF32, false, false, true>), grid2, block, 0, s, p);
        else if (a.aux && a.colsum)
          hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiGeluBwd, false, false, true>), grid2, block, 0, s, p);
        else
          return hipErrorInvalidValue;
        return hipGetLastError();
      }
      if (a.a_kmajor) {
        // both operands [K][.]: the weight-gradient products
        if (a.epi != kEpiBiasF32) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_gemm_ring<NWM, NWN, FM, FN, kEpiBiasF32, false, false, true, true>), grid, block, 0, s,
                           p);
        return hipGetLastError();
      }
      switch (a.epi) {
        case kEpiBiasGelu:
          hipLaunchKernelGGL((k_gemm_ring<NWM, NWN, FM, FN, kEpiBiasGelu, false, false, true>), grid, block, 0, s, p);
          break;
        case kEpiBias:
          hipLaunchKernelGGL((k_gemm_ring<NWM, NWN, FM, FN, kEpiBias, false, false, true>), grid, block, 0, s, p);
          break;
        case kEpiBiasF32:
          hipLaunchKernelGGL((k_gemm_ring<NWM, NWN, FM, FN, kEpiBiasF32, false, false, true>), grid, block, 0, s, p);
          break;
        case kEpiGeluBwd:
          if (!a.aux || !a.colsum) return hipErrorInvalidValue;
          hipLaunchKernelGGL((k_gemm_ring<NWM, NWN, FM, FN, kEpiGeluBwd, false, false, true>), grid, block, 0, s, p);
          break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (!ragged && !(a.epi == kEpiBiasGelu || a.epi == kEpiBias || a.epi == kEpiBiasF32 || a.epi == kEpiSwiglu ||
                   (a.epi == kEpiBiasGeluDual && a.C2)))
    return hipErrorInvalidValue;

  if constexpr (FM == 4 && FN == 2) {
    // the pipelined ring addresses operands by 32-bit byte offsets from the
    // group's base: the largest A row index is below M (dense, gathered) or
    // below M * G (ragged compacted rows)
    const long long arows = ragged && !a.a_rowidx ? (long long)a.M * a.G : a.M;
    const bool fits = ((arows - 1) * a.a_rs + a.K) * 2 < (1LL << 32) &&
                      ((long long)(a.N - 1) * a.K + a.K) * 2 < (1LL << 32);
    if (ring && fits && a.pipe != 0) {
      // persistent: one workgroup per CU (the ring takes all of LDS), a
      // multiple of 8 of them so each stays on its XCD
      const int cus = device_cus();
      const dim3 grid2(grid.x <= (unsigned)cus ? grid.x : (unsigned)(cus / 8 * 8 > 0 ? cus / 8 * 8 : cus));
      const dim3 block(NWM * NWN * kWave);
      if (ragged) {
        if (a.a_rowidx)
          hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiBiasGelu, true, true>), grid2, block, 0, s, p);
        else
          hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiBiasScale, true, false>), grid2, block, 0, s, p);
      } else {
        switch (a.epi) {
          case kEpiBiasGelu:
            hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiBiasGelu, false, false>), grid2, block, 0, s, p);
            break;
          case kEpiBias: hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiBias, false, false>), grid2, block, 0, s, p); break;
          case kEpiSwiglu:
            hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiSwiglu, false, false>), grid2, block, 0, s, p);
            break;
          case kEpiBiasGeluDual:
            hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiBiasGeluDual, false, false>), grid2, block, 0, s, p);
            break;
          default: hipLaunchKernelGGL((k_gemm_pipe<NWM, NWN, kEpiBiasF32, false, false>), grid2, block, 0, s, p); break;
        }
      }
      return hipGetLastError();
    }
  }
  if (a.epi == kEpiSwiglu || a.epi == kEpiBiasGeluDual) return hipErrorInvalidValue;  // the pipelined kernel only
  if (ragged) {
    if (a.a_rowidx)
      launch_one<NWM, NWN, FM, FN, kEpiBiasGelu, true, true>(a, p, grid, s, ring);
    else
      launch_one<NWM, NWN, FM, FN, kEpiBiasScale, true, false>(a, p, grid, s, ring);
  } else {
    switch (a.epi) {
      case kEpiBiasGelu: launch_one<NWM, NWN, FM, FN, kEpiBiasGelu, false, false>(a, p, grid, s, ring); break;
      case kEpiBias: launch_one<NWM, NWN, FM, FN, kEpiBias, false, false>(a, p, grid, s, ring); break;
      default: launch_one<NWM, NWN, FM, FN, kEpiBiasF32, false, false>(a, p, grid, s, ring); break;
    }
  }
  return hipGetLastError();
}

}  // namespace

// compute units of the current device (cached per device)
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int gemm_tile_m(const GemmArgs& a) { return kCfgs[choose_cfg(a)].bm(); }

bool gemm_wt_eligible(const GemmArgs& a) {
  if (a.dt != kBF16 || a.K % 64 || a.row_off || a.N % 8 || a.N < 256) return false;
  // the backward's fp32 products (dS) take 256 x 256 tiles whatever their
  // count: the alternative is a transposed copy of the weight
  if (a.epi == kEpiBiasF32 && a.M >= 256) return true;
  GemmArgs b = a;
  b.w_kmajor = 0;
  return choose_cfg(b) == 0;
}

bool gemm_kmajor_eligible(const GemmArgs& a) {
  if (a.dt != kBF16 || a.K % 64 || a.row_off || a.a_rowidx || !a.w_kmajor || a.pipe == 0) return false;
  if (a.M < 256 || a.N < 256 || a.N % 8 || a.b_gs % 8) return false;
  if (a.a_kmajor) return a.epi == kEpiBiasF32 && a.M % 8 == 0 && a.a_rs % 8 == 0 && a.a_rs >= a.M && a.a_gs % 8 == 0;
  const int64_t ags = a.aux_gs >= 0 ? a.aux_gs : a.c_gs, ars = a.aux_rs >= 0 ? a.aux_rs : a.c_rs;
  return a.epi == kEpiGeluBwd && a.c_rs % 8 == 0 && a.c_gs % 8 == 0 && ags % 8 == 0 && ars % 8 == 0;
}

int gemm_colsum_parts(int M) { return ceil_div(M, 256) * 16; }

bool gemm_pipe_eligible(const GemmArgs& a) {
  const TileCfg& t = kCfgs[choose_cfg(a)];
  if (!(t.fm == 4 && t.fn == 2) || a.dt != kBF16 || a.K % 64 || a.pipe == 0) return false;
  const long long arows = a.row_off && !a.a_rowidx ? (long long)a.M * a.G : a.M;
  return ((arows - 1) * a.a_rs + a.K) * 2 < (1LL << 32) && ((long long)(a.N - 1) * a.K + a.K) * 2 < (1LL << 32);
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.a_kmajor || a.epi == kEpiGeluBwd) return gemm_kmajor_eligible(a) ? launch_cfg<2, 4, 4, 2>(a, s) : hipErrorInvalidValue;
  if (a.w_kmajor) return gemm_wt_eligible(a) ? launch_cfg<2, 4, 4, 2>(a, s) : hipErrorInvalidValue;
  if (epilogue_overlap() && gemm_defer_eligible(a)) return launch_gemm_defer(a, s);
  switch (choose_cfg(a)) {
    case 0: return launch_cfg<2, 4, 4, 2>(a, s);
    case 1: return launch_cfg<2, 2, 4, 2>(a, s);
    case 2: return launch_cfg<2, 2, 2, 2>(a, s);
    default: return launch_cfg<2, 2, 1, 1>(a, s);
  }
}

}  // namespace rm

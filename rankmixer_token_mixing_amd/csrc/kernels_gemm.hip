// Grouped MFMA GEMM with fused epilogues: the two products of the per-token
// FFN ("Rankmixer: 硬件效率优化", section "Per-Token FFN": T independent
// FFNs, run as one grouped [T,B,d] x [T,d,h] product as in section 3.2 of
// "重新理解 RankMixer：扩参为什么有效，又为什么划算？") and the ragged
// per-(token, expert) products of the ReLU MoE.
//
// C_g[m][n] = sum_k A_g[m][k] W_g[n][k]: both operands are read along k
// (weights stored [out][in]).  One workgroup computes a BM x BN tile of one
// group; 16-byte chunks of A and W stream global -> registers -> LDS (double
// buffered, XOR-swizzled rows of 8 chunks), and each wave multiplies its
// FM x FN grid of 16x16 fragments with MFMA (bf16: 16x16x32 bf16, fp32:
// 16x16x4 f32), accumulating in fp32.  The MFMA is issued with the weight
// fragment as its first operand, so each lane ends up holding 4 consecutive
// output columns of one row: the epilogue writes 8- or 16-byte vectors.
#include "common.hpp"
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
  void* C;
  long long c_gs, c_rs;
  const float* bias;
  long long bias_gs;
  const void* R;
  long long r_gs, r_rs;
  const float* rowscale;
  const int* row_off;
  const int* tiles;
  const int* ntiles;
  int M, N, K, G, tiles_m, tiles_n;
};

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  // one chunk = 8 bf16 along k; one 16x16x32 MFMA per chunk
  static __device__ __forceinline__ void run(floatx4& c, const uint4& a, const uint4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                0, 0, 0);
  }
};

template <> struct Mma<float> {
  // one chunk = 4 fp32 along k; four 16x16x4 MFMAs (element e of every lane's
  // chunk forms the k-slice of MFMA e, the same slice in both operands)
  static __device__ __forceinline__ void run(floatx4& c, const uint4& a, const uint4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

constexpr int kCpr = 8;  // 16-byte chunks per LDS tile row (128 bytes of k)

// physical chunk slot of (row, chunk): XOR swizzle so that the 16 rows read by
// one quarter-wave and the 2 rows written by 16 lanes hit distinct banks
__device__ __forceinline__ int swz(int row, int c) { return row * kCpr + (c ^ ((row >> 1) & 7)); }

template <typename T, int NWM, int NWN, int FM, int FN, int EPI, bool RAGGED, bool AIDX>
__global__ __launch_bounds__(NWM* NWN* kWave) void k_gemm(KParams p) {
  constexpr int NT = NWM * NWN * kWave;
  constexpr int BM = NWM * FM * 16, BN = NWN * FN * 16;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per chunk
  constexpr int BK = kCpr * EPC;
  constexpr int RPP = NT / kCpr;  // tile rows covered by one pass of the loader
  constexpr int ACH = BM / RPP, BCH = BN / RPP;
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of the loader pass");
  typedef typename std::conditional<EPI == kEpiBiasGelu || EPI == kEpiBias, T, float>::type TO;

  __shared__ uint4 lds[2][(BM + BN) * kCpr];

  const int tid = threadIdx.x;

  // ---- which tile
  int g, m0, n0, Mg;
  long long row_base;
  if constexpr (RAGGED) {
    const int nv = (*p.ntiles) * p.tiles_n;
    if ((int)blockIdx.x >= nv) return;
    const int lid = xcd_remap(blockIdx.x, nv);
    const int slot = lid / p.tiles_n;
    n0 = (lid - slot * p.tiles_n) * BN;
    g = p.tiles[2 * slot];
    m0 = p.tiles[2 * slot + 1];
    row_base = p.row_off[g];
    Mg = p.row_off[g + 1] - (int)row_base;
  } else {
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int per = p.tiles_m * p.tiles_n;
    g = lid / per;
    const int r = lid - g * per;
    const int tn = r / p.tiles_m;
    m0 = (r - tn * p.tiles_m) * BM;
    n0 = tn * BN;
    row_base = 0;
    Mg = p.M;
  }

  // ---- loader: thread owns chunk column kc of rows lrow + i*RPP
  const int kc = tid % kCpr;
  const int lrow = tid / kCpr;
  const T* aptr[ACH];
  const T* bptr[BCH];
  {
    const T* Ab = (const T*)p.A + (long long)(g / p.a_gdiv) * p.a_gs + kc * EPC;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int m = min(m0 + lrow + i * RPP, Mg - 1);  // rows past the end re-read the last row
      const long long r = AIDX ? (long long)p.a_rowidx[row_base + m] : row_base + m;
      aptr[i] = Ab + r * p.a_rs;
    }
    const T* Bb = (const T*)p.W + (long long)g * p.b_gs + kc * EPC;
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int n = min(n0 + lrow + i * RPP, p.N - 1);
      bptr[i] = Bb + (long long)n * p.K;
    }
  }

  uint4 ra[ACH], rb[BCH];
  const int K = p.K;
  auto gload = [&](int kt) {
    const int koff = kt * BK;
    if (koff + BK <= K) {
#pragma unroll
      for (int i = 0; i < ACH; ++i) ra[i] = *reinterpret_cast<const uint4*>(aptr[i] + koff);
#pragma unroll
      for (int i = 0; i < BCH; ++i) rb[i] = *reinterpret_cast<const uint4*>(bptr[i] + koff);
    } else {  // k tail: chunks past K are zero (K is a multiple of the chunk)
      const bool ok = koff + kc * EPC < K;
      const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < ACH; ++i) ra[i] = ok ? *reinterpret_cast<const uint4*>(aptr[i] + koff) : z;
#pragma unroll
      for (int i = 0; i < BCH; ++i) rb[i] = ok ? *reinterpret_cast<const uint4*>(bptr[i] + koff) : z;
    }
  };
  auto sstore = [&](int st) {
    uint4* As = lds[st];
    uint4* Bs = lds[st] + BM * kCpr;
#pragma unroll
    for (int i = 0; i < ACH; ++i) As[swz(lrow + i * RPP, kc)] = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) Bs[swz(lrow + i * RPP, kc)] = rb[i];
  };

  // ---- MFMA
  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / NWN, wn = wave % NWN;
  const int lr = lane & 15, lk = lane >> 4;
  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st) {
    const uint4* As = lds[st];
    const uint4* Bs = lds[st] + BM * kCpr;
#pragma unroll
    for (int sub = 0; sub < kCpr / 4; ++sub) {
      uint4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = As[swz(wm * FM * 16 + i * 16 + lr, sub * 4 + lk)];
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = Bs[swz(wn * FN * 16 + j * 16 + lr, sub * 4 + lk)];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mma<T>::run(acc[i][j], bfr[j], af[i]);
    }
  };

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    compute(kt & 1);
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[m0 + wm*FM*16 + i*16 + lr][n .. n+3] of fragment (i, j)
  float4 bias[FN];
  bool nvalid[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * FN * 16 + j * 16 + lk * 4;
    nvalid[j] = n < p.N;
    bias[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (p.bias && nvalid[j]) bias[j] = *reinterpret_cast<const float4*>(p.bias + (long long)g * p.bias_gs + n);
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * FM * 16 + i * 16 + lr;
    if (m >= Mg) continue;
    const long long orow = (row_base + m) * p.c_rs + (long long)g * p.c_gs;
    float scale = 1.f;
    if constexpr (EPI == kEpiBiasScaleF32) scale = p.rowscale[row_base + m];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if (!nvalid[j]) continue;
      const int n = n0 + wn * FN * 16 + j * 16 + lk * 4;
      float v[4] = {acc[i][j][0] + bias[j].x, acc[i][j][1] + bias[j].y, acc[i][j][2] + bias[j].z,
                    acc[i][j][3] + bias[j].w};
      if constexpr (EPI == kEpiBiasGelu) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu_erf(v[e]);
      }
      if constexpr (EPI == kEpiBiasResidF32) {
        float r[4];
        load_f32<T, 4>((const T*)p.R + (row_base + m) * p.r_rs + (long long)g * p.r_gs + n, r);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += r[e];
      }
      if constexpr (EPI == kEpiBiasScaleF32) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= scale;
      }
      store_from_f32<TO, 4>((TO*)p.C + orow + n, v);
    }
  }
}

struct TileCfg {
  int nwm, nwn, fm, fn;
  int bm() const { return nwm * fm * 16; }
  int bn() const { return nwn * fn * 16; }
  int threads() const { return nwm * nwn * kWave; }
};
constexpr TileCfg kCfgs[] = {
    {2, 4, 8, 4},  // 0: 256 x 256, 8 waves
    {2, 2, 8, 4},  // 1: 256 x 128, 4 waves
    {2, 2, 4, 4},  // 2: 128 x 128, 4 waves
    {2, 2, 2, 2},  // 3:  64 x  64, 4 waves
};
constexpr int kNumCfgs = 4;
constexpr int kMoeCfg = 2;

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

int choose_cfg(const GemmArgs& a) {
  if (a.tile_cfg >= 0 && a.tile_cfg < kNumCfgs) return a.tile_cfg;
  if (a.row_off) return kMoeCfg;
  for (int c = 0; c < kNumCfgs; ++c) {
    const TileCfg& t = kCfgs[c];
    const long long tm = ceil_div(a.M, t.bm()), tn = ceil_div(a.N, t.bn());
    const long long tiles = (long long)a.G * tm * tn;
    const double eff = (double)a.M * a.N / ((double)tm * t.bm() * tn * t.bn());
    if (tiles >= 512 && eff >= 0.8) return c;
  }
  return kNumCfgs - 1;
}

template <typename T, int NWM, int NWN, int FM, int FN>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr int BM = NWM * FM * 16, BN = NWN * FN * 16;
  KParams p;
  p.A = a.A; p.a_gs = a.a_gs; p.a_rs = a.a_rs; p.a_gdiv = a.a_gdiv; p.a_rowidx = a.a_rowidx;
  p.W = a.W; p.b_gs = a.b_gs;
  p.C = a.C; p.c_gs = a.c_gs; p.c_rs = a.c_rs;
  p.bias = a.bias; p.bias_gs = a.bias_gs;
  p.R = a.R; p.r_gs = a.r_gs; p.r_rs = a.r_rs;
  p.rowscale = a.rowscale;
  p.row_off = a.row_off; p.tiles = a.tiles; p.ntiles = a.ntiles;
  p.M = a.M; p.N = a.N; p.K = a.K; p.G = a.G;
  p.tiles_m = ceil_div(a.M, BM);
  p.tiles_n = ceil_div(a.N, BN);
  const dim3 block(NWM * NWN * kWave);
  if (a.row_off) {
    const dim3 grid((unsigned)((long long)a.max_mtiles * p.tiles_n));
    if (grid.x == 0) return hipSuccess;
    if (a.epi == kEpiBiasGelu && a.a_rowidx)
      hipLaunchKernelGGL((k_gemm<T, NWM, NWN, FM, FN, kEpiBiasGelu, true, true>), grid, block, 0, s, p);
    else if (a.epi == kEpiBiasScaleF32 && !a.a_rowidx)
      hipLaunchKernelGGL((k_gemm<T, NWM, NWN, FM, FN, kEpiBiasScaleF32, true, false>), grid, block, 0, s, p);
    else
      return hipErrorInvalidValue;
  } else {
    const dim3 grid((unsigned)((long long)a.G * p.tiles_m * p.tiles_n));
    if (grid.x == 0) return hipSuccess;
    switch (a.epi) {
      case kEpiBiasGelu:
        hipLaunchKernelGGL((k_gemm<T, NWM, NWN, FM, FN, kEpiBiasGelu, false, false>), grid, block, 0, s, p);
        break;
      case kEpiBias:
        hipLaunchKernelGGL((k_gemm<T, NWM, NWN, FM, FN, kEpiBias, false, false>), grid, block, 0, s, p);
        break;
      case kEpiBiasResidF32:
        hipLaunchKernelGGL((k_gemm<T, NWM, NWN, FM, FN, kEpiBiasResidF32, false, false>), grid, block, 0, s, p);
        break;
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const GemmArgs& a, hipStream_t s) {
  switch (choose_cfg(a)) {
    case 0: return launch_cfg<T, 2, 4, 8, 4>(a, s);
    case 1: return launch_cfg<T, 2, 2, 8, 4>(a, s);
    case 2: return launch_cfg<T, 2, 2, 4, 4>(a, s);
    default: return launch_cfg<T, 2, 2, 2, 2>(a, s);
  }
}

}  // namespace

int gemm_tile_m(const GemmArgs& a) { return kCfgs[choose_cfg(a)].bm(); }

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  return a.dt == kBF16 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace rm

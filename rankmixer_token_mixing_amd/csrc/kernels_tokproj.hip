// Projection tokenizer ("特征交叉 —— RankMixer 精读笔记", section
// "特征的Tokenization"): segment t of each sample's concatenated embedding
// through its own linear layer into R^D, fused with the padding and the cast
// of the embedding so that it crosses HBM once.
#include <algorithm>

#include "common.hpp"
#include "frag.hpp"
#include "launch.hpp"

namespace rm {

namespace {

// Element offsets: A row m of segment g at m * a_rs + g * a_gs floats, valid
// while the column (from the row start) is below a_klim; W_g row n at
// g * b_gs + n * K; output row m of group g at m * c_rs + g * c_gs; bias of
// group g at g * bias_gs.
struct AfParams {
  const float* A;
  long long a_gs, a_rs, a_klim;
  const bf16* W;
  long long b_gs;
  bf16* C;
  long long c_gs, c_rs;
  const float* bias;
  long long bias_gs;
  int M, N, K, G, tiles_n, unit_rows;
};

// 16 zero bytes: the source of every weight chunk that lies past K
__device__ __align__(16) uint4 g_zero_chunk = {0, 0, 0, 0};

// fragments of one 16-wide k-step of the projection kernel: the A block and
// the five 32-column weight blocks
struct AfFrags {
  u32x4 a, w0, w1, w2, w3, w4;
};
#define AF_MF(j) "v_mfma_f32_32x32x16_bf16 %[c" #j "], %[w" #j "], %[a], %[c" #j "]\n\t"
#define AF_RD(dst, addr, off) "ds_read_b128 %[" #dst "], %[" #addr "] offset:" #off "\n\t"
#define AF_ACC [c0] "+v"(acc[0]), [c1] "+v"(acc[1]), [c2] "+v"(acc[2]), [c3] "+v"(acc[3]), [c4] "+v"(acc[4])
#define AF_CUR \
  [a] "v"(cu.a), [w0] "v"(cu.w0), [w1] "v"(cu.w1), [w2] "v"(cu.w2), [w3] "v"(cu.w3), [w4] "v"(cu.w4)

// read one k-step's fragments (A block at la, weight block j at lw + 4096 j)
__device__ __forceinline__ void af_read(AfFrags& nx, uint32_t la, uint32_t lw) {
  asm volatile(AF_RD(na, la, 0) AF_RD(nw0, lw, 0) AF_RD(nw1, lw, 4096) AF_RD(nw2, lw, 8192) AF_RD(nw3, lw, 12288)
                   AF_RD(nw4, lw, 16384) "s_waitcnt lgkmcnt(0)\n\t"
               : [na] "=&v"(nx.a), [nw0] "=&v"(nx.w0), [nw1] "=&v"(nx.w1), [nw2] "=&v"(nx.w2), [nw3] "=&v"(nx.w3),
                 [nw4] "=&v"(nx.w4)
               : [la] "v"(la), [lw] "v"(lw)
               : "memory");
}
// five MFMAs on cu while the next k-step's fragments are read into nx
__device__ __forceinline__ void af_kstep(floatx16 (&acc)[5], const AfFrags& cu, AfFrags& nx, uint32_t la,
                                         uint32_t lw) {
  asm volatile(AF_MF(0) AF_RD(na, la, 0) AF_MF(1) AF_RD(nw0, lw, 0) AF_MF(2) AF_RD(nw1, lw, 4096) AF_MF(3)
                   AF_RD(nw2, lw, 8192) AF_MF(4) AF_RD(nw3, lw, 12288) AF_RD(nw4, lw, 16384) "s_waitcnt lgkmcnt(0)\n\t"
               : AF_ACC, [na] "=&v"(nx.a), [nw0] "=&v"(nx.w0), [nw1] "=&v"(nx.w1), [nw2] "=&v"(nx.w2),
                 [nw3] "=&v"(nx.w3), [nw4] "=&v"(nx.w4)
               : AF_CUR, [la] "v"(la), [lw] "v"(lw)
               : "memory");
}
__device__ __forceinline__ void af_klast(floatx16 (&acc)[5], const AfFrags& cu) {
  asm volatile(AF_MF(0) AF_MF(1) AF_MF(2) AF_MF(3) AF_MF(4) : AF_ACC : AF_CUR : "memory");
}

constexpr int kAfBN = 160;   // columns per unit (5 blocks of 32)
constexpr int kAfKmax = 384; // longest resident k (6 slices of 64)
constexpr int kAfWaves = 8;

// A is the fp32 embedding read in place: row m at m * a_rs floats,
// segment g at column g * a_gs, columns at or past a_klim (the embedding's
// length) are the zero padding of the last segment.  The embedding crosses
// HBM once, is rounded to bf16 on chip, and no padded copy is ever written.
//
// The product is short in k (one segment, K <= kAfKmax) and the embedding is
// twice the bytes of everything else, so the kernel is built to stream it:
//  * a unit of work is (segment g, a run of unit_rows rows, an N tile of
//    kAfBN columns); the N tile's weights W_g[n0 .. n0+kAfBN) for all of K and
//    its bias are loaded into LDS once per unit and stay there;
//  * each wave owns 32 rows at a time and walks their k-slices alone: it
//    loads a 32 x 64 fp32 slice with coalesced 16-byte loads (four whole rows
//    per instruction), rounds it to bf16 into its own LDS slot, reads the
//    MFMA fragments back and multiplies them with the resident weights.  No
//    barrier inside a unit: the eight waves drift freely and cover each
//    other's memory latency, and each keeps two slices of loads in flight;
//  * persistent workgroups (one per CU, the resident weights take most of
//    LDS) walk strided runs of units of their XCD's contiguous share; the N
//    tiles of one (segment, rows) unit are neighbours, so they run side by
//    side on one XCD and the second reads the embedding rows from L2.
__global__ __launch_bounds__(kAfWaves* kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_tok_proj(AfParams p) {
  constexpr int FN = kAfBN / 32, BN = kAfBN, BK = 64, NSL = kAfKmax / BK;
  constexpr int kXcd = 8;
  __shared__ uint4 wl[NSL * BN * kCpr];        // resident weights, slice-major, swizzled rows
  __shared__ uint4 al[kAfWaves][32 * kCpr];    // each wave's bf16 k-slice of its 32 rows
  __shared__ float4 lbias[BN / 4];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane & 31, lh = lane >> 5;
  const int K = p.K, nk = (K + BK - 1) / BK;
  const int R = p.unit_rows;  // rows per unit, a multiple of 32 * kAfWaves
  // byte offset of this lane's fragment chunk for k-step kk inside a 32-row
  // block (swizzled: chunk ^ (row/2 mod 8)); block j of the weights is 4 KB on
  const uint32_t inner[4] = {(uint32_t)swz(lr, 0 + lh) * 16, (uint32_t)swz(lr, 2 + lh) * 16,
                             (uint32_t)swz(lr, 4 + lh) * 16, (uint32_t)swz(lr, 6 + lh) * 16};
  const uint32_t la0 = (uint32_t)(uintptr_t)al[wave];
  const uint32_t wl0 = (uint32_t)(uintptr_t)wl;
  const int nch = (p.M + R - 1) / R;
  const int units = p.G * nch * p.tiles_n;
  const int x = blockIdx.x % kXcd, l = blockIdx.x / kXcd, per_x = gridDim.x / kXcd;
  const int lo = (int)((long long)units * x / kXcd), hi = (int)((long long)units * (x + 1) / kXcd);

  floatx16 acc[FN];
  float4 a0[8], a1[8];  // two k-slices in flight: float4 i = row 4i + lane/16, columns 4*(lane%16) .. +3
  int cur_w = -1;       // (g, n tile) whose weights are resident

  for (int u = lo + l; u < hi; u += per_x) {
    const int n_t = u % p.tiles_n;
    const int gc = u / p.tiles_n;
    const int g = gc / nch, c = gc - g * nch;
    const int n0 = n_t * BN;
    const int wkey = g * p.tiles_n + n_t;
    // valid k of this segment: [0, klim), a multiple of 4 (checked on the host)
    const long long kl = p.a_klim - (long long)g * p.a_gs;
    const int klim = kl < K ? (int)kl : K;
    const float* Ab = p.A + (long long)g * p.a_gs;
    // this wave's row blocks in the unit: rows c*R + rb*256 + wave*32 + [0, 32)
    const int rbs = R / (32 * kAfWaves);
    int nblk = 0;
    for (int rb = 0; rb < rbs; ++rb)
      if (c * R + rb * 32 * kAfWaves + wave * 32 < p.M) nblk = rb + 1;
    const int steps = nblk * nk;

    // Loads are unconditional, so the compiler can count them and wait for one
    // slice while the other stays in flight (a skipped load would make it wait
    // for everything): columns past the segment load column 0 of the row and
    // are zeroed when the slice is rounded to bf16, rows past the end re-read
    // the last row (their outputs are not stored).
    auto load = [&](float4 (&a)[8], int st) {
      const int kt = st % nk;
      const int col = kt * BK + 4 * (lane & 15);
      const int m0 = c * R + (st / nk) * 32 * kAfWaves + wave * 32 + (lane >> 4);
      const float* src = Ab + (col < klim ? col : 0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        a[i] = *reinterpret_cast<const float4*>(src + (long long)min(m0 + 4 * i, p.M - 1) * p.a_rs);
    };
    uint2* aw = reinterpret_cast<uint2*>(al[wave]);
    auto step = [&](float4 (&a)[8], int st) {
      // bf16 slice into this wave's slot (its previous reads are complete: their
      // data fed the MFMAs of the previous step)
      // a bit mask, not a branch: a branch here would also make the compiler
      // wait for the other slice's loads
      const unsigned keep = 0u - (unsigned)((st % nk) * BK + 4 * (lane & 15) < klim);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v[4] = {__uint_as_float(__float_as_uint(a[i].x) & keep), __uint_as_float(__float_as_uint(a[i].y) & keep),
                            __uint_as_float(__float_as_uint(a[i].z) & keep), __uint_as_float(__float_as_uint(a[i].w) & keep)};
        const bf16 h[4] = {from_f32<bf16>(v[0]), from_f32<bf16>(v[1]), from_f32<bf16>(v[2]), from_f32<bf16>(v[3])};
        const int c4 = lane & 15;
        aw[2 * swz(4 * i + (lane >> 4), c4 >> 1) + (c4 & 1)] = __builtin_bit_cast(uint2, h);
      }
      // unconditional for the same reason (past the end: the last slice again,
      // never used)
      load(a, min(st + 2, steps - 1));
      const int kt = st % nk;
      // the four 16-wide k-steps of the slice, each one asm block: its five
      // MFMAs run while the next k-step's six fragments are read (left to the
      // compiler, every MFMA waited for its own fragment read)
      const uint32_t lw = wl0 + (uint32_t)(kt * BN * kCpr * 16);
      AfFrags f0, f1;
      af_read(f0, la0 + inner[0], lw + inner[0]);
      af_kstep(acc, f0, f1, la0 + inner[1], lw + inner[1]);
      af_kstep(acc, f1, f0, la0 + inner[2], lw + inner[2]);
      af_kstep(acc, f0, f1, la0 + inner[3], lw + inner[3]);
      af_klast(acc, f1);
      if (kt == nk - 1) {
        // the MFMAs' results are read by ordinary code from here on
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t" ::);
        // epilogue: register 4q+e of block j holds row rowbase + lr, column
        // n0 + j*32 + 8q + 4lh + e; bias from LDS, bf16 out
        const int m = c * R + (st / nk) * 32 * kAfWaves + wave * 32 + lr;
        if (m < p.M) {
          bf16* orow = p.C + (long long)m * p.c_rs + (long long)g * p.c_gs;
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int nl = j * 32 + 8 * q + 4 * lh;
              if (n0 + nl >= p.N) continue;
              const float4 b = lbias[nl >> 2];
              float v[4] = {acc[j][4 * q + 0] + b.x, acc[j][4 * q + 1] + b.y, acc[j][4 * q + 2] + b.z,
                            acc[j][4 * q + 3] + b.w};
              store_from_f32<bf16, 4>(orow + n0 + nl, v);
            }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
      }
    };

    // the first slice of A goes out before the weights are fetched, so the
    // two latencies overlap (for a wave without rows: in-bounds loads, unused)
    load(a0, 0);
    if (wkey != cur_w) {
      __syncthreads();  // every wave is done with the previous weights
      // the weights stream straight into LDS (global_load_lds, no registers):
      // 1 KB block b of slice kt holds rows 8b .. 8b+7, lane L fetching the
      // 16-byte chunk that belongs at its slot (row 8b + L/8, physical chunk
      // L%8 = logical chunk ^ (row/2 mod 8)); chunks past K come from a zero block
      const int nblk_w = nk * (BN / 8);
      const bf16* Wb = p.W + (long long)g * p.b_gs;
      for (int b = wave; b < nblk_w; b += kAfWaves) {
        const int kt = b / (BN / 8), rb8 = b - kt * (BN / 8);
        const int r = 8 * rb8 + (lane >> 3);
        const int lc = (lane & 7) ^ ((r >> 1) & 7);
        const int k = kt * BK + lc * 8;
        const int n = min(n0 + r, p.N - 1);
        const void* src = k < K ? (const void*)(Wb + (long long)n * K + k) : (const void*)&g_zero_chunk;
        __builtin_amdgcn_global_load_lds((global_cvoid*)src, (lds_void*)(wl + kt * BN * kCpr + rb8 * 64), 16, 0, 0);
      }
      const int nb = min(n0 + 4 * (tid % (BN / 4)), p.N - 4);
      const float4 bv = *reinterpret_cast<const float4*>(p.bias + (long long)g * p.bias_gs + nb);
      wait_vmcnt<0>();  // this wave's weight blocks (and the first A slice) landed
      if (tid < BN / 4) lbias[tid] = n0 + 4 * tid < p.N ? bv : make_float4(0.f, 0.f, 0.f, 0.f);
      __syncthreads();
      cur_w = wkey;
    }
    load(a1, max(0, min(1, steps - 1)));
    if (steps == 0) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    int st = 0;
    for (; st + 1 < steps; st += 2) {
      step(a0, st);
      step(a1, st + 1);
    }
    if (st < steps) step(a0, st);
  }
}

}  // namespace

hipError_t launch_tokenize_project(const float* emb, const void* w, const float* bias, void* x0, int64_t B, int64_t F,
                                   int T, int seg, int D, hipStream_t s) {
  // bf16 weights and output, whole float4s of the embedding, the weights of
  // one N tile resident in LDS
  if (B <= 0) return hipSuccess;
  if (!bias || seg % 8 || seg > kAfKmax || F % 4 || D % 8 || F > (int64_t)T * seg || B >= (1LL << 31))
    return hipErrorInvalidValue;
  AfParams p;
  p.A = emb; p.a_gs = seg; p.a_rs = F; p.a_klim = F;
  p.W = (const bf16*)w; p.b_gs = (long long)D * seg;
  p.C = (bf16*)x0; p.c_gs = D; p.c_rs = (long long)T * D;
  p.bias = bias; p.bias_gs = D;
  p.M = (int)B; p.N = D; p.K = seg; p.G = T;
  p.tiles_n = (D + kAfBN - 1) / kAfBN;
  // rows per unit: enough that the units about fill one workgroup per CU
  const int cus = device_cus();
  const long long rows_blk = 32LL * kAfWaves;
  const long long tiles_m = (B + rows_blk - 1) / rows_blk;
  const long long blocks = (long long)T * p.tiles_n * tiles_m;
  const long long rb = std::max(1LL, blocks / std::max(1, cus));
  p.unit_rows = (int)(std::min(rb, tiles_m) * rows_blk);
  const long long units = (long long)T * p.tiles_n * ((B + p.unit_rows - 1) / p.unit_rows);
  if (units >= (1LL << 31)) return hipErrorInvalidValue;
  const long long grid = std::max(8LL, std::min((units + 7) / 8 * 8, (long long)cus / 8 * 8));
  hipLaunchKernelGGL(k_tok_proj, dim3((unsigned)grid), dim3(kAfWaves * kWave), 0, s, p);
  return hipGetLastError();
}

// largest segment the fused kernel keeps resident
int tokenize_project_max_seg() { return kAfKmax; }

}  // namespace rm

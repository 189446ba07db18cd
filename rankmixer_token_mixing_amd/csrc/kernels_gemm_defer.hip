// Grouped GEMM with a deferred epilogue: the per-token FFN products of
// "Rankmixer: 硬件效率优化" (section "Per-Token FFN"), run as one grouped
// [T,B,d] x [T,d,h] product as in section 3.2 of "重新理解 RankMixer：扩参为
// 什么有效，又为什么划算？", C_g[m][n] = sum_k A_g[m][k] W_g[n][k] + bias_g[n]
// with GELU (W1 product), plain (W2 product) or both (training forward).
//
// Why another main loop.  The products' epilogue (bias, GELU, bf16 packing
// and the stores of a 256 x 256 tile) is ALU and store work during which no
// MFMA issues; run after each tile by every wave at once, it also sends every
// compute unit's 128 KB of output to memory in the same few microseconds.
// Here a finished tile is packed to bf16 in registers and its epilogue is
// spread over the next tile's main loop: each k-step carries one "unit" of it
// (four values of one output row: GELU, pack, one 8-byte store) between its
// MFMAs, where the ALU work issues while the matrix cores run, and the stores
// trickle out at the rate the tile computes.  Eight consecutive units complete
// 32 whole 128-byte output lines, so lines are written back whole.  The bias
// joins the accumulators as the tile's main loop ends: one extra MFMA per
// block adds the bf16 high and low parts of each column's bias (within 2^-17
// of it, relative).  Its loads are issued as the tile starts, so by the time
// it is used the previous tile's 64 stores have issued behind them and the
// wait for them never waits for the operand copies in flight.
//
// Measured on MI355X (bench.py --op epilogue_overlap) this kernel is a few
// per cent slower than the ring kernel with the epilogue after each tile: the
// products run power-limited (the clock drops well below its peak under
// them), and moving ALU work under the MFMAs does not lower a tile's energy.
// It runs only when the caller selects it (rm_set_epilogue_overlap).
//
// Layout.  256 x 256 tiles, four waves (one per SIMD), each owning 128 x 128
// as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16 with the 256 fp32 accumulators
// in AGPRs; the previous tile's 16384 outputs per wave wait in 128 VGPRs as
// packed bf16.  Operands stream global -> LDS with global_load_lds_dwordx4
// through a ring of five 32 KB slots (rows of 8 XOR-swizzled 16-byte chunks,
// as in kernels_gemm.hip): k-stage s (64 k) of the workgroup's tile sequence
// reads A_s from slot 2s mod 5 and W_s from slot 2s+1 mod 5, and during stage s
// A_{s+2} and W_{s+2} are fetched -- across tile boundaries, so the next
// tile's first slices land during the current tile's last stages.  Each
// k-step is one asm block (gemm_defer_kstep.inc, written by gemm_defer_gen.py)
// that waits for its own LDS reads at its end; the DMA waits are explicit.
//
// Tiles never hang over the edge: the last tile of a row or column is moved
// back to end at M (N), so rows (columns) it shares with its neighbour are
// computed twice, identically, and stored twice with the same bits.  This
// needs M, N >= 256 and keeps every lane's store unconditional.
#include <atomic>
#include <utility>

#include "common.hpp"
#include "frag.hpp"
#include "launch.hpp"

namespace rm {

namespace {

struct Frag8 {
  u32x4 a0, a1, a2, a3, w0, w1, w2, w3;
};

#include "gemm_defer_kstep.inc"

// the eight fragment reads of one k-step on their own (first k-step)
__device__ __forceinline__ void read_frags8(Frag8& nx, uint32_t la, uint32_t lb) {
  asm volatile(
      "ds_read_b128 %[na0], %[la] offset:0\n\t"
      "ds_read_b128 %[nw0], %[lb] offset:0\n\t"
      "ds_read_b128 %[nw1], %[lb] offset:4096\n\t"
      "ds_read_b128 %[nw2], %[lb] offset:8192\n\t"
      "ds_read_b128 %[nw3], %[lb] offset:12288\n\t"
      "ds_read_b128 %[na1], %[la] offset:4096\n\t"
      "ds_read_b128 %[na2], %[la] offset:8192\n\t"
      "ds_read_b128 %[na3], %[la] offset:12288\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      : [na0] "=&v"(nx.a0), [na1] "=&v"(nx.a1), [na2] "=&v"(nx.a2), [na3] "=&v"(nx.a3), [nw0] "=&v"(nx.w0),
        [nw1] "=&v"(nx.w1), [nw2] "=&v"(nx.w2), [nw3] "=&v"(nx.w3)
      : [la] "v"(la), [lb] "v"(lb));
}

struct DParams {
  const char* A;     // group g's A at A + (g / a_gdiv) * a_gs bytes, row m at m * a_rs bytes
  long long a_gs, a_rs;
  int a_gdiv;
  const char* W;     // group g's W at W + (g / b_gdiv) * b_gs bytes, row n at n * K * 2 bytes
  long long b_gs;
  int b_gdiv;
  char* C;           // output row m of group g at C + g * c_gs + m * c_rs bytes
  char* C2;          // kEpiBiasGeluDual: GELU(C), same layout
  long long c_gs, c_rs;
  const float* bias; // bias of group g at bias + g * bias_gs floats (or null)
  long long bias_gs;
  int M, N, K, G, tiles_m, tiles_n, n_fast;
};

constexpr int kSlot = 32768;  // bytes per ring slot: 256 rows x 128 bytes

// zeros read as the bias of products without one (every block column reads
// element 0, so no bias needs no branch)
__device__ __align__(16) float g_no_bias[4] = {0.f, 0.f, 0.f, 0.f};

constexpr int kUnits = 64;    // epilogue units per wave and tile: 4 x 4 blocks x 4 column quads

struct DTile {
  int g, m0, n0;
};

// the DMA sources of one tile: group bases and this lane's 32-bit offset of
// its 16-byte chunk in rows 8 * wave + lane / 8 (+ 32 i for op i)
struct DDma {
  const char* a;
  const char* w;
  uint32_t va, vw;
};

// the previous tile's store side: output bases and, per row block i, the
// lane's offset of its row and first column
struct DPrev {
  char* c;
  char* c2;
  uint32_t off[4];
};

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2v r;
  r[0] = (bf16)lo;
  r[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// block b (constant after unrolling) of the accumulators, packed
__device__ __forceinline__ void pack_block(int b, uint32_t (&o)[8]) {
  switch (b) {
    case 0: dk_pack_b0(o); break;
    case 1: dk_pack_b1(o); break;
    case 2: dk_pack_b2(o); break;
    case 3: dk_pack_b3(o); break;
    case 4: dk_pack_b4(o); break;
    case 5: dk_pack_b5(o); break;
    case 6: dk_pack_b6(o); break;
    case 7: dk_pack_b7(o); break;
    case 8: dk_pack_b8(o); break;
    case 9: dk_pack_b9(o); break;
    case 10: dk_pack_b10(o); break;
    case 11: dk_pack_b11(o); break;
    case 12: dk_pack_b12(o); break;
    case 13: dk_pack_b13(o); break;
    case 14: dk_pack_b14(o); break;
    default: dk_pack_b15(o); break;
  }
}

// unit u = 16 i + 4 j + q: row block i, block column j, column quad q --
// columns wn*128 + 32 j + 8 q + 4 lh + 0..3 of row wm*128 + 32 i + lr, stored
// at off[i] + 64 j + 16 q bytes.  Units 8 h .. 8 h + 7 (i = h / 2, j = 2 (h % 2)
// and 2 (h % 2) + 1) cover 64 columns = one 128-byte line of each of the 32
// rows, so consecutive units complete whole lines.
__device__ __forceinline__ int unit_i(int u) { return u / 16; }
__device__ __forceinline__ int unit_col_bytes(int u) { return 16 * (u % 16); }

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_defer(DParams p) {
  __shared__ uint4 lds[5 * kSlot / 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lh = lane >> 5;
  const int ntile = p.G * p.tiles_m * p.tiles_n;
  int v = blockIdx.x;
  if (v >= ntile) return;
  const int nk = p.K / 64;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const uint32_t wof = (uint32_t)wave * 1024;

  // fragment addresses for k-step kk: row * 128 + swizzled chunk; block i
  // (j) of the wave is 32 rows = 4096 bytes further (the asm's read offsets)
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t ch = (uint32_t)(((kk * 2 + lh) ^ ((lr >> 1) & 7)) * 16);
    oa[kk] = (uint32_t)(wm * 128 + lr) * 128 + ch;
    ob[kk] = (uint32_t)(wn * 128 + lr) * 128 + ch;
  }
  // DMA op i of a wave fills LDS rows 8 (wave + 4 i) .. + 7 of a slot (1 KB at
  // slot + wave * 1024 + i * 4096): lane L takes row 8 (wave + 4 i) + L / 8,
  // physical chunk L % 8, i.e. the global chunk (L % 8) ^ (row / 2 mod 8),
  // which does not depend on i
  const int drow = 8 * wave + (lane >> 3);
  const uint32_t dch = (uint32_t)(((lane & 7) ^ ((4 * wave + (lane >> 4)) & 7)) * 16);

  auto tile_of = [&](int vv) {
    DTile t;
    const int lid = xcd_remap(vv, ntile);
    const int per = p.tiles_m * p.tiles_n;
    t.g = lid / per;
    const int r = lid - t.g * per;
    const int tn = p.n_fast ? r % p.tiles_n : r / p.tiles_m;
    const int tm = p.n_fast ? r / p.tiles_n : r - tn * p.tiles_m;
    t.m0 = min(tm * 256, p.M - 256);
    t.n0 = min(tn * 256, p.N - 256);
    return t;
  };
  auto dma_of = [&](const DTile& t) {
    DDma d;
    d.a = p.A + (long long)(t.g / p.a_gdiv) * p.a_gs;
    d.w = p.W + (long long)(t.g / p.b_gdiv) * p.b_gs;
    d.va = (uint32_t)((long long)(t.m0 + drow) * p.a_rs) + dch;
    d.vw = (uint32_t)((long long)(t.n0 + drow) * p.K * 2) + dch;
    return d;
  };
  auto slot = [&](int j) -> uint32_t { return lds0 + (uint32_t)(j % 5) * kSlot; };
  // bytes between a wave's consecutive DMA ops (32 rows further)
  const uint32_t a_blk = (uint32_t)(32 * p.a_rs), w_blk = (uint32_t)(32LL * p.K * 2);
  auto asb = [&](const DDma& d, int ks, int i) -> const void* {
    return d.a + (long long)ks * 128 + (long long)i * a_blk;
  };
  auto wsb = [&](const DDma& d, int ks, int i) -> const void* {
    return d.w + (long long)ks * 128 + (long long)i * w_blk;
  };

  DTile t = tile_of(v);
  DDma cur = dma_of(t);
  int vn = v + (int)gridDim.x;
  bool has_next = vn < ntile;
  DTile tn = t;
  DDma nxt = cur;
  if (has_next) {
    tn = tile_of(vn);
    nxt = dma_of(tn);
  }
  // the slice stage k + 2 reads: this tile's, the next tile's first ones,
  // or (after the last tile) this tile's last one again, into a slot nothing
  // reads any more
  auto src_of = [&](int k2, DDma& d, int& ks) {
    const bool here = k2 < nk, ahead = !here && has_next;
    d.a = ahead ? nxt.a : cur.a;
    d.w = ahead ? nxt.w : cur.w;
    d.va = ahead ? nxt.va : cur.va;
    d.vw = ahead ? nxt.vw : cur.vw;
    ks = here ? k2 : (ahead ? k2 - nk : nk - 1);
  };
  auto issue_a = [&](int s, const DDma& d, int ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dma1(slot(2 * s) + wof + i * 4096, asb(d, ks, i), d.va);
  };
  auto issue_w = [&](int s, const DDma& d, int ks) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dma1(slot(2 * s + 1) + wof + i * 4096, wsb(d, ks, i), d.vw);
  };

  // the accumulators are AGPRs a0..a255, named only inside the asm
  Frag8 f0, f1;
  uint32_t P[2 * kUnits];  // the previous tile, bias included, packed bf16
  DPrev prev;
  const float c6 = 3.4358014090685174e-05f;  // degree-6 coefficient of the GELU tail (common.hpp)
  const float s65 = 6.5f;

  // prologue: A_0, W_0, A_1; then W_1 once A_0 and W_0 have landed
  issue_a(0, cur, 0);
  issue_w(0, cur, 0);
  issue_a(1, cur, min(1, nk - 1));
  wait_vmcnt<8>();
  __builtin_amdgcn_s_barrier();
  issue_w(1, cur, min(1, nk - 1));
  read_frags8(f0, slot(0) + oa[0], slot(1) + ob[0]);

  int s5 = 0;  // global stage index mod 5

  // one k-stage without epilogue units (zero: the tile's first, whose first
  // k-step starts the accumulators from zero)
  auto stage_plain = [&](int k, auto zc) {
    const uint32_t sA = slot(2 * s5), sW = slot(2 * s5 + 1);
    DDma dd;
    int ks;
    src_of(k + 2, dd, ks);
    const DDma* d = &dd;
    const uint32_t mA = slot(2 * s5 + 4) + wof;
    if constexpr (decltype(zc)::value)
      dk_z_d4_none(f0, f1, sA + oa[1], sW + ob[1], mA, d->va, asb(*d, ks, 0), a_blk);
    else
      dk_a_d4_none(f0, f1, sA + oa[1], sW + ob[1], mA, d->va, asb(*d, ks, 0), a_blk);
    dk_a_d4_none(f1, f0, sA + oa[2], sW + ob[2], mA + 4 * 4096, d->va, asb(*d, ks, 4), a_blk);
    dk_a_d0_none(f0, f1, sA + oa[3], sW + ob[3]);
    // everything but A_{s+2} has landed (A_{s+1}, W_{s+1}); every wave is
    // past its reads of stage s
    wait_vmcnt<8>();
    __builtin_amdgcn_s_barrier();
    const uint32_t mW = slot(2 * s5) + wof;  // W_{s+2} into A_s's slot
    dk_a_d8_none(f1, f0, slot(2 * s5 + 2) + oa[0], slot(2 * s5 + 3) + ob[0], mW, d->vw, wsb(*d, ks, 0), w_blk);
    s5 = s5 == 4 ? 0 : s5 + 1;
  };

  // the column bias of a tile as one float per lane and block column j: the
  // bias of column n0 + wn*128 + 32 j + lr; loaded as the tile starts and
  // used as it ends, past the previous tile's stores (so waiting for it does
  // not wait for the operand copies in flight)
  auto bias_of = [&](const DTile& t, float (&bv)[4]) {
    const float* bp = p.bias ? p.bias + (long long)t.g * p.bias_gs + t.n0 + wn * 128 + lr : g_no_bias;
    const int js = p.bias ? 32 : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = bp[j * js];
  };
  // a finished tile's accumulators gain its bias: block (i, j) += W'_j x
  // ONES, W'_j's row lr holding bf16 hi(b) and lo(b - hi(b)) of its column's
  // bias in k elements 0, 1 and ONES holding 1.0 there
  auto bias_add = [&](const float (&bv)[4]) {
    u32x4 wb[4], ones;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float b = lh ? 0.f : bv[j];  // the upper lanes hold k elements 8..15: zero
      const float hi = (float)(bf16)b;
      wb[j] = u32x4{pack_bf16(hi, b - hi), 0u, 0u, 0u};
    }
    ones = u32x4{lh ? 0u : pack_bf16(1.f, 1.f), 0u, 0u, 0u};
    dk_bias_add(wb, ones);
  };

  auto store_unit = [&](int u, uint32_t o0, uint32_t o1, char* base) {
    *reinterpret_cast<uint2*>(base + prev.off[unit_i(u)] + unit_col_bytes(u)) = make_uint2(o0, o1);
  };

  // one k-step of a unit stage: unit u of the previous tile rides along
  // (kind 0: the tile's first k-step, from zero, 4 DMA ops; 1: 4 DMA ops;
  // 2: none; 3: 8 DMA ops)
  auto unit_step = [&](auto uc, auto kind, const Frag8& cu, Frag8& nx, uint32_t la, uint32_t lb, uint32_t mb,
                       uint32_t vo, const void* sb, uint32_t sblk) {
    constexpr int u = decltype(uc)::value;
    constexpr int K = decltype(kind)::value;
    if constexpr (EPI == kEpiBias) {
      // the packed bias-added product is the output
      if constexpr (K == 0) dk_z_d4_none(cu, nx, la, lb, mb, vo, sb, sblk);
      if constexpr (K == 1) dk_a_d4_none(cu, nx, la, lb, mb, vo, sb, sblk);
      if constexpr (K == 2) dk_a_d0_none(cu, nx, la, lb);
      if constexpr (K == 3) dk_a_d8_none(cu, nx, la, lb, mb, vo, sb, sblk);
      store_unit(u, P[2 * u], P[2 * u + 1], prev.c);
    } else {
      uint32_t o0, o1;
      if constexpr (K == 0) dk_z_d4_gelu(cu, nx, la, lb, mb, vo, sb, sblk, P[2 * u], P[2 * u + 1], o0, o1, c6, s65);
      if constexpr (K == 1) dk_a_d4_gelu(cu, nx, la, lb, mb, vo, sb, sblk, P[2 * u], P[2 * u + 1], o0, o1, c6, s65);
      if constexpr (K == 2) dk_a_d0_gelu(cu, nx, la, lb, P[2 * u], P[2 * u + 1], o0, o1, c6, s65);
      if constexpr (K == 3) dk_a_d8_gelu(cu, nx, la, lb, mb, vo, sb, sblk, P[2 * u], P[2 * u + 1], o0, o1, c6, s65);
      if constexpr (EPI == kEpiBiasGeluDual) {
        // the pre-activation (bias included, rounded) and its GELU
        store_unit(u, P[2 * u], P[2 * u + 1], prev.c);
        store_unit(u, o0, o1, prev.c2);
      } else {
        store_unit(u, o0, o1, prev.c);
      }
    }
  };

  // stage S (0..15) of a tile that follows another: units 4S .. 4S+3 of the
  // previous tile, one per k-step
  auto stage_units = [&](auto sc) {
    constexpr int S = decltype(sc)::value;
    const int k = S;
    const uint32_t sA = slot(2 * s5), sW = slot(2 * s5 + 1);
    DDma dd;
    int ks;
    src_of(k + 2, dd, ks);
    const DDma* d = &dd;
    const uint32_t mA = slot(2 * s5 + 4) + wof;
    using I0 = std::integral_constant<int, 4 * S>;
    using I1 = std::integral_constant<int, 4 * S + 1>;
    using I2 = std::integral_constant<int, 4 * S + 2>;
    using I3 = std::integral_constant<int, 4 * S + 3>;
    unit_step(I0(), std::integral_constant<int, S == 0 ? 0 : 1>(), f0, f1, sA + oa[1], sW + ob[1], mA, d->va,
              asb(*d, ks, 0), a_blk);
    unit_step(I1(), std::integral_constant<int, 1>(), f1, f0, sA + oa[2], sW + ob[2], mA + 4 * 4096, d->va,
              asb(*d, ks, 4), a_blk);
    unit_step(I2(), std::integral_constant<int, 2>(), f0, f1, sA + oa[3], sW + ob[3], 0, 0, nullptr, 0);
    wait_vmcnt<8>();
    __builtin_amdgcn_s_barrier();
    unit_step(I3(), std::integral_constant<int, 3>(), f1, f0, slot(2 * s5 + 2) + oa[0], slot(2 * s5 + 3) + ob[0],
              slot(2 * s5) + wof, d->vw, wsb(*d, ks, 0), w_blk);
    s5 = s5 == 4 ? 0 : s5 + 1;
  };

  // the finished tile's accumulators -> P (packed bf16) and its store side
  auto transition = [&](const DTile& tp) {
    // the last MFMAs' results are read by ordinary code from here on
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\t" ::);
    // block by block: 16 AGPR reads and 8 packs each (pinned registers, so no
    // block is copied out whole)
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int i = b / 4, j = b % 4;
      uint32_t o[8];
      pack_block(b, o);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = 16 * i + 4 * j + q;
        P[2 * u] = o[2 * q];
        P[2 * u + 1] = o[2 * q + 1];
      }
    }
    prev.c = p.C + (long long)tp.g * p.c_gs;
    prev.c2 = p.C2 ? p.C2 + (long long)tp.g * p.c_gs : nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      prev.off[i] = (uint32_t)((long long)(tp.m0 + wm * 128 + i * 32 + lr) * p.c_rs) +
                    (uint32_t)(tp.n0 + wn * 128 + 4 * lh) * 2;
  };

  using Zero = std::integral_constant<bool, true>;
  using Acc = std::integral_constant<bool, false>;
  float bc[4];
  // the first tile: no previous tile to finish
  bias_of(t, bc);
  stage_plain(0, Zero());
  for (int k = 1; k < nk; ++k) stage_plain(k, Acc());
  bias_add(bc);
  DTile tprev = t;
  while (has_next) {
    t = tn;
    cur = nxt;
    vn += (int)gridDim.x;
    has_next = vn < ntile;
    if (has_next) {
      tn = tile_of(vn);
      nxt = dma_of(tn);
    }
    bias_of(t, bc);
    transition(tprev);
    stage_units(std::integral_constant<int, 0>());
    stage_units(std::integral_constant<int, 1>());
    stage_units(std::integral_constant<int, 2>());
    stage_units(std::integral_constant<int, 3>());
    stage_units(std::integral_constant<int, 4>());
    stage_units(std::integral_constant<int, 5>());
    stage_units(std::integral_constant<int, 6>());
    stage_units(std::integral_constant<int, 7>());
    stage_units(std::integral_constant<int, 8>());
    stage_units(std::integral_constant<int, 9>());
    stage_units(std::integral_constant<int, 10>());
    stage_units(std::integral_constant<int, 11>());
    stage_units(std::integral_constant<int, 12>());
    stage_units(std::integral_constant<int, 13>());
    stage_units(std::integral_constant<int, 14>());
    stage_units(std::integral_constant<int, 15>());
    for (int k = kUnits / 4; k < nk; ++k) stage_plain(k, Acc());
    bias_add(bc);
    tprev = t;
  }
  wait_vmcnt<0>();  // no DMA may land in LDS after this point

  // the last tile's epilogue, plainly
  transition(tprev);
#pragma unroll
  for (int u = 0; u < kUnits; ++u) {
    if constexpr (EPI == kEpiBias) {
      store_unit(u, P[2 * u], P[2 * u + 1], prev.c);
    } else {
      float x[4] = {bf16_lo(P[2 * u]), bf16_hi(P[2 * u]), bf16_lo(P[2 * u + 1]), bf16_hi(P[2 * u + 1])};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = gelu_erf(x[e]);
      if constexpr (EPI == kEpiBiasGeluDual) store_unit(u, P[2 * u], P[2 * u + 1], prev.c);
      store_unit(u, pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), EPI == kEpiBiasGeluDual ? prev.c2 : prev.c);
    }
  }
}

}  // namespace

namespace {
std::atomic<int> g_overlap{0};
}  // namespace

void set_epilogue_overlap(int on) { g_overlap.store(on ? 1 : 0, std::memory_order_relaxed); }
bool epilogue_overlap() { return g_overlap.load(std::memory_order_relaxed) != 0; }

bool gemm_defer_eligible(const GemmArgs& a) {
  if (a.dt != kBF16 || a.row_off || a.a_rowidx || a.rowscale || a.w_kmajor || a.pipe == 0) return false;
  if (!(a.epi == kEpiBiasGelu || a.epi == kEpiBias || (a.epi == kEpiBiasGeluDual && a.C2))) return false;
  if (a.K % 64 || a.K / 64 < kUnits / 4 || a.M < 256 || a.N < 256 || a.G < 1) return false;
  // overlapping edge tiles: at most 1/8 of the computed area recomputed
  const long long tm = (a.M + 255) / 256, tn = (a.N + 255) / 256;
  if (tm * 256 * 8 > 9LL * a.M || tn * 256 * 8 > 9LL * a.N) return false;
  // 32-bit byte offsets from each group's base
  if (((long long)(a.M - 1) * a.a_rs + a.K) * 2 >= (1LL << 32)) return false;
  if ((long long)a.N * a.K * 2 >= (1LL << 32)) return false;
  if (((long long)(a.M - 1) * a.c_rs + a.N) * 2 >= (1LL << 32)) return false;
  // 16-byte aligned operand rows and 8-byte aligned output rows
  if (a.a_rs % 8 || a.a_gs % 8 || a.b_gs % 8 || a.c_rs % 4 || a.c_gs % 4) return false;
  return true;
}

hipError_t launch_gemm_defer(const GemmArgs& a, hipStream_t s) {
  DParams p;
  p.A = (const char*)a.A; p.a_gs = a.a_gs * 2; p.a_rs = a.a_rs * 2; p.a_gdiv = a.a_gdiv;
  p.W = (const char*)a.W; p.b_gs = a.b_gs * 2; p.b_gdiv = a.b_gdiv;
  p.C = (char*)a.C; p.C2 = (char*)a.C2; p.c_gs = a.c_gs * 2; p.c_rs = a.c_rs * 2;
  p.bias = a.bias; p.bias_gs = a.bias_gs;
  p.M = a.M; p.N = a.N; p.K = a.K; p.G = a.G;
  p.tiles_m = (a.M + 255) / 256;
  p.tiles_n = (a.N + 255) / 256;
  // walk the N tiles of an M row when a group's W panels take less space than
  // its A panels (the smaller set is the one kept in L2 across the walk)
  p.n_fast = (double)p.tiles_n < (double)p.tiles_m ? 1 : 0;
  const long long tiles = (long long)a.G * p.tiles_m * p.tiles_n;
  const int cus = device_cus();
  const unsigned grid = (unsigned)(tiles <= cus ? tiles : (cus / 8 * 8 > 0 ? cus / 8 * 8 : cus));
  const dim3 block(256);
  switch (a.epi) {
    case kEpiBiasGelu: hipLaunchKernelGGL(k_gemm_defer<kEpiBiasGelu>, dim3(grid), block, 0, s, p); break;
    case kEpiBias: hipLaunchKernelGGL(k_gemm_defer<kEpiBias>, dim3(grid), block, 0, s, p); break;
    default: hipLaunchKernelGGL(k_gemm_defer<kEpiBiasGeluDual>, dim3(grid), block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace rm

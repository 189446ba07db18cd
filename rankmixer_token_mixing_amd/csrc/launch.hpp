// Host-side launchers of the RankMixer kernels.  Each returns the
// hipError_t of its launch(es); argument checking is done by the caller
// (abi.cpp) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rm {

enum ElemType { kF32 = 0, kBF16 = 1 };

// ---- elementwise / row kernels (kernels_rows.hip) ---------------------------

// The row kernels keep one [D] row per wave in registers: D must be a
// multiple of 8 and of T, and at most 1024 chunks wide (D <= 8192 when the
// head width d = D/T is a multiple of 8).
bool row_width_supported(int T, int D, int dt);

hipError_t launch_tokenize_padsplit(const float* emb, int64_t B, int64_t F, int T, int D, int dt,
                                    void* x0, hipStream_t s);
hipError_t launch_token_mix(const void* x, void* y, int64_t B, int T, int D, int dt, hipStream_t s);
// S = LN(TokenMix(X) + X) row by row; S row (b, t) is written at [b][t] or,
// token_major, at [t][b] (so the rows of one token are contiguous)
hipError_t launch_mix_ln(const void* x, void* s_out, const float* g, const float* b, int64_t B,
                         int T, int D, int dt, bool token_major, hipStream_t s);
// the same S, token-major, from the pad-split tokenizer's fp32 input emb
// [B][F] (X0[b][t][k] = emb[b][t*D + k] cast to dt, 0 past F) without
// writing X0; F % 4 == 0 and F <= T*D
bool mix_ln_emb_supported(int T, int D, int64_t F, int dt);
hipError_t launch_mix_ln_emb(const float* emb, int64_t F, void* s_out, const float* g, const float* b, int64_t B,
                             int T, int D, int dt, hipStream_t s);
// out = LN(z) for fp32 rows z [rows][D]
// out[r] = LN(z[r] + res[r]) * g + b over rows r = b*Tn + t (fp32 math); z,
// res (optional) and out in dtype dt, res row r at res + b * res_bs + t * res_ts
// elements
hipError_t launch_ln_rows(const void* z, const void* res, int64_t res_bs, int64_t res_ts, int Tn, void* out,
                          const float* g, const float* b, int64_t rows, int D, int dt, hipStream_t s);
// block boundary: S' = LN1'(TM(X') + X') with X' = LN2(Z + S), per sample in
// one workgroup; Z [B][T][D], S token-major, overwritten by S' (token-major).
// X' stays in LDS (T rows of D + one head), so only shapes that fit are
// supported.
bool ln_mix_ln_supported(int T, int D, int dt);
hipError_t launch_ln_mix_ln(const void* z, void* s, const float* g2, const float* b2, const float* g1,
                            const float* b1, int64_t B, int T, int D, int dt, hipStream_t st);
// pooled[b] = mean_t x[b,t,:]; logit[b] = w . pooled[b] + c
hipError_t launch_pool_logit(const void* x, const float* w, float c, float* pooled, float* logits,
                             int64_t B, int T, int D, int dt, hipStream_t s);

// ---- MoE routing and combine (kernels_moe.hip) -------------------------------

struct MoeWork {
  float* gates;     // [B][T][E]
  int* counts;      // [G]   G = T*E
  int* offsets;     // [G+1]
  int* rows;        // [B*T*E]  sample index per compacted entry
  float* gatec;     // [B*T*E]  gate per compacted entry
  int* pos;         // [B][T][E] compacted index or -1
  int* tiles;       // [2 * max_tiles] (group, m0) pairs
  int* ntiles;      // [1]
};
// S row (b, t) of the MoE kernels sits at b * sb + t * st (elements)
hipError_t launch_moe_router(const void* s, int64_t sb, int64_t st_, const void* wr, const float* br,
                             float* gates, int64_t B, int T, int D, int E, int dt, hipStream_t st);
hipError_t launch_moe_compact(const MoeWork& w, int64_t B, int T, int E, int bm, hipStream_t st);
// v[b,t,:] = sum_j y[pos[b,t,j], :]; if ln: out = LN(v + s) else out = v
hipError_t launch_moe_combine(const void* y, const int* pos, const void* s, int64_t sb, int64_t st_,
                              const float* g, const float* b, void* out, int64_t B, int T, int D,
                              int E, bool ln, int dt, hipStream_t st);

// ---- grouped MFMA GEMM (kernels_gemm.hip) ------------------------------------

// compute units of the current device (cached per device)
int device_cus();

enum Epilogue {
  kEpiBiasGelu = 0,       // C(dt)  = GELU(acc + bias[n])
  kEpiBias = 1,           // C(dt)  = acc + bias[n]
  kEpiBiasF32 = 2,        // C(f32) = acc + bias[n]
  kEpiBiasScale = 3,      // C(dt)  = rowscale[m] * (acc + bias[n])
  // C(dt)[m][h] = SiLU(acc_g + bias[h]) * (acc_u + bias[Hs + h]), h < Hs = N/2:
  // W rows 0..Hs-1 are the gate rows, Hs..N-1 the up rows; C is Hs wide.
  // Pipelined kernel only (gemm_pipe_eligible).
  kEpiSwiglu = 4,
  // C(dt) = acc + bias[n] and C2(dt) = GELU(C) (same layout; training keeps
  // the pre-activation).  Pipelined kernel only.
  kEpiBiasGeluDual = 5,
  // backward through the GELU: C(dt) = acc * GELU'(aux), aux (dt) the
  // pre-activation U at C's layout, and colsum[(g * tiles_m + tm) * 16 + r][n]
  // = the sum of the rounded C over rows m0 + r, m0 + r + 16, ... of M tile
  // tm (256 rows) -- 16 partial column sums per M tile (the bias gradient).
  // No bias.  K-major ring only (gemm_kmajor_eligible).
  kEpiGeluBwd = 6,
};

// C_g[m][n] = sum_k A_g[m][k] * W_g[n][k], g = 0..G-1, followed by an epilogue.
// Element offsets (not bytes).  Row m of A in group g sits at
//   (g / a_gdiv) * a_gs + rowid(m) * a_rs,   rowid(m) = a_rowidx ? a_rowidx[base+m] : base+m
// with base = row_off ? row_off[g] : 0; W_g row n at (g / b_gdiv) * b_gs + n * K; output
// row m of group g at (base + m) * c_rs + g * c_gs (the residual the same way
// with r_rs / r_gs); bias of group g at g * bias_gs.
struct GemmArgs {
  int dt = kBF16;
  int epi = kEpiBias;
  int M = 0, N = 0, K = 0, G = 0;
  const void* A = nullptr; int64_t a_gs = 0, a_rs = 0; int a_gdiv = 1;
  const int* a_rowidx = nullptr;
  const void* W = nullptr; int64_t b_gs = 0; int b_gdiv = 1;  // W group of g at (g / b_gdiv) * b_gs
  void* C = nullptr; int64_t c_gs = 0, c_rs = 0;
  void* C2 = nullptr;  // kEpiBiasGeluDual
  const float* bias = nullptr; int64_t bias_gs = 0;
  const float* rowscale = nullptr;
  // ragged mode (MoE): group g has row_off[g+1]-row_off[g] rows; the tiles
  // to run are the (g, m0) pairs tiles[0..2*ntiles) with *ntiles on the device;
  // max_mtiles bounds *ntiles (the grid is sized for it).
  const int* row_off = nullptr;
  const int* tiles = nullptr;
  const int* ntiles = nullptr;
  int max_mtiles = 0;
  // W group stored K-major, [K][N] (element (k, n) at (g / b_gdiv) * b_gs +
  // k * N + n), read along its rows with transposed LDS fragment reads, where
  // gemm_wt_eligible (bf16, K % 64 == 0, dense, 256 x 256 tiles): the
  // backward epilogues (fp32 result, GELU backward) on the hand-scheduled
  // pipelined kernel, the forward ones on the compiler-scheduled ring
  int w_kmajor = 0;
  // A group stored K-major, [K][M] (element (k, m) at (g / a_gdiv) * a_gs +
  // k * a_rs + m), with w_kmajor: both operands read along their rows with
  // transposed LDS fragment reads (the weight-gradient products, K = batch)
  int a_kmajor = 0;
  const void* aux = nullptr;  // kEpiGeluBwd: the pre-activation
  int64_t aux_gs = -1, aux_rs = -1;  // its group and row strides (elements; -1: C's)
  float* colsum = nullptr;    // kEpiGeluBwd: the partial column sums
  int tile_cfg = -1;  // -1: choose automatically
  int pipe = -1;      // 0: never use the hand-scheduled ring (for comparisons)
};
// Row count of the M tile a launch of `a` will use (ragged tile lists are
// built for this).
int gemm_tile_m(const GemmArgs& a);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);
// whether launch_gemm would run `a` on the hand-scheduled pipelined kernel
// (the ring kernel with the epilogue after each tile, or the deferred-epilogue
// kernel)
bool gemm_pipe_eligible(const GemmArgs& a);
// the deferred-epilogue kernel (kernels_gemm_defer.hip): bf16, dense, bias /
// bias + GELU / both, K a multiple of 64 and at least 1024, M and N at least
// 256; launch_gemm takes it for those when the epilogue-overlap mode is on
bool gemm_defer_eligible(const GemmArgs& a);
// the epilogue-overlap mode (process-wide, off by default)
void set_epilogue_overlap(int on);
bool epilogue_overlap();
hipError_t launch_gemm_defer(const GemmArgs& a, hipStream_t s);
// whether launch_gemm takes `a` with a K-major W (w_kmajor)
bool gemm_wt_eligible(const GemmArgs& a);
// whether launch_gemm takes `a` with K-major operands and 256 x 256 tiles
// whatever the tile count: both operands K-major (a_kmajor, w_kmajor,
// kEpiBiasF32) or a K-major W with the kEpiGeluBwd epilogue.  bf16, dense,
// K a multiple of 64, M and N at least 256 and multiples of 8.  They run on
// the hand-scheduled pipelined kernel (the ring where a 32-bit DMA offset
// would not fit)
bool gemm_kmajor_eligible(const GemmArgs& a);
// number of partial column sums per group that kEpiGeluBwd writes
int gemm_colsum_parts(int M);

// ---- dense block backward (kernels_bwd.hip) -----------------------------------

// LayerNorm backward over rows (b, t).  mode 0: Y = z + res (z [B][T][D], res
// token-major), upstream dout [B][T][D], dY written token-major in dt.  mode 1:
// Y = TM(z) + z (z = X [B][T][D]), upstream dres (token-major, dt) + dres32
// (token-major fp32), dY written [B][T][D] fp32.  part receives, per workgroup
// g < ln_bwd_grid(B, T, D), the partial sums of dout * xhat and dout: part[g][2][D].
int ln_bwd_grid(int64_t B, int T, int D);
int ln_bwd_max_width();
hipError_t launch_ln_bwd(int mode, const void* dout, const void* dres, const float* dres32, const void* z,
                         const void* res, const float* gamma, void* dy, float* part, int64_t B, int T, int D, int dt,
                         hipStream_t s, const float* dres32b = nullptr);
// out[g][c][r] = op(in[g][r][c]) for r < ldo (zero for r >= R), in [G][R][C];
// op 0 identity, 1 GELU, 2 in * GELU'(aux) (direct, if set, receives op(in);
// out2, if set, receives GELU(aux) transposed like out).  colsum, if set,
// receives [G][transpose_row_tiles][C] sums of op(in) over each 64-row tile.
// C and ldo multiples of 8, ldo >= R.  Input (and aux) element (g, r, c) at
// g * in_gs + r * in_rs + c (defaults: in_rs = C, in_gs = R * in_rs); direct
// element (g, r, c) at g * dir_gs + r * dir_rs + c (defaults: the input's).
int transpose_row_tiles(int64_t R, int64_t ldo);
hipError_t launch_transpose(int op, const void* in, const void* aux, void* out, void* direct, void* out2,
                            float* colsum, int G, int64_t R, int64_t C, int64_t ldo, int dt, hipStream_t s,
                            int64_t in_gs = -1, int64_t in_rs = -1, int64_t dir_gs = -1, int64_t dir_rs = -1);
// dx = dy + TM(dy): dy fp32 [B][T][D], dx in dt
hipError_t launch_tm_add(const float* dy, void* dx, int64_t B, int T, int D, int dt, hipStream_t s);
// out[g][c] = scale * sum_p part[g][p][c] (fixed order); c < split -> out0, else out1
hipError_t launch_sum_parts(const float* part, float* out0, float* out1, int G, int P, int64_t C, int64_t split,
                            hipStream_t s, float scale = 1.0f);
// part[g][b][c] = sum of in[g][r][c] over the rows of 64-row block b
// (colsum64_parts(R) blocks; in [G][R][C], C a multiple of 8)
int colsum64_parts(int64_t R);
hipError_t launch_colsum64(const void* in, float* part, int G, int64_t R, int64_t C, int dt, hipStream_t s);
// h = GELU(u), n elements (a multiple of 8)
hipError_t launch_gelu_ew(const void* u, void* h, int64_t n, int dt, hipStream_t s);

// ---- block variants (kernels_variants.hip) -------------------------------------

// SwiGLU: h[r][j] = SiLU(gu[r][j]) * gu[r][Hs + j] over rows of 2*Hs (Hs % 8 == 0)
hipError_t launch_swiglu_ew(const void* gu, void* h, int64_t rows, int Hs, int dt, hipStream_t s);

// ---- MoE training, dense-training / sparse-inference (kernels_moe_train.hip) --

// z[r][:] = sum_j gate[r][j] * y[r][j][:] over rows r < rows (y [rows][E][D], y and z in dt)
hipError_t launch_moe_combine_dense(const void* y, const float* gate, void* z, int64_t rows, int E, int D, int dt,
                                    hipStream_t s);
// per row (b, t): dy = G_train * dV (written [T][E][B][D]), dz = (dV . y_j)
// [G_train > 0], mask = [G_infer > 0], dsr = sum_j dz_j Wr_train[t][j] (see
// kernels_moe_train.hip)
hipError_t launch_moe_bwd_rows(const void* dv, const void* y, const float* gt, const float* gi, const void* wr,
                               void* dy, void* dz, void* mask, float* dsr, int64_t B, int T, int E, int D, int dt,
                               hipStream_t s);
// out[0] = sum of x[0 .. n), fixed order, through part[sum_all_parts(n)]
// partial sums (part at most kSumParts floats)
constexpr int kSumParts = 512;
int sum_all_parts(int64_t n);
hipError_t launch_sum_all(const float* x, float* out, int64_t n, float* part, hipStream_t s);
// x *= scale
hipError_t launch_scale(float* x, int64_t n, float scale, hipStream_t s);

// ---- projection tokenizer (kernels_tokproj.hip) -------------------------------

// x0[b][t][:] = W_t . bf16(pad(emb[b])[t*seg : (t+1)*seg]) + bias_t in one
// kernel that reads the fp32 embedding in place: bf16 weights [T][D][seg]
// and output [B][T][D], F % 4 == 0, seg % 8 == 0, seg <= the returned
// maximum, D % 8 == 0
hipError_t launch_tokenize_project(const float* emb, const void* w, const float* bias, void* x0, int64_t B, int64_t F,
                                   int T, int seg, int D, hipStream_t s);
int tokenize_project_max_seg();

// ---- measurement probes (kernels_probe.hip) ------------------------------------

// waves of one probe_mfma launch (8 per compute unit); frags holds 64 sets of
// 16 fragments of 64 lanes x 16 bytes
int probe_mfma_waves();
constexpr long long kProbeFragBytes = 64LL * 16 * 64 * 16;
hipError_t launch_probe_mfma(const void* frags, float* out, int iters, hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, long long n16, hipStream_t s);
// the k-step probe: one workgroup of 8 waves per compute unit; slab: the A and
// W slices (kProbeSlabBytes of bf16), out: probe_kstep_blocks() * 512 floats
constexpr int kProbeSlabBytes = 65536;
int probe_kstep_blocks();
hipError_t launch_probe_kstep(const void* slab, float* out, int iters, hipStream_t s);

}  // namespace rm

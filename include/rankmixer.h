/*
 * rankmixer.h - C ABI of librankmixer.so: the RankMixer block forward on
 * AMD MI355X (gfx950), built from hand-written HIP kernels.
 *
 * Pages cited (titles as printed on them):
 *   [FR] "Rankmixer: 硬件效率优化" (fun-rec textbook chapter)
 *   [WL] "特征交叉 —— RankMixer 精读笔记" (reading notes on arXiv 2507.15551)
 *   [TB] "淘宝闪购-爆品团精排 Scaling Up 迭代实践" (BestBlogs.dev report)
 *   [SX] "重新理解 RankMixer：扩参为什么有效，又为什么划算？" (sxkj888.cn blog)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, contiguous, row-major device buffers.  Activations
 *    are [B][T][D]: B samples, T tokens, token width D.  Weight matrices are
 *    stored [out][in], so every product reads both operands along the
 *    reduction axis.  Biases, LayerNorm gamma/beta, the router bias and the
 *    logit head are float32.  Activations and weight matrices are float32 or
 *    bf16 (rm_dtype); products accumulate in float32.
 *  - Every device pointer must be 16-byte aligned.  Optional pointers may be
 *    NULL where stated.
 *  - B is the batch size; B = 0 is an empty batch: the call checks its other
 *    arguments, returns RM_OK and enqueues nothing (data pointers may then be
 *    NULL), except the backward calls, which write zero gradients, and
 *    rm_moe_block_fwd_train, which writes a zero sparsity loss.  B < 0 is
 *    RM_ERR_INVALID.
 *  - Width limits of this build: D a multiple of 8 (and of T wherever tokens
 *    are mixed), hidden widths a multiple of 8, one [D] row per wavefront in
 *    registers, at most 1024 16-byte chunks of one head width (bf16:
 *    D <= 8192 when D/T is a multiple of 8; fp32: D <= 4096 when D/T is a
 *    multiple of 4; narrower heads allow proportionally less); the FFN and
 *    MoE calls, blocks with an MoE and the training calls: D <= 4096; MoE:
 *    1 <= E <= 32, T*E <= 4096.
 *    Larger shapes are RM_ERR_UNSUPPORTED.
 *  - The caller owns every buffer, including the workspace `ws`, sized with
 *    the matching rm_*_workspace_bytes call.  The library never allocates,
 *    frees or synchronises (its one fixed device array, the scratch of
 *    rm_moe_route_noalloc, is part of its code object); work is enqueued on
 *    `stream` (a hipStream_t, NULL for the default stream) and is complete
 *    when that stream is.
 *  - Outputs must not alias inputs.
 *  - Results are deterministic: two calls with the same inputs give the same
 *    bits (no floating-point atomics anywhere).
 *  - Every argument check runs on the host before anything is enqueued.  A
 *    failing call returns a non-zero rm_status, enqueues nothing and leaves a
 *    message for rm_last_error() (per thread).  RM_ERR_HIP reports a launch
 *    failure; a fault inside a kernel surfaces at the caller's next
 *    synchronisation of the stream.
 */
#ifndef RANKMIXER_H
#define RANKMIXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rm_status {
  RM_OK = 0,
  RM_ERR_INVALID = 1,     /* NULL pointer, non-positive size, misaligned pointer */
  RM_ERR_UNSUPPORTED = 2, /* shape the method or this build does not define (D % T != 0, ...) */
  RM_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the matching rm_*_workspace_bytes */
  RM_ERR_HIP = 4          /* the HIP runtime refused a launch */
} rm_status;

typedef enum rm_dtype { RM_F32 = 0, RM_BF16 = 1 } rm_dtype;

typedef enum rm_block_kind { RM_BLOCK_DENSE = 0, RM_BLOCK_MOE = 1, RM_BLOCK_SWIGLU = 2 } rm_block_kind;

/* rm_block_params.flags: drop the Add & Norm after the token mix, S = TM(X)
 * ([TB] section 3.5 reports the block that lost it) */
#define RM_BLOCK_NO_MIX_NORM 1

/* Per-token FFN of one block ([FR] "Per-Token FFN"; [WL] "Per-Token FFN"):
 *   v_t = W2_t GELU(W1_t s_t + b1_t) + b2_t,  t = 0..T-1, GELU the exact erf form.
 * The pages print W1_t as R^{D x kD} but apply it to s_t in R^D; W1_t here maps
 * R^D -> R^Hd and is stored [Hd][D]. */
typedef struct rm_pffn_params {
  const void* w1;  /* [T][Hd][D], dtype */
  const float* b1; /* [T][Hd] */
  const void* w2;  /* [T][D][Hd], dtype */
  const float* b2; /* [T][D] */
} rm_pffn_params;

/* ReLU-gated per-token MoE ([FR] "Sparse MoE扩展"; [WL] ReLU routing):
 *   G_{t,j} = ReLU(Wr_t s_t + br_t)_j,   v_t = sum_j G_{t,j} e_{t,j}(s_t),
 *   e_{t,j}(s) = W2_{t,j} GELU(W1_{t,j} s + b1_{t,j}) + b2_{t,j}.
 * Only the inference router exists in the forward (dense-train/sparse-infer
 * keeps h_infer at inference).  A zero gate means the expert is skipped. */
typedef struct rm_moe_params {
  const void* wr;  /* [T][E][D], dtype */
  const float* br; /* [T][E] */
  const void* w1;  /* [T][E][He][D], dtype */
  const float* b1; /* [T][E][He] */
  const void* w2;  /* [T][E][D][He], dtype */
  const float* b2; /* [T][E][D] */
} rm_moe_params;

/* One block ([FR] "RankMixer整体架构", block equations):
 *   S = LN1(TokenMix(X) + X),   X' = LN2(F(S) + S),
 * F the per-token FFN (kind DENSE), the ReLU MoE (kind MOE) or the per-token
 * SwiGLU FFN (kind SWIGLU, [TB] section 3.6 "SwiGLU D->4/3D"):
 *   v_t = W2_t (SiLU(Wg_t s_t + bg_t) * (Wu_t s_t + bu_t)) + b2_t,
 * its pffn.w1 [T][2*Hs][D] holding the gate rows Wg_t then the up rows Wu_t,
 * pffn.b1 [T][2*Hs] likewise, pffn.w2 [T][D][Hs], hidden = Hs.  With flag
 * RM_BLOCK_NO_MIX_NORM, S = TokenMix(X) (ln1_g / ln1_b unused).  LayerNorm:
 * biased variance over the D entries of one token, epsilon 1e-5. */
typedef struct rm_block_params {
  int kind;                   /* rm_block_kind */
  const float* ln1_g;         /* [D] */
  const float* ln1_b;         /* [D] */
  const float* ln2_g;         /* [D] */
  const float* ln2_b;         /* [D] */
  rm_pffn_params pffn;        /* used when kind == RM_BLOCK_DENSE or RM_BLOCK_SWIGLU */
  rm_moe_params moe;          /* used when kind == RM_BLOCK_MOE */
  int flags;                  /* 0 or RM_BLOCK_NO_MIX_NORM */
  /* The block's own widths, which size every weight above: hidden = Hd
   * (DENSE), Hs (SWIGLU) or He (MOE); E = experts per token (MOE), else 0.
   * rm_model_fwd sizes and runs each block from these two fields, so the
   * blocks of one stack may differ in kind, hidden width and expert count.
   * The single-block calls take hidden and E as arguments; there, 0 in a
   * field means "as the argument", and a non-zero field that differs from
   * the argument is RM_ERR_INVALID. */
  int hidden;
  int E;
} rm_block_params;

/* Gradients of one dense block: float32 device buffers, overwritten (not
 * accumulated) by rm_block_bwd. */
typedef struct rm_block_grads {
  float* w1;     /* [T][Hd][D] */
  float* b1;     /* [T][Hd] */
  float* w2;     /* [T][D][Hd] */
  float* b2;     /* [T][D] */
  float* ln1_g;  /* [D] */
  float* ln1_b;  /* [D] */
  float* ln2_g;  /* [D] */
  float* ln2_b;  /* [D] */
} rm_block_grads;

/* A stack of L blocks ([FR] "RankMixer整体架构": X_L = block_L(...block_1(X_0))),
 * with an optional pad-split tokenizer in front and optional mean pooling
 * plus a D -> 1 logit behind ([WL]: the last block's tokens are averaged). */
typedef struct rm_model_desc {
  int T, D;                   /* tokens and token width, shared by every block */
  int dtype;                  /* rm_dtype of activations and weight matrices */
  int L;                      /* number of blocks */
  const rm_block_params* blocks; /* host array of L block descriptors */
  int64_t F;                  /* > 0: the input is an fp32 embedding [B][F], pad-split tokenized */
  const float* head_w;        /* [D] device, or NULL: no pooling / logit */
  float head_c;               /* logit bias */
} rm_model_desc;

/* Pad-split tokenizer ([TB] section 3.4: concatenate -> pad -> split, no
 * projection).  x0[b][t][j] = emb[b][t*D + j] cast to out_dtype (round to
 * nearest even) when t*D + j < F, else 0.
 *   emb: [B][F] fp32 device; x0: [B][T][D] out_dtype device.
 * Errors: F > T*D -> RM_ERR_UNSUPPORTED. */
rm_status rm_tokenize_padsplit(const float* emb, int64_t B, int64_t F, int T, int D,
                               int out_dtype, void* x0, void* stream);

/* Weights of the projection tokenizer: one linear layer per token. */
typedef struct rm_proj_params {
  const void* w;   /* [T][D][seg], dtype: W_t maps a segment R^seg -> R^D */
  const float* b;  /* [T][D] */
} rm_proj_params;

/* Projection tokenizer ([WL] "特征的Tokenization": the concatenated embedding
 * is cut evenly into T segments and each segment goes through its own linear
 * layer into R^D).  Segments have length seg >= ceil(F/T); emb is zero-padded
 * to T*seg and cast to dtype (round to nearest even), then
 *   x0[b][t][:] = W_t pad(emb[b])[t*seg : (t+1)*seg] + b_t,
 * accumulated in fp32 and rounded once to dtype.
 *   emb: [B][F] fp32 device; x0: [B][T][D] dtype device; params as
 *   rm_proj_params (device pointers).
 * Workspace: rm_tokenize_project_workspace_bytes(B, F, T, seg, dtype): 0 for
 * bf16 with F a multiple of 4 and seg <= 384 (one launch reads emb in place
 * and rounds it to bf16 on the way into the product; ws may then be NULL),
 * else room for the padded, cast segments.
 * Errors: F > T*seg, seg or D not a multiple of 8 -> RM_ERR_UNSUPPORTED. */
rm_status rm_tokenize_project(const float* emb, const rm_proj_params* p, int64_t B, int64_t F,
                              int T, int seg, int D, int dtype, void* x0, void* ws,
                              size_t ws_bytes, void* stream);
size_t rm_tokenize_project_workspace_bytes(int64_t B, int64_t F, int T, int seg, int dtype);

/* Multi-head token mixing with H = T ([FR] "Token Mixing机制"; [WL] "Multi-Head
 * Token Mixer"): SplitHead cuts token t into T heads of width d = D/T, Concat
 * joins head h of all tokens in token order:
 *   y[b][h][t*d + j] = x[b][t][h*d + j].
 * Pure data movement, bit-exact; applying it twice gives x back.
 *   x, y: [B][T][D] dtype device.  Errors: D % T != 0 -> RM_ERR_UNSUPPORTED. */
rm_status rm_token_mix(const void* x, void* y, int64_t B, int T, int D, int dtype, void* stream);

/* Per-token FFN without residual or LayerNorm: v = PFFN(s).
 *   s, v: [B][T][D] dtype device; params as rm_pffn_params (device pointers).
 * Workspace: rm_pffn_workspace_bytes(B, T, D, Hd, dtype). */
rm_status rm_pffn_fwd(const void* s, const rm_pffn_params* p, void* v, int64_t B, int T, int D,
                      int Hd, int dtype, void* ws, size_t ws_bytes, void* stream);
size_t rm_pffn_workspace_bytes(int64_t B, int T, int D, int Hd, int dtype);

/* ReLU-gated per-token MoE without residual or LayerNorm: v = MoE(s).
 *   s, v: [B][T][D] dtype device; gates: optional [B][T][E] fp32 device output
 *   of G (NULL to skip).  E <= 32.  Experts run only on compacted lists of the
 *   (sample, token) rows whose gate is positive.
 * Workspace: rm_moe_workspace_bytes(B, T, D, E, He, dtype). */
rm_status rm_moe_relu_fwd(const void* s, const rm_moe_params* p, void* v, float* gates, int64_t B,
                          int T, int D, int E, int He, int dtype, void* ws, size_t ws_bytes,
                          void* stream);
size_t rm_moe_workspace_bytes(int64_t B, int T, int D, int E, int He, int dtype);

/* Routing step of the MoE alone: gates and the compacted active lists.
 *   gates:   [B][T][E] fp32 device output, G = ReLU(Wr_t s + br_t).
 *   offsets: [T*E + 1] int32 device output; list g = t*E + j holds entries
 *            offsets[g] .. offsets[g+1]-1.
 *   rows:    [B*T*E] int32 device output; rows[i] = sample b of entry i, in
 *            increasing b within each list (only offsets[T*E] entries are set).
 * Workspace: rm_moe_workspace_bytes(...) (the same buffer as rm_moe_relu_fwd). */
rm_status rm_moe_route(const void* s, const void* wr, const float* br, float* gates, int* offsets,
                       int* rows, int64_t B, int T, int D, int E, int dtype, void* ws,
                       size_t ws_bytes, void* stream);

/* rm_moe_route without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, outputs and errors as rm_moe_route,
 * minus ws / ws_bytes: its scratch (per-list counts, the tile list, the
 * compacted gates and the entry map) lives in one fixed device array of
 * rm_moe_route_noalloc_max_scratch_bytes() = 16 MiB that the library holds
 * on each device it runs on until the process ends.  A call needs
 * rm_moe_route_noalloc_scratch_bytes(B, T, E) of it (about 8 bytes per
 * (sample, token, expert) entry: B*T*E up to about 2 million); larger calls
 * -> RM_ERR_UNSUPPORTED.  The call allocates nothing (no hipMalloc, no
 * allocating library routine); its first call on a device looks up that
 * device's copy of the array.  Every call on a device shares the array:
 * calls that overlap on one device (two streams, two threads) race and must
 * be ordered by the caller.  Nothing in the array needs clearing between
 * calls (each call writes every element it reads). */
size_t rm_moe_route_noalloc_scratch_bytes(int64_t B, int T, int E);
size_t rm_moe_route_noalloc_max_scratch_bytes(void);
rm_status rm_moe_route_noalloc(const void* s, const void* wr, const float* br, float* gates, int* offsets,
                               int* rows, int64_t B, int T, int D, int E, int dtype, void* stream);

/* One block: x_out = LN2(F(S) + S), S = LN1(TokenMix(x) + x).
 *   x, x_out: [B][T][D] dtype device.  hidden = Hd (dense) or He (MoE);
 *   E = experts per token (MoE) or 0.
 * Workspace: rm_block_workspace_bytes(kind, B, T, D, hidden, E, dtype). */
rm_status rm_block_fwd(const void* x, const rm_block_params* p, void* x_out, int64_t B, int T,
                       int D, int hidden, int E, int dtype, void* ws, size_t ws_bytes,
                       void* stream);
size_t rm_block_workspace_bytes(int kind, int64_t B, int T, int D, int hidden, int E, int dtype);

/* The whole stack.  Block l is sized from its own descriptor
 * (m->blocks[l].hidden and .E, which must be set: hidden > 0, E in 1..32 for
 * MoE blocks and 0 otherwise), so its weights must have exactly those widths.
 *   in:     m->F > 0: emb [B][F] fp32 device; else x0 [B][T][D] dtype device.
 *   x_out:  [B][T][D] dtype device output of the last block, or NULL.
 *   pooled: [B][D] fp32 device output of the token mean, or NULL (needs head_w).
 *   logits: [B] fp32 device output, or NULL (needs head_w).
 * Workspace: rm_model_workspace_bytes(m, B). */
rm_status rm_model_fwd(const rm_model_desc* m, const void* in, void* x_out, float* pooled,
                       float* logits, int64_t B, void* ws, size_t ws_bytes, void* stream);
size_t rm_model_workspace_bytes(const rm_model_desc* m, int64_t B);

/* Dense block training forward: the forward of rm_block_fwd, which also keeps
 * what rm_block_bwd needs in the caller's `saved` buffer (S, the W1 product +
 * b1 before GELU, its GELU, the W2 product + b2; size rm_block_saved_bytes).
 * The output
 * equals rm_block_fwd's up to the rounding of the GELU input to dtype.
 *   Workspace: rm_block_workspace_bytes(RM_BLOCK_DENSE, B, T, D, hidden, 0, dtype).
 * Errors: a block that is not DENSE or has flags, D > 4096 -> RM_ERR_UNSUPPORTED
 * (besides rm_block_fwd's). */
size_t rm_block_saved_bytes(int64_t B, int T, int D, int hidden, int dtype);
rm_status rm_block_fwd_train(const void* x, const rm_block_params* p, void* x_out, void* saved,
                             size_t saved_bytes, int64_t B, int T, int D, int hidden, int dtype,
                             void* ws, size_t ws_bytes, void* stream);

/* Dense block backward: the chain rule through the block equations of
 * [FR] "RankMixer整体架构" (the pages train the block but print no backward).
 * Given d_out = dL/dX' it writes dx = dL/dX and every parameter gradient:
 *   LN2:  dY2 = LNbwd(d_out);  dV = dY2;  dgamma2 = sum d_out*xhat2, dbeta2 = sum d_out
 *   W2:   db2_t = sum_b dV_t;  dW2_t = dV_t^T H_t;  dH_t = dV_t W2_t
 *   GELU: dU = dH * GELU'(U)
 *   W1:   db1_t = sum_b dU_t;  dW1_t = dU_t^T S_t;  dS = dY2 + dU_t W1_t
 *   LN1:  dY1 = LNbwd(dS);  dX = dY1 + TM(dY1)   (TM is its own transpose)
 * with LNbwd(g) = (g*gamma - mean(g*gamma) - xhat * mean(g*gamma*xhat)) / sigma.
 *   x: the block input [B][T][D] dtype; saved: from rm_block_fwd_train on the
 *   same x and params; d_out, dx: [B][T][D] dtype; g: gradients (fp32).
 * Products run in dtype with fp32 accumulation (bf16: dV and dU rounded to
 * bf16, and dH too where it is stored); sums over the batch and over rows run
 * in a fixed order, so results are deterministic.  bf16 with B a multiple of
 * 64 and D, hidden >= 256: the dH product applies GELU' in its epilogue (dH is
 * never stored) and the batch-contracting products read their operands as
 * stored; otherwise they read transposed copies.  B = 0 writes zero
 * gradients.
 *   Workspace: rm_block_bwd_workspace_bytes(B, T, D, hidden, dtype).
 * Errors: as rm_block_fwd_train; dx aliasing x or d_out -> RM_ERR_INVALID. */
size_t rm_block_bwd_workspace_bytes(int64_t B, int T, int D, int hidden, int dtype);
rm_status rm_block_bwd(const void* x, const rm_block_params* p, const void* saved, size_t saved_bytes,
                       const void* d_out, void* dx, const rm_block_grads* g, int64_t B, int T,
                       int D, int hidden, int dtype, void* ws, size_t ws_bytes, void* stream);

/* Gradients of one MoE block trained with the dense-training / sparse-
 * inference routers: float32 device buffers, overwritten by rm_moe_block_bwd. */
typedef struct rm_moe_grads {
  float* w1;        /* [T][E][He][D] */
  float* b1;        /* [T][E][He] */
  float* w2;        /* [T][E][D][He] */
  float* b2;        /* [T][E][D] */
  float* wr_train;  /* [T][E][D]  training router h_train */
  float* br_train;  /* [T][E] */
  float* wr_infer;  /* [T][E][D]  inference router h_infer (p->moe.wr) */
  float* br_infer;  /* [T][E] */
  float* ln1_g;     /* [D] */
  float* ln1_b;     /* [D] */
  float* ln2_g;     /* [D] */
  float* ln2_b;     /* [D] */
} rm_moe_grads;

/* MoE block training forward with two routers per token ([FR] "Sparse
 * MoE扩展", dense-training / sparse-inference; [WL] ReLU routing):
 *   S = LN1(TM(X) + X);  G_train = ReLU(S_t Wr_train_t^T + br_train_t)
 *   G_infer = ReLU(S_t Wr_t^T + br_t)   (Wr, br: the block's own router p->moe)
 *   v_t = sum_j G_train[t, j] * (W2_tj GELU(W1_tj s_t + b1_tj) + b2_tj)
 *   X' = LN2(v + S);  *l_reg = sum over b, t, j of G_infer[b, t, j]
 * The training router routes; the inference router only feeds the sparsity
 * loss L_reg (at inference, rm_block_fwd routes with p->moe alone).  Every
 * expert runs on every token (dense training); a zero gate contributes zero.
 *   x: [B][T][D] dtype; p: an MoE block without flags; wr_train: [T][E][D]
 *   dtype device; br_train: [T][E] fp32 device; x_out: [B][T][D] dtype;
 *   l_reg: one fp32 on the device; saved: the caller's buffer of
 *   rm_moe_saved_bytes for rm_moe_block_bwd (S, the W1 products + b1 and
 *   their GELU, the expert outputs, both gate sets, v).
 *   Workspace: rm_moe_train_workspace_bytes(B, T, D, He, E, dtype).
 * B = 0 writes *l_reg = 0.
 * Errors: a block that is not MOE or has flags, D > 4096, T*E not a multiple
 * of 8, B*T*E*He >= 2^31 -> RM_ERR_UNSUPPORTED; NULL pointers, x_out aliasing
 * x -> RM_ERR_INVALID; a short saved buffer or workspace -> RM_ERR_WORKSPACE. */
size_t rm_moe_saved_bytes(int64_t B, int T, int D, int He, int E, int dtype);
size_t rm_moe_train_workspace_bytes(int64_t B, int T, int D, int He, int E, int dtype);
rm_status rm_moe_block_fwd_train(const void* x, const rm_block_params* p, const void* wr_train,
                                 const float* br_train, void* x_out, float* l_reg, void* saved,
                                 size_t saved_bytes, int64_t B, int T, int D, int He, int E, int dtype,
                                 void* ws, size_t ws_bytes, void* stream);

/* MoE block backward of L = <d_out, X'> + lambda * L_reg, the chain rule
 * through the equations of rm_moe_block_fwd_train (the pages print no
 * backward).  L_reg is applied to h_infer only, so its gradient reaches
 * h_infer's weights and bias and nothing else; the task loss reaches every
 * parameter but h_infer:
 *   dV = LNbwd2(d_out);  dy_tj = G_train[t, j] dV_t;  dG_tj = dV_t . y_tj
 *   experts (per t, j): db2 = sum_b dy;  dW2 = dy^T H;  dU = (dy W2) * GELU'(U)
 *              db1 = sum_b dU;  dW1 = dU^T S_t;  dS_t += dU W1
 *   h_train:   dz = dG [G_train > 0];  dbr_train = sum_b dz;  dWr_train = dz^T S_t;
 *              dS_t += dz Wr_train_t
 *   h_infer:   dzi = lambda [G_infer > 0];  dbr = sum_b dzi;  dWr = dzi^T S_t
 *   dS += dV;  dY1 = LNbwd1(dS);  dX = dY1 + TM(dY1)
 * Arguments as rm_moe_block_fwd_train (saved from that call on the same x and
 * parameters); d_out, dx: [B][T][D] dtype; g: fp32 gradients.  Products in
 * dtype with fp32 accumulation (bf16: the expert outputs y, dV, dy and dU are
 * stored in bf16 between kernels, and dH where it is stored); every sum over
 * the batch in a fixed order.  bf16 with B a multiple of 64 and D, He >= 256:
 * the dH products apply GELU' in their epilogue and the batch-contracting
 * expert products read their operands as stored (no transposes of dy, H, dU
 * or W2); otherwise they read transposed copies.
 * B = 0 writes zero gradients.
 *   Workspace: rm_moe_train_workspace_bytes(B, T, D, He, E, dtype) (the same
 *   size as the forward's; the two calls may share one buffer).
 * Errors: as rm_moe_block_fwd_train; dx aliasing x or d_out -> RM_ERR_INVALID. */
rm_status rm_moe_block_bwd(const void* x, const rm_block_params* p, const void* wr_train,
                           const float* br_train, float lambda, const void* saved, size_t saved_bytes,
                           const void* d_out, void* dx, const rm_moe_grads* g, int64_t B, int T, int D,
                           int He, int E, int dtype, void* ws, size_t ws_bytes, void* stream);

/* Launch timing for benchmarks.  While enabled, every group of kernel
 * launches an entry point makes (the W1 product, the W2 product, a LayerNorm,
 * ...) is bracketed by two HIP events recorded on the caller's stream, under
 * a fixed name ("mix_ln1", "ffn1", "ffn2", "ln2", "moe_ffn1", ...).
 * rm_profile_enable(on) clears what was recorded and switches recording on or
 * off (creating events is a host-side cost; leave it off outside timing).
 * rm_profile_count() is the number of names recorded; rm_profile_read(i, ...)
 * waits for entry i's events and returns its name, the summed event-to-event
 * time in ms and the number of launch groups.  rm_profile_only(name)
 * restricts recording to the groups of that name (NULL or "": every group),
 * so a timed region can carry events around one kernel only; it persists
 * across rm_profile_enable calls.  Not thread-safe against concurrent
 * launches on other threads. */
int rm_profile_enable(int on);
int rm_profile_only(const char* name);
int rm_profile_count(void);
int rm_profile_read(int idx, char* name, size_t name_len, double* total_ms, int* launches);

/* Measurement probes: the chip's own ceilings, which bench.py reports beside
 * the data-sheet peaks (not part of the method).
 * rm_probe_mfma_bf16: eight waves per compute unit (two per SIMD) that do
 * nothing but v_mfma_f32_32x32x16_bf16, the grouped products' instruction,
 * on the random bf16 operands in `frags` (device, rm_probe_mfma_frag_bytes()
 * bytes, the caller's random bits): each wave holds 16 fragments and eight
 * 32x32 fp32 accumulators and runs iters rounds of 64 MFMAs, every MFMA on a
 * different pair of fragments; out (device, rm_probe_mfma_out_floats() fp32)
 * receives one sum per lane so nothing is optimised away.
 * rm_probe_mfma_flop(iters) is the launch's flop count (32768 per MFMA).
 * rm_probe_kstep_bf16: the grouped products' k-step on its own -- per wave
 * and k-step eight v_mfma_f32_32x32x16_bf16 on a 128 x 64 tile and the six
 * 16-byte LDS fragment reads of the next k-step, from the products' own LDS
 * layout -- with eight waves per compute unit and no DMA or barriers, for
 * iters rounds of four k-steps; `slab` (device, rm_probe_kstep_slab_bytes()
 * bytes of bf16, the caller's random values) is copied into LDS as the A and
 * W slices; out (device, rm_probe_kstep_out_floats() fp32) receives one sum
 * per lane.  rm_probe_kstep_flop(iters) is the launch's flop count.
 * rm_probe_copy: dst[0..bytes) = src[0..bytes) with 16-byte loads and stores
 * (bytes a multiple of 16; src, dst 16-byte aligned, not overlapping).
 * Errors: NULL or misaligned pointers, iters < 1 -> RM_ERR_INVALID. */
size_t rm_probe_mfma_frag_bytes(void);
int64_t rm_probe_mfma_out_floats(void);
double rm_probe_mfma_flop(int iters);
rm_status rm_probe_mfma_bf16(const void* frags, float* out, int iters, void* stream);
size_t rm_probe_kstep_slab_bytes(void);
int64_t rm_probe_kstep_out_floats(void);
double rm_probe_kstep_flop(int iters);
rm_status rm_probe_kstep_bf16(const void* slab, float* out, int iters, void* stream);
rm_status rm_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

/* How the bf16 grouped products finish a tile (bias, GELU, packing to bf16,
 * stores).  0 (the default): after the tile's main loop, by every wave of the
 * workgroup.  1: inside the next tile's main loop, four output values per
 * MFMA k-step, so the epilogue's ALU work and stores issue while the matrix
 * cores run (a deferred epilogue), for the products that qualify: dense
 * operands, a bias, bias + GELU or bias + GELU keeping the pre-activation
 * epilogue, K a multiple of 64 and at least 1024, M and N at least 256, edge
 * tiles that recompute at most 1/8 of the area; the others run as with 0.
 * Both modes compute the same products within bf16 output rounding (mode 1
 * adds the bias at the end of the tile, mode 0 starts from it).  Applies to
 * launches made after the call, process-wide.  Measured on MI355X the
 * deferred epilogue is slower (the products are power-limited, and overlap
 * does not lower a tile's energy), so 0 stays the default; mode 1 is kept
 * for measurement (bench.py --op epilogue_overlap).
 * Errors: on not 0 or 1 -> RM_ERR_INVALID.  rm_get_epilogue_overlap returns
 * the current mode. */
rm_status rm_set_epilogue_overlap(int on);
int rm_get_epilogue_overlap(void);

/* Host-side audit of what the launches would read (needs no GPU).  While
 * enabled (rm_audit_enable(1), per process), every entry point checks its
 * arguments as usual but enqueues nothing; instead, for each launch it would
 * make, it records every caller-owned buffer that launch reads -- the
 * weights, biases, LayerNorm vectors, router, logit head and the input
 * activations -- as (name, base pointer, bytes past the base the launch reads
 * at most).  The extents come from the same arguments the launch would get,
 * so a caller can check them against its allocations.  rm_audit_enable clears
 * the record; rm_audit_count() is the number of records; rm_audit_read(i,
 * ...) returns record i (RM_ERR_INVALID past the end).  Not thread-safe
 * against concurrent calls on other threads. */
int rm_audit_enable(int on);
int rm_audit_count(void);
int rm_audit_read(int idx, char* name, size_t name_len, uint64_t* base, uint64_t* bytes);

/* Text of a status code; never NULL. */
const char* rm_status_string(int status);
/* Message of the last failing call on this thread ("" if none); valid until
 * the next call on this thread. */
const char* rm_last_error(void);
/* Library version string. */
const char* rm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RANKMIXER_H */

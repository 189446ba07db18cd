// C ABI of librankmixer.so (declared in include/rankmixer.h): argument
// checks, workspace carving and kernel dispatch.  Nothing here allocates,
// frees or synchronises; every check runs before the first launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/rankmixer.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

rm_status fail(rm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

rm_status ok() {
  g_last_error.clear();
  return RM_OK;
}

rm_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return RM_OK;
}

// ---------------------------------------------------------------------------
// host-side audit (rm_audit_*): while it is on, nothing is enqueued; each
// launch site records the caller-owned buffers its launch would read and the
// bytes past their base it would read at most, from the launch's own arguments

struct AuditRec {
  std::string name;
  uint64_t base, bytes;
};
std::mutex g_audit_mu;
std::atomic<bool> g_audit{false};
std::vector<AuditRec> g_audit_recs;

bool auditing() { return g_audit.load(std::memory_order_relaxed); }

void audit(const std::string& name, const void* base, int64_t bytes) {
  if (!auditing() || !base) return;
  std::lock_guard<std::mutex> lk(g_audit_mu);
  g_audit_recs.push_back({name, (uint64_t)(uintptr_t)base, (uint64_t)(bytes > 0 ? bytes : 0)});
}

// ---------------------------------------------------------------------------
// optional launch timing (rm_profile_*): a pair of HIP events around every
// launch group, recorded on the stream the kernels go to

struct ProfEntry {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_only;  // non-empty: record only launch groups of this name
std::vector<std::string> g_prof_names;
std::map<std::string, ProfEntry> g_prof;

struct ProfScope {
  hipEvent_t a = nullptr, b = nullptr;
  hipStream_t st;
  const char* name;
  ProfScope(const char* n, hipStream_t s) : st(s), name(n) {
    if (!g_prof_on || auditing() || (!g_prof_only.empty() && g_prof_only != n)) return;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
      a = b = nullptr;
      return;
    }
    (void)hipEventRecord(a, st);
  }
  ~ProfScope() {
    if (!a) return;
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    auto it = g_prof.find(name);
    if (it == g_prof.end()) {
      g_prof_names.push_back(name);
      it = g_prof.emplace(name, ProfEntry()).first;
    }
    it->second.ev.emplace_back(a, b);
  }
};

void prof_clear() {
  for (auto& kv : g_prof)
    for (auto& e : kv.second.ev) {
      (void)hipEventDestroy(e.first);
      (void)hipEventDestroy(e.second);
    }
  g_prof.clear();
  g_prof_names.clear();
}

#define RM_TRY(expr)                     \
  do {                                   \
    const rm_status _st = (expr);        \
    if (_st != RM_OK) return _st;        \
  } while (0)

// a HIP call (launch, copy); skipped, not evaluated, while auditing
#define RM_HIP(expr, what)                                   \
  do {                                                       \
    if (!auditing()) RM_TRY(hip_status((expr), (what)));     \
  } while (0)
#define RM_PROF_CAT2(a, b) a##b
#define RM_PROF_CAT(a, b) RM_PROF_CAT2(a, b)
// time the launches of the enclosing statement under `name`
#define RM_TIMED(name, st, expr)                         \
  do {                                                   \
    ProfScope RM_PROF_CAT(_ps, __LINE__)((name), (st));  \
    expr;                                                \
  } while (0)

int elem_bytes(int dt) { return dt == RM_BF16 ? 2 : 4; }

rm_status check_ptr(const void* p, const char* name, bool required = true) {
  if (!p) return required ? fail(RM_ERR_INVALID, "%s is NULL", name) : RM_OK;
  if (reinterpret_cast<uintptr_t>(p) % 16) return fail(RM_ERR_INVALID, "%s is not 16-byte aligned", name);
  return RM_OK;
}

rm_status check_dtype(int dt) {
  if (dt != RM_F32 && dt != RM_BF16) return fail(RM_ERR_UNSUPPORTED, "unsupported dtype %d", dt);
  return RM_OK;
}

rm_status check_shape(int64_t B, int T, int D, int dt) {
  RM_TRY(check_dtype(dt));
  if (B < 0 || T <= 0 || D <= 0) return fail(RM_ERR_INVALID, "B must be >= 0, T and D positive (B=%lld T=%d D=%d)", (long long)B, T, D);
  if (D % T) return fail(RM_ERR_UNSUPPORTED, "D=%d is not divisible by H=T=%d", D, T);
  if (D % 8) return fail(RM_ERR_UNSUPPORTED, "D=%d must be a multiple of 8", D);
  if (!rm::row_width_supported(T, D, dt)) return fail(RM_ERR_UNSUPPORTED, "D=%d with T=%d is wider than the row kernels support", D, T);
  if (B * T > (int64_t)1 << 31) return fail(RM_ERR_UNSUPPORTED, "B*T too large");
  return RM_OK;
}

// shapes of the per-token FFN / MoE alone (no token mixing, so D need not
// divide by T)
rm_status check_ffn_shape(int64_t B, int T, int D, int dt) {
  RM_TRY(check_dtype(dt));
  if (B < 0 || T <= 0 || D <= 0) return fail(RM_ERR_INVALID, "B must be >= 0, T and D positive (B=%lld T=%d D=%d)", (long long)B, T, D);
  if (D % 8) return fail(RM_ERR_UNSUPPORTED, "D=%d must be a multiple of 8", D);
  if (D > 4096) return fail(RM_ERR_UNSUPPORTED, "D=%d is wider than the row kernels support (4096)", D);
  if (B * T > (int64_t)1 << 31) return fail(RM_ERR_UNSUPPORTED, "B*T too large");
  return RM_OK;
}

rm_status check_hidden(int hidden) {
  if (hidden <= 0) return fail(RM_ERR_INVALID, "hidden width must be positive (%d)", hidden);
  if (hidden % 8) return fail(RM_ERR_UNSUPPORTED, "hidden width %d must be a multiple of 8", hidden);
  return RM_OK;
}

rm_status check_moe_shape(int64_t B, int T, int E) {
  if (E < 1 || E > 32) return fail(RM_ERR_UNSUPPORTED, "E=%d experts per token (supported: 1..32)", E);
  if ((int64_t)T * E > 4096) return fail(RM_ERR_UNSUPPORTED, "T*E=%lld lists (supported: <= 4096)", (long long)T * E);
  if (B * T * E >= ((int64_t)1 << 31)) return fail(RM_ERR_UNSUPPORTED, "B*T*E too large");
  return RM_OK;
}

// One grouped product.  While auditing, it records instead how far each
// operand the launch reads extends: A rows below M per group (gathered rows
// index samples below M), or below M * G for the compacted rows of a ragged
// product; W group g at (g / b_gdiv) * b_gs, N * K elements; the bias of group
// g at g * bias_gs, N floats.
rm_status gemm_go(const char* name, const rm::GemmArgs& a, hipStream_t st) {
  if (auditing()) {
    if (a.G <= 0 || a.M <= 0 || a.N <= 0 || a.K <= 0) return RM_OK;
    const int64_t e = elem_bytes(a.dt);
    const int64_t arows = a.row_off && !a.a_rowidx ? (int64_t)a.M * a.G : a.M;
    const std::string n(name);
    const int64_t a_ext = a.a_kmajor ? ((int64_t)a.K - 1) * a.a_rs + a.M : (arows - 1) * a.a_rs + a.K;
    audit(n + ".A", a.A, (((int64_t)(a.G - 1) / a.a_gdiv) * a.a_gs + a_ext) * e);
    audit(n + ".W", a.W, (((int64_t)(a.G - 1) / a.b_gdiv) * a.b_gs + (int64_t)a.N * a.K) * e);
    if (a.bias) audit(n + ".bias", a.bias, ((int64_t)(a.G - 1) * a.bias_gs + a.N) * 4);
    return RM_OK;
  }
  return hip_status(rm::launch_gemm(a, st), name);
}

// a block's widths given as arguments must agree with its descriptor's own
// (0 there: as the argument)
rm_status check_block_dims(const rm_block_params* p, int hidden, int E) {
  if (p->hidden && p->hidden != hidden)
    return fail(RM_ERR_INVALID, "block params hidden=%d differ from the argument hidden=%d", p->hidden, hidden);
  if (p->E && p->E != E) return fail(RM_ERR_INVALID, "block params E=%d differ from the argument E=%d", p->E, E);
  return RM_OK;
}

// ---------------------------------------------------------------------------
// workspace carving: sub-buffers aligned to 256 bytes

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

constexpr int kMoeTileM = 256;  // M tile of the ragged expert products (see kernels_gemm.hip)

struct PffnWs {
  void* H;
};
size_t pffn_ws(Carver& c, int64_t B, int T, int Hd, int dt, PffnWs* w) {
  PffnWs x;
  x.H = c.take((size_t)B * T * Hd * elem_bytes(dt));
  if (w) *w = x;
  return c.off;
}

struct MoeWs {
  rm::MoeWork mw;
  void* Hc;
  void* Yc;  // gate-scaled expert outputs of the compacted rows, activation dtype
  int max_mtiles;
};
size_t moe_ws(Carver& c, int64_t B, int T, int D, int E, int He, int dt, MoeWs* w) {
  MoeWs x;
  const int64_t G = (int64_t)T * E;
  const int64_t nmax = B * G;
  x.max_mtiles = (int)(G * ((B + kMoeTileM - 1) / kMoeTileM));
  x.mw.gates = (float*)c.take(nmax * 4);
  x.mw.counts = (int*)c.take(G * 4);
  x.mw.offsets = (int*)c.take((G + 1) * 4);
  x.mw.ntiles = (int*)c.take(4);
  x.mw.tiles = (int*)c.take((size_t)x.max_mtiles * 2 * 4);
  x.mw.rows = (int*)c.take(nmax * 4);
  x.mw.gatec = (float*)c.take(nmax * 4);
  x.mw.pos = (int*)c.take(nmax * 4);
  x.Hc = c.take((size_t)nmax * He * elem_bytes(dt));
  x.Yc = c.take((size_t)nmax * D * elem_bytes(dt));
  if (w) *w = x;
  return c.off;
}

struct BlockWs {
  void* S;
  void* Z;   // W2 product + bias, activation dtype
  void* GU;  // SwiGLU: the gate | up product [T][B][2*Hs]
  PffnWs pffn;
  MoeWs moe;
};
size_t block_ws(Carver& c, int kind, int64_t B, int T, int D, int hidden, int E, int dt, BlockWs* w) {
  BlockWs x;
  x.S = c.take((size_t)B * T * D * elem_bytes(dt));
  x.GU = nullptr;
  if (kind == RM_BLOCK_DENSE || kind == RM_BLOCK_SWIGLU) {
    x.Z = c.take((size_t)B * T * D * elem_bytes(dt));
    pffn_ws(c, B, T, hidden, dt, &x.pffn);
    if (kind == RM_BLOCK_SWIGLU) x.GU = c.take((size_t)B * T * 2 * hidden * elem_bytes(dt));
  } else {
    x.Z = nullptr;
    moe_ws(c, B, T, D, E, hidden, dt, &x.moe);
  }
  if (w) *w = x;
  return c.off;
}

// ---------------------------------------------------------------------------
// launch sequences

// S row (b, t) at b * sb + t * st elements: [B][T][D] is sb = T*D, st = D; the
// block path keeps S token-major ([T][B][D]: sb = D, st = B*D) so the rows the
// W1 product reads for one token are contiguous.
rm::GemmArgs ffn1_args(const void* s, int64_t sb, int64_t st, const rm_pffn_params* p, void* H, int64_t B, int T,
                       int D, int Hd, int dt) {
  rm::GemmArgs a;
  a.dt = dt;
  a.epi = rm::kEpiBiasGelu;
  a.M = (int)B; a.N = Hd; a.K = D; a.G = T;
  a.A = s; a.a_gs = st; a.a_rs = sb;
  a.W = p->w1; a.b_gs = (int64_t)Hd * D;
  a.C = H; a.c_gs = B * Hd; a.c_rs = Hd;
  a.bias = p->b1; a.bias_gs = Hd;
  return a;
}

rm::GemmArgs ffn2_args(const void* H, const rm_pffn_params* p, int64_t B, int T, int D, int Hd, int dt) {
  rm::GemmArgs a;
  a.dt = dt;
  a.M = (int)B; a.N = D; a.K = Hd; a.G = T;
  a.A = H; a.a_gs = B * Hd; a.a_rs = Hd;
  a.W = p->w2; a.b_gs = (int64_t)D * Hd;
  a.c_gs = D; a.c_rs = (int64_t)T * D;
  a.bias = p->b2; a.bias_gs = D;
  return a;
}

rm_status run_pffn(const void* s, const rm_pffn_params* p, void* v, int64_t B, int T, int D, int Hd, int dt,
                   const PffnWs& w, hipStream_t st) {
  RM_TIMED("ffn1", st, RM_TRY(gemm_go("pffn W1 product", ffn1_args(s, (int64_t)T * D, D, p, w.H, B, T, D, Hd, dt), st)));
  rm::GemmArgs a2 = ffn2_args(w.H, p, B, T, D, Hd, dt);
  a2.epi = rm::kEpiBias;
  a2.C = v;
  RM_TIMED("ffn2", st, RM_TRY(gemm_go("pffn W2 product", a2, st)));
  return RM_OK;
}

// v = MoE(s); if ln_g: out = LN(v + s) instead.  S row (b, t) at b * sb + t * sT.
rm_status run_moe(const void* s, int64_t sb, int64_t sT, const rm_moe_params* p, void* out, float* gates_out,
                  const float* ln_g, const float* ln_b, int64_t B, int T, int D, int E, int He, int dt, MoeWs w,
                  hipStream_t st) {
  if (gates_out) w.mw.gates = gates_out;
  const int64_t e = elem_bytes(dt);
  audit("moe_router.wr", p->wr, (int64_t)T * E * D * e);
  audit("moe_router.br", p->br, (int64_t)T * E * 4);
  RM_TIMED("moe_router", st, RM_HIP(rm::launch_moe_router(s, sb, sT, p->wr, p->br, w.mw.gates, B, T, D, E, dt, st), "moe router"));
  RM_TIMED("moe_compact", st, RM_HIP(rm::launch_moe_compact(w.mw, B, T, E, kMoeTileM, st), "moe compaction"));
  const int G = T * E;
  rm::GemmArgs a;
  a.dt = dt;
  a.epi = rm::kEpiBiasGelu;
  a.M = (int)B; a.N = He; a.K = D; a.G = G;
  a.A = s; a.a_gdiv = E; a.a_gs = sT; a.a_rs = sb; a.a_rowidx = w.mw.rows;
  a.W = p->w1; a.b_gs = (int64_t)He * D;
  a.C = w.Hc; a.c_gs = 0; a.c_rs = He;
  a.bias = p->b1; a.bias_gs = He;
  a.row_off = w.mw.offsets; a.tiles = w.mw.tiles; a.ntiles = w.mw.ntiles; a.max_mtiles = w.max_mtiles;
  if (rm::gemm_tile_m(a) != kMoeTileM) return fail(RM_ERR_HIP, "internal: MoE tile size mismatch");
  RM_TIMED("moe_ffn1", st, RM_TRY(gemm_go("moe W1 product", a, st)));
  rm::GemmArgs b;
  b.dt = dt;
  b.epi = rm::kEpiBiasScale;
  b.M = (int)B; b.N = D; b.K = He; b.G = G;
  b.A = w.Hc; b.a_gs = 0; b.a_rs = He;
  b.W = p->w2; b.b_gs = (int64_t)D * He;
  b.C = w.Yc; b.c_gs = 0; b.c_rs = D;
  b.bias = p->b2; b.bias_gs = D;
  b.rowscale = w.mw.gatec;
  b.row_off = w.mw.offsets; b.tiles = w.mw.tiles; b.ntiles = w.mw.ntiles; b.max_mtiles = w.max_mtiles;
  if (rm::gemm_tile_m(b) != kMoeTileM) return fail(RM_ERR_HIP, "internal: MoE tile size mismatch");
  RM_TIMED("moe_ffn2", st, RM_TRY(gemm_go("moe W2 product", b, st)));
  audit("moe_combine.ln_g", ln_g, (int64_t)D * 4);
  audit("moe_combine.ln_b", ln_b, (int64_t)D * 4);
  RM_TIMED("moe_combine", st,
           RM_HIP(rm::launch_moe_combine(w.Yc, w.mw.pos, s, sb, sT, ln_g, ln_b, out, B, T, D, E, ln_g != nullptr, dt, st),
                  "moe combine"));
  return RM_OK;
}

rm_status check_block_params(const rm_block_params* p, int dt) {
  if (!p) return fail(RM_ERR_INVALID, "block params is NULL");
  RM_TRY(check_ptr(p->ln1_g, "ln1_g")); RM_TRY(check_ptr(p->ln1_b, "ln1_b"));
  RM_TRY(check_ptr(p->ln2_g, "ln2_g")); RM_TRY(check_ptr(p->ln2_b, "ln2_b"));
  if (p->flags & ~RM_BLOCK_NO_MIX_NORM) return fail(RM_ERR_UNSUPPORTED, "unknown block flags %d", p->flags);
  if (p->kind == RM_BLOCK_DENSE || p->kind == RM_BLOCK_SWIGLU) {
    RM_TRY(check_ptr(p->pffn.w1, "pffn.w1")); RM_TRY(check_ptr(p->pffn.b1, "pffn.b1"));
    RM_TRY(check_ptr(p->pffn.w2, "pffn.w2")); RM_TRY(check_ptr(p->pffn.b2, "pffn.b2"));
  } else if (p->kind == RM_BLOCK_MOE) {
    RM_TRY(check_ptr(p->moe.wr, "moe.wr")); RM_TRY(check_ptr(p->moe.br, "moe.br"));
    RM_TRY(check_ptr(p->moe.w1, "moe.w1")); RM_TRY(check_ptr(p->moe.b1, "moe.b1"));
    RM_TRY(check_ptr(p->moe.w2, "moe.w2")); RM_TRY(check_ptr(p->moe.b2, "moe.b2"));
  } else {
    return fail(RM_ERR_UNSUPPORTED, "unknown block kind %d", p->kind);
  }
  (void)dt;
  return RM_OK;
}

rm_status check_block_shape(int kind, int64_t B, int T, int D, int hidden, int E, int dt) {
  RM_TRY(check_shape(B, T, D, dt));
  RM_TRY(check_hidden(hidden));
  if (kind == RM_BLOCK_MOE) {
    RM_TRY(check_moe_shape(B, T, E));
    if (D > 4096) return fail(RM_ERR_UNSUPPORTED, "D=%d is wider than the MoE row kernels support (4096)", D);
  }
  return RM_OK;
}

// One block X -> xo.  s_given: S = LN1(TM(X) + X) is already in w.S
// (token-major; x is not read).  next: instead of LN2 into xo, run the block
// boundary, which leaves the next block's S in w.S (the block's output is not
// materialised); the caller checks fusable_boundary first.
rm_status run_block(const void* x, const rm_block_params* p, void* xo, int64_t B, int T, int D, int hidden,
                    int E, int dt, const BlockWs& w, hipStream_t st, bool s_given = false,
                    const rm_block_params* next = nullptr) {
  int64_t sb, sT;  // S row (b, t) at b * sb + t * sT
  if (s_given) {
    sb = D;
    sT = B * D;
  } else if (p->flags & RM_BLOCK_NO_MIX_NORM) {
    // S = TM(X), [B][T][D]
    audit("mix.x", x, B * T * D * (int64_t)elem_bytes(dt));
    RM_TIMED("mix", st, RM_HIP(rm::launch_token_mix(x, w.S, B, T, D, dt, st), "token mix"));
    sb = (int64_t)T * D;
    sT = D;
  } else {
    // S = LN1(TM(X) + X), token-major so one token's rows are contiguous
    audit("mix_ln1.x", x, B * T * D * (int64_t)elem_bytes(dt));
    audit("mix_ln1.ln1_g", p->ln1_g, (int64_t)D * 4);
    audit("mix_ln1.ln1_b", p->ln1_b, (int64_t)D * 4);
    RM_TIMED("mix_ln1", st, RM_HIP(rm::launch_mix_ln(x, w.S, p->ln1_g, p->ln1_b, B, T, D, dt, true, st), "token mix + LayerNorm"));
    sb = D;
    sT = B * D;
  }
  if (p->kind == RM_BLOCK_DENSE || p->kind == RM_BLOCK_SWIGLU) {
    if (p->kind == RM_BLOCK_DENSE) {
      RM_TIMED("ffn1", st, RM_TRY(gemm_go("block W1 product", ffn1_args(w.S, sb, sT, &p->pffn, w.pffn.H, B, T, D, hidden, dt), st)));
    } else {
      // one product over the gate and up rows (N = 2*Hs); on the pipelined
      // kernel its epilogue pairs them and writes H = SiLU(G) * U directly,
      // otherwise the product writes [G | U] and a pointwise pass combines
      rm::GemmArgs a1 = ffn1_args(w.S, sb, sT, &p->pffn, w.pffn.H, B, T, D, 2 * hidden, dt);
      a1.c_gs = B * hidden;
      a1.c_rs = hidden;
      a1.epi = rm::kEpiSwiglu;
      if (rm::gemm_pipe_eligible(a1)) {
        RM_TIMED("ffn1", st, RM_TRY(gemm_go("block gate / up product + SwiGLU", a1, st)));
      } else {
        a1 = ffn1_args(w.S, sb, sT, &p->pffn, w.GU, B, T, D, 2 * hidden, dt);
        a1.epi = rm::kEpiBias;
        RM_TIMED("ffn1", st, RM_TRY(gemm_go("block gate / up product", a1, st)));
        RM_TIMED("swiglu", st, RM_HIP(rm::launch_swiglu_ew(w.GU, w.pffn.H, B * T, hidden, dt, st), "SwiGLU"));
      }
    }
    rm::GemmArgs a2 = ffn2_args(w.pffn.H, &p->pffn, B, T, D, hidden, dt);
    // Z = W2 product + bias in the activation dtype; the residual S is added
    // inside LayerNorm 2 (fp32 arithmetic), which streams Z anyway, instead of
    // by loads in the product's epilogue
    a2.epi = rm::kEpiBias;
    a2.C = w.Z;
    RM_TIMED("ffn2", st, RM_TRY(gemm_go("block W2 product", a2, st)));
    if (next) {
      audit("ln2_mix_ln1.ln2_g", p->ln2_g, (int64_t)D * 4);
      audit("ln2_mix_ln1.ln2_b", p->ln2_b, (int64_t)D * 4);
      audit("ln2_mix_ln1.ln1_g", next->ln1_g, (int64_t)D * 4);
      audit("ln2_mix_ln1.ln1_b", next->ln1_b, (int64_t)D * 4);
      RM_TIMED("ln2_mix_ln1", st, RM_HIP(rm::launch_ln_mix_ln(w.Z, w.S, p->ln2_g, p->ln2_b, next->ln1_g, next->ln1_b,
                                                              B, T, D, dt, st),
                                         "LayerNorm 2 + next block's token mix + LayerNorm 1"));
      return RM_OK;
    }
    audit("ln2.ln2_g", p->ln2_g, (int64_t)D * 4);
    audit("ln2.ln2_b", p->ln2_b, (int64_t)D * 4);
    RM_TIMED("ln2", st, RM_HIP(rm::launch_ln_rows(w.Z, w.S, sb, sT, T, xo, p->ln2_g, p->ln2_b, B * T, D, dt, st),
                               "residual + LayerNorm 2"));
    return RM_OK;
  }
  return run_moe(w.S, sb, sT, &p->moe, xo, nullptr, p->ln2_g, p->ln2_b, B, T, D, E, hidden, dt, w.moe, st);
}

// whether block l's LN2 and block l + 1's mix + LN1 run as one boundary pass
// (block l a dense or SwiGLU block, neither block without the Add & Norm
// after the mix, and the sample's T rows fit in LDS)
bool fusable_boundary(const rm_model_desc* m, int l) {
  if (l + 1 >= m->L) return false;
  const rm_block_params& a = m->blocks[l];
  const rm_block_params& b = m->blocks[l + 1];
  return (a.kind == RM_BLOCK_DENSE || a.kind == RM_BLOCK_SWIGLU) && a.flags == 0 && b.flags == 0 &&
         rm::ln_mix_ln_supported(m->T, m->D, m->dtype);
}

// Two [B][T][D] ping-pong buffers, then one block region large enough for
// the largest block of the stack, each block sized from its own kind, hidden
// width and expert count; every block carves its own layout from the region's
// start (S first, so a boundary pass can leave the next block's S there).
size_t model_ws(Carver& c, const rm_model_desc* m, int64_t B, void** x0, void** x1, void** blk) {
  const size_t xb = (size_t)B * m->T * m->D * elem_bytes(m->dtype);
  void* a = c.take(xb);
  void* b = c.take(xb);
  if (x0) *x0 = a;
  if (x1) *x1 = b;
  size_t best = 0;
  for (int l = 0; l < m->L; ++l) {
    const rm_block_params& p = m->blocks[l];
    Carver probe(nullptr);
    best = std::max(best, block_ws(probe, p.kind, B, m->T, m->D, p.hidden, p.E, m->dtype, nullptr));
  }
  void* r = c.take(best);
  if (blk) *blk = r;
  return c.off;
}

}  // namespace

// ===========================================================================
extern "C" {

const char* rm_status_string(int st) {
  switch (st) {
    case RM_OK: return "ok";
    case RM_ERR_INVALID: return "invalid argument";
    case RM_ERR_UNSUPPORTED: return "unsupported shape or type";
    case RM_ERR_WORKSPACE: return "workspace too small";
    case RM_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* rm_last_error(void) { return g_last_error.c_str(); }

#ifndef RM_SRC_HASH
#define RM_SRC_HASH "unknown"
#endif
// the build passes the hash of the sources it compiled
const char* rm_version(void) { return "rankmixer-mi355x 0.2 (gfx950) src " RM_SRC_HASH; }

size_t rm_probe_mfma_frag_bytes(void) { return (size_t)rm::kProbeFragBytes; }

int64_t rm_probe_mfma_out_floats(void) { return (int64_t)rm::probe_mfma_waves() * 64; }

double rm_probe_mfma_flop(int iters) { return (double)rm::probe_mfma_waves() * iters * 64 * 32768.0; }

rm_status rm_probe_mfma_bf16(const void* frags, float* out, int iters, void* stream) {
  RM_TRY(check_ptr(frags, "frags"));
  RM_TRY(check_ptr(out, "out"));
  if (iters < 1) return fail(RM_ERR_INVALID, "iters=%d must be positive", iters);
  RM_HIP(rm::launch_probe_mfma(frags, out, iters, (hipStream_t)stream), "MFMA probe");
  return ok();
}

size_t rm_probe_kstep_slab_bytes(void) { return (size_t)rm::kProbeSlabBytes; }

int64_t rm_probe_kstep_out_floats(void) { return (int64_t)rm::probe_kstep_blocks() * 512; }

double rm_probe_kstep_flop(int iters) { return (double)rm::probe_kstep_blocks() * 8 * iters * 32 * 32768.0; }

rm_status rm_probe_kstep_bf16(const void* slab, float* out, int iters, void* stream) {
  RM_TRY(check_ptr(slab, "slab"));
  RM_TRY(check_ptr(out, "out"));
  if (iters < 1) return fail(RM_ERR_INVALID, "iters=%d must be positive", iters);
  RM_HIP(rm::launch_probe_kstep(slab, out, iters, (hipStream_t)stream), "k-step probe");
  return ok();
}

rm_status rm_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  RM_TRY(check_ptr(src, "src"));
  RM_TRY(check_ptr(dst, "dst"));
  if (bytes % 16) return fail(RM_ERR_INVALID, "bytes=%zu must be a multiple of 16", bytes);
  const char *a = (const char*)src, *b = (const char*)dst;
  if (a < b + bytes && b < a + bytes) return fail(RM_ERR_INVALID, "src and dst overlap");
  if (bytes) RM_HIP(rm::launch_probe_copy(src, dst, (long long)(bytes / 16), (hipStream_t)stream), "copy probe");
  return ok();
}

rm_status rm_set_epilogue_overlap(int on) {
  if (on != 0 && on != 1) return fail(RM_ERR_INVALID, "epilogue overlap mode must be 0 or 1 (%d)", on);
  rm::set_epilogue_overlap(on);
  return ok();
}

int rm_get_epilogue_overlap(void) { return rm::epilogue_overlap() ? 1 : 0; }

int rm_audit_enable(int on) {
  std::lock_guard<std::mutex> lk(g_audit_mu);
  g_audit_recs.clear();
  g_audit.store(on != 0, std::memory_order_relaxed);
  return RM_OK;
}

int rm_audit_count(void) {
  std::lock_guard<std::mutex> lk(g_audit_mu);
  return (int)g_audit_recs.size();
}

int rm_audit_read(int idx, char* name, size_t name_len, uint64_t* base, uint64_t* bytes) {
  std::lock_guard<std::mutex> lk(g_audit_mu);
  if (idx < 0 || idx >= (int)g_audit_recs.size() || !name || !base || !bytes)
    return fail(RM_ERR_INVALID, "audit record %d does not exist", idx);
  snprintf(name, name_len, "%s", g_audit_recs[idx].name.c_str());
  *base = g_audit_recs[idx].base;
  *bytes = g_audit_recs[idx].bytes;
  return RM_OK;
}

int rm_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  prof_clear();
  g_prof_on = on != 0;
  return RM_OK;
}

int rm_profile_only(const char* name) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = name ? name : "";
  return RM_OK;
}

int rm_profile_count(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  return (int)g_prof_names.size();
}

int rm_profile_read(int idx, char* name, size_t name_len, double* total_ms, int* launches) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (idx < 0 || idx >= (int)g_prof_names.size() || !name || !total_ms || !launches)
    return fail(RM_ERR_INVALID, "profile entry %d does not exist", idx);
  const std::string& n = g_prof_names[idx];
  snprintf(name, name_len, "%s", n.c_str());
  double tot = 0.0;
  for (auto& e : g_prof[n].ev) {
    RM_HIP(hipEventSynchronize(e.second), "profile event");
    float ms = 0.f;
    RM_HIP(hipEventElapsedTime(&ms, e.first, e.second), "profile event");
    tot += ms;
  }
  *total_ms = tot;
  *launches = (int)g_prof[n].ev.size();
  return RM_OK;
}

rm_status rm_tokenize_padsplit(const float* emb, int64_t B, int64_t F, int T, int D, int out_dtype, void* x0,
                               void* stream) {
  RM_TRY(check_dtype(out_dtype));
  if (B < 0 || F <= 0 || T <= 0 || D <= 0) return fail(RM_ERR_INVALID, "B must be >= 0, F, T, D positive");
  if (F > (int64_t)T * D) return fail(RM_ERR_UNSUPPORTED, "F=%lld floats do not fit in T*D=%lld", (long long)F, (long long)T * D);
  if (B == 0) return ok();  // empty batch: nothing to do
  RM_TRY(check_ptr(emb, "emb"));
  RM_TRY(check_ptr(x0, "x0"));
  audit("tokenize.emb", emb, B * F * 4);
  RM_TIMED("tokenize", (hipStream_t)stream, RM_HIP(rm::launch_tokenize_padsplit(emb, B, F, T, D, out_dtype, x0, (hipStream_t)stream), "tokenize"));
  return ok();
}

// bf16 with whole float4 segments of the embedding: one fused launch that
// reads the fp32 embedding in place; otherwise pad-split into the workspace
// (token width seg) and one grouped product over the padded copy
static bool project_fused(int64_t F, int seg, int dtype) {
  return dtype == RM_BF16 && F % 4 == 0 && seg <= rm::tokenize_project_max_seg();
}

size_t rm_tokenize_project_workspace_bytes(int64_t B, int64_t F, int T, int seg, int dtype) {
  if (project_fused(F, seg, dtype) || B <= 0) return 0;
  Carver c(nullptr);
  c.take((size_t)B * T * seg * elem_bytes(dtype));
  return c.off;
}

// Group t maps segment rows (stride F in place, or T*seg in the padded copy)
// through W_t [D][seg] into x0's token-t rows (stride T*D), b_t added in the
// epilogue.
rm_status rm_tokenize_project(const float* emb, const rm_proj_params* p, int64_t B, int64_t F, int T, int seg,
                              int D, int dtype, void* x0, void* ws, size_t ws_bytes, void* stream) {
  RM_TRY(check_dtype(dtype));
  if (B < 0 || F <= 0 || T <= 0 || seg <= 0 || D <= 0)
    return fail(RM_ERR_INVALID, "B must be >= 0, F, T, seg, D positive");
  if (F > (int64_t)T * seg)
    return fail(RM_ERR_UNSUPPORTED, "F=%lld floats do not fit in T*seg=%lld", (long long)F, (long long)T * seg);
  if (seg % 8) return fail(RM_ERR_UNSUPPORTED, "seg=%d must be a multiple of 8", seg);
  if (D % 8) return fail(RM_ERR_UNSUPPORTED, "D=%d must be a multiple of 8", D);
  if (B * T > (int64_t)1 << 31 || B > INT32_MAX) return fail(RM_ERR_UNSUPPORTED, "B*T too large");
  if (B == 0) return ok();
  if (!p) return fail(RM_ERR_INVALID, "params is NULL");
  RM_TRY(check_ptr(emb, "emb"));
  RM_TRY(check_ptr(p->w, "w")); RM_TRY(check_ptr(p->b, "b"));
  RM_TRY(check_ptr(x0, "x0"));
  const bool fused = project_fused(F, seg, dtype);
  const size_t need = rm_tokenize_project_workspace_bytes(B, F, T, seg, dtype);
  if (need) RM_TRY(check_ptr(ws, "ws"));
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  audit("tokenize.emb", emb, B * F * 4);
  if (fused) {
    audit("tokenize_proj.W", p->w, (int64_t)T * D * seg * elem_bytes(dtype));
    audit("tokenize_proj.bias", p->b, (int64_t)T * D * 4);
    RM_TIMED("tokenize_proj", st,
             RM_HIP(rm::launch_tokenize_project(emb, p->w, p->b, x0, B, F, T, seg, D, st), "tokenize projection"));
    return ok();
  }
  RM_TIMED("tokenize", st, RM_HIP(rm::launch_tokenize_padsplit(emb, B, F, T, seg, dtype, ws, st), "tokenize pad-split"));
  rm::GemmArgs a;
  a.dt = dtype;
  a.epi = rm::kEpiBias;
  a.M = (int)B; a.N = D; a.K = seg; a.G = T;
  a.A = ws; a.a_gs = seg; a.a_rs = (int64_t)T * seg;
  a.W = p->w; a.b_gs = (int64_t)D * seg;
  a.C = x0; a.c_gs = D; a.c_rs = (int64_t)T * D;
  a.bias = p->b; a.bias_gs = D;
  RM_TIMED("tokenize_proj", st, RM_TRY(gemm_go("tokenize projection", a, st)));
  return ok();
}

rm_status rm_token_mix(const void* x, void* y, int64_t B, int T, int D, int dtype, void* stream) {
  RM_TRY(check_dtype(dtype));
  if (B < 0 || T <= 0 || D <= 0) return fail(RM_ERR_INVALID, "B must be >= 0, T and D positive");
  if (D % T) return fail(RM_ERR_UNSUPPORTED, "D=%d is not divisible by H=T=%d", D, T);
  if (B == 0) return ok();
  RM_TRY(check_ptr(x, "x"));
  RM_TRY(check_ptr(y, "y"));
  if (x == y) return fail(RM_ERR_INVALID, "y must not alias x");
  audit("token_mix.x", x, B * T * D * (int64_t)elem_bytes(dtype));
  RM_TIMED("token_mix", (hipStream_t)stream, RM_HIP(rm::launch_token_mix(x, y, B, T, D, dtype, (hipStream_t)stream), "token mix"));
  return ok();
}

size_t rm_pffn_workspace_bytes(int64_t B, int T, int D, int Hd, int dtype) {
  (void)D;
  Carver c(nullptr);
  return pffn_ws(c, B, T, Hd, dtype, nullptr);
}

rm_status rm_pffn_fwd(const void* s, const rm_pffn_params* p, void* v, int64_t B, int T, int D, int Hd, int dtype,
                      void* ws, size_t ws_bytes, void* stream) {
  RM_TRY(check_ffn_shape(B, T, D, dtype));
  RM_TRY(check_hidden(Hd));
  if (B == 0) return ok();
  if (!p) return fail(RM_ERR_INVALID, "params is NULL");
  RM_TRY(check_ptr(s, "s")); RM_TRY(check_ptr(v, "v"));
  RM_TRY(check_ptr(p->w1, "w1")); RM_TRY(check_ptr(p->b1, "b1"));
  RM_TRY(check_ptr(p->w2, "w2")); RM_TRY(check_ptr(p->b2, "b2"));
  if (s == v) return fail(RM_ERR_INVALID, "v must not alias s");
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_pffn_workspace_bytes(B, T, D, Hd, dtype);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  Carver c(ws);
  PffnWs w;
  pffn_ws(c, B, T, Hd, dtype, &w);
  RM_TRY(run_pffn(s, p, v, B, T, D, Hd, dtype, w, (hipStream_t)stream));
  return ok();
}

size_t rm_moe_workspace_bytes(int64_t B, int T, int D, int E, int He, int dtype) {
  Carver c(nullptr);
  return moe_ws(c, B, T, D, E, He, dtype, nullptr);
}

static rm_status check_moe_params(const rm_moe_params* p) {
  if (!p) return fail(RM_ERR_INVALID, "params is NULL");
  RM_TRY(check_ptr(p->wr, "wr")); RM_TRY(check_ptr(p->br, "br"));
  RM_TRY(check_ptr(p->w1, "w1")); RM_TRY(check_ptr(p->b1, "b1"));
  RM_TRY(check_ptr(p->w2, "w2")); RM_TRY(check_ptr(p->b2, "b2"));
  return RM_OK;
}

rm_status rm_moe_relu_fwd(const void* s, const rm_moe_params* p, void* v, float* gates, int64_t B, int T, int D,
                          int E, int He, int dtype, void* ws, size_t ws_bytes, void* stream) {
  RM_TRY(check_ffn_shape(B, T, D, dtype));
  RM_TRY(check_hidden(He));
  RM_TRY(check_moe_shape(B, T, E));
  if (B == 0) return ok();
  RM_TRY(check_moe_params(p));
  RM_TRY(check_ptr(s, "s")); RM_TRY(check_ptr(v, "v")); RM_TRY(check_ptr(gates, "gates", false));
  if (s == v) return fail(RM_ERR_INVALID, "v must not alias s");
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_moe_workspace_bytes(B, T, D, E, He, dtype);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  Carver c(ws);
  MoeWs w;
  moe_ws(c, B, T, D, E, He, dtype, &w);
  RM_TRY(run_moe(s, (int64_t)T * D, D, p, v, gates, nullptr, nullptr, B, T, D, E, He, dtype, w, (hipStream_t)stream));
  return ok();
}

rm_status rm_moe_route(const void* s, const void* wr, const float* br, float* gates, int* offsets, int* rows,
                       int64_t B, int T, int D, int E, int dtype, void* ws, size_t ws_bytes, void* stream) {
  RM_TRY(check_ffn_shape(B, T, D, dtype));
  RM_TRY(check_moe_shape(B, T, E));
  if (B == 0) return ok();
  RM_TRY(check_ptr(s, "s")); RM_TRY(check_ptr(wr, "wr")); RM_TRY(check_ptr(br, "br"));
  RM_TRY(check_ptr(gates, "gates")); RM_TRY(check_ptr(offsets, "offsets")); RM_TRY(check_ptr(rows, "rows"));
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_moe_workspace_bytes(B, T, D, E, 8, dtype);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  Carver c(ws);
  MoeWs w;
  moe_ws(c, B, T, D, E, 8, dtype, &w);
  w.mw.gates = gates;
  w.mw.offsets = offsets;
  w.mw.rows = rows;
  hipStream_t st = (hipStream_t)stream;
  audit("moe_router.s", s, B * T * D * (int64_t)elem_bytes(dtype));
  audit("moe_router.wr", wr, (int64_t)T * E * D * elem_bytes(dtype));
  audit("moe_router.br", br, (int64_t)T * E * 4);
  RM_HIP(rm::launch_moe_router(s, (int64_t)T * D, D, wr, br, gates, B, T, D, E, dtype, st), "moe router");
  RM_HIP(rm::launch_moe_compact(w.mw, B, T, E, kMoeTileM, st), "moe compaction");
  return ok();
}

// ---------------------------------------------------------------------------
// rm_moe_route_noalloc: the routing step with its scratch (per-list counts,
// the tile list and its length, the compacted gates and the (b, t, j) ->
// entry map) in a fixed device array instead of a caller workspace.  Every
// scratch element the call reads is written earlier in the same call, so
// nothing is cleared between calls.

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> that device's copy of `scratch`

// the current device's address of `scratch`, looked up once per device
rm_status scratch_base(void** out) {
  int dev = -1;
  RM_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    RM_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return RM_OK;
}

size_t route_scratch(Carver& c, int64_t B, int T, int E, rm::MoeWork* w) {
  const int64_t G = (int64_t)T * E;
  const int64_t nmax = B * G;
  rm::MoeWork x{};
  x.counts = (int*)c.take(G * 4);
  x.ntiles = (int*)c.take(4);
  x.tiles = (int*)c.take((size_t)(G * ((B + kMoeTileM - 1) / kMoeTileM)) * 2 * 4);
  x.gatec = (float*)c.take(nmax * 4);
  x.pos = (int*)c.take(nmax * 4);
  if (w) *w = x;
  return c.off;
}

}  // namespace

size_t rm_moe_route_noalloc_scratch_bytes(int64_t B, int T, int E) {
  if (B < 0 || T <= 0 || E <= 0) return 0;
  Carver c(nullptr);
  return route_scratch(c, B, T, E, nullptr);
}

size_t rm_moe_route_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

rm_status rm_moe_route_noalloc(const void* s, const void* wr, const float* br, float* gates, int* offsets, int* rows,
                               int64_t B, int T, int D, int E, int dtype, void* stream) {
  RM_TRY(check_ffn_shape(B, T, D, dtype));
  RM_TRY(check_moe_shape(B, T, E));
  if (B == 0) return ok();
  RM_TRY(check_ptr(s, "s")); RM_TRY(check_ptr(wr, "wr")); RM_TRY(check_ptr(br, "br"));
  RM_TRY(check_ptr(gates, "gates")); RM_TRY(check_ptr(offsets, "offsets")); RM_TRY(check_ptr(rows, "rows"));
  const size_t need = rm_moe_route_noalloc_scratch_bytes(B, T, E);
  if (need > kNoAllocScratchBytes)
    return fail(RM_ERR_UNSUPPORTED, "B*T*E = %lld needs %zu bytes of scratch, more than the fixed %zu",
                (long long)(B * T * E), need, kNoAllocScratchBytes);
  void* base = nullptr;
  if (!auditing()) RM_TRY(scratch_base(&base));
  Carver c(base);
  rm::MoeWork w;
  route_scratch(c, B, T, E, &w);
  w.gates = gates;
  w.offsets = offsets;
  w.rows = rows;
  hipStream_t st = (hipStream_t)stream;
  audit("moe_router.s", s, B * T * D * (int64_t)elem_bytes(dtype));
  audit("moe_router.wr", wr, (int64_t)T * E * D * elem_bytes(dtype));
  audit("moe_router.br", br, (int64_t)T * E * 4);
  RM_HIP(rm::launch_moe_router(s, (int64_t)T * D, D, wr, br, gates, B, T, D, E, dtype, st), "moe router");
  RM_HIP(rm::launch_moe_compact(w, B, T, E, kMoeTileM, st), "moe compaction");
  return ok();
}

size_t rm_block_workspace_bytes(int kind, int64_t B, int T, int D, int hidden, int E, int dtype) {
  Carver c(nullptr);
  return block_ws(c, kind, B, T, D, hidden, E, dtype, nullptr);
}

rm_status rm_block_fwd(const void* x, const rm_block_params* p, void* x_out, int64_t B, int T, int D, int hidden,
                       int E, int dtype, void* ws, size_t ws_bytes, void* stream) {
  RM_TRY(check_block_params(p, dtype));
  RM_TRY(check_block_dims(p, hidden, E));
  RM_TRY(check_block_shape(p->kind, B, T, D, hidden, E, dtype));
  if (B == 0) return ok();
  RM_TRY(check_ptr(x, "x")); RM_TRY(check_ptr(x_out, "x_out"));
  if (x == x_out) return fail(RM_ERR_INVALID, "x_out must not alias x");
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_block_workspace_bytes(p->kind, B, T, D, hidden, E, dtype);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  Carver c(ws);
  BlockWs w;
  block_ws(c, p->kind, B, T, D, hidden, E, dtype, &w);
  RM_TRY(run_block(x, p, x_out, B, T, D, hidden, E, dtype, w, (hipStream_t)stream));
  return ok();
}

// ---------------------------------------------------------------------------
// dense block training forward and backward

namespace {

// what the training forward keeps for the backward: S (token-major), U (the
// W1 product + b1 before GELU, token-major [T][B][Hd]) and Z (the W2 product +
// b2, [B][T][D])
struct Saved {
  void* S;  // [T][B][D] token-major
  void* U;  // [T][B][Hd] W1 product + b1
  void* H;  // [T][B][Hd] GELU(U)
  void* Z;  // [T][B][D] W2 product + b2
};
size_t saved_carve(Carver& c, int64_t B, int T, int D, int Hd, int dt, Saved* w) {
  Saved x;
  x.S = c.take((size_t)B * T * D * elem_bytes(dt));
  x.U = c.take((size_t)B * T * Hd * elem_bytes(dt));
  x.H = c.take((size_t)B * T * Hd * elem_bytes(dt));
  x.Z = c.take((size_t)B * T * D * elem_bytes(dt));
  if (w) *w = x;
  return c.off;
}

int64_t pad64(int64_t v) { return (v + 63) / 64 * 64; }

// workspace of the backward; the K = batch products read the transposed
// activations with rows padded to Bp = B rounded up to 64 (zero tail)
// The products of the dense backward.  dH = dV W2 reads W2_t [D][Hd] as a
// K-major W; with kmajor (below) its epilogue also applies GELU'(U) and
// writes dU plus the b1 partial sums.  dW2 = dV^T H and dW1 = dU^T S
// contract over the batch: with kmajor both operands are read as they are
// (token-major [B][.] per token = K-major), else from transposes padded to
// Bp rows.
rm::GemmArgs bwd_dH_args(const void* dV, const void* w2, void* C, int64_t B, int T, int D, int Hd, int dt) {
  rm::GemmArgs g;
  g.dt = dt; g.epi = rm::kEpiBias;
  g.M = (int)B; g.N = Hd; g.K = D; g.G = T;
  g.A = dV; g.a_gs = B * D; g.a_rs = D;
  g.W = w2; g.b_gs = (int64_t)Hd * D; g.w_kmajor = 1;
  g.C = C; g.c_gs = B * Hd; g.c_rs = Hd;
  return g;
}
rm::GemmArgs bwd_dW_args(const void* A, int M, const void* W, int N, void* C, int64_t B, int T, int dt) {
  rm::GemmArgs g;
  g.dt = dt; g.epi = rm::kEpiBiasF32;
  g.M = M; g.N = N; g.K = (int)B; g.G = T;
  g.A = A; g.a_gs = B * M; g.a_rs = M; g.a_kmajor = 1;
  g.W = W; g.b_gs = B * N; g.w_kmajor = 1;
  g.C = C; g.c_gs = (int64_t)M * N; g.c_rs = N;
  return g;
}
// dS (W1 branch) = dU W1 (fp32, token-major): W1_t [Hd][D] read K-major
rm::GemmArgs bwd_dS_args(const void* dU, const void* w1, float* C, int64_t B, int T, int D, int Hd, int dt) {
  rm::GemmArgs g;
  g.dt = dt; g.epi = rm::kEpiBiasF32;
  g.M = (int)B; g.N = D; g.K = Hd; g.G = T;
  g.A = dU; g.a_gs = B * Hd; g.a_rs = Hd;
  g.W = w1; g.b_gs = (int64_t)D * Hd; g.w_kmajor = 1;
  g.C = C; g.c_gs = B * D; g.c_rs = D;
  return g;
}
// whether the backward runs without transposes (a shape property)
bool bwd_kmajor(int64_t B, int T, int D, int Hd, int dt) {
  rm::GemmArgs h = bwd_dH_args(nullptr, nullptr, nullptr, B, T, D, Hd, dt);
  h.epi = rm::kEpiGeluBwd;
  return rm::gemm_kmajor_eligible(h) && rm::gemm_kmajor_eligible(bwd_dW_args(nullptr, D, nullptr, Hd, nullptr, B, T, dt)) &&
         rm::gemm_kmajor_eligible(bwd_dW_args(nullptr, Hd, nullptr, D, nullptr, B, T, dt));
}

struct BwdWs {
  bool km;  // bwd_kmajor
  void *dV, *dVt, *W2t, *dH, *dU, *dUt, *Ht, *St, *W1t;
  float *dSf, *dY1, *ln2p, *ln1p, *b2p, *b1p;
  int b2_parts, b1_parts;  // partial sums per token of b2, b1
};
size_t bwd_carve(Carver& c, int64_t B, int T, int D, int Hd, int dt, BwdWs* w) {
  const size_t e = elem_bytes(dt);
  const int64_t Bp = pad64(B);
  const int64_t rt = rm::transpose_row_tiles(B, Bp);
  const int lg = rm::ln_bwd_grid(B, T, D);
  BwdWs x{};
  x.km = bwd_kmajor(B, T, D, Hd, dt);
  if (x.km) {
    x.b2_parts = rm::colsum64_parts(B);
    x.b1_parts = rm::gemm_colsum_parts((int)B);
    x.dV = c.take((size_t)T * B * D * e);
    x.dU = c.take((size_t)T * B * Hd * e);
    // W1^T only where the dS product cannot read W1 as stored
    x.W1t = rm::gemm_wt_eligible(bwd_dS_args(nullptr, nullptr, nullptr, B, T, D, Hd, dt))
                ? nullptr : c.take((size_t)T * D * Hd * e);
    x.dSf = (float*)c.take((size_t)T * B * D * 4);
    x.dY1 = (float*)c.take((size_t)B * T * D * 4);
    x.ln2p = (float*)c.take((size_t)lg * 2 * D * 4);
    x.ln1p = (float*)c.take((size_t)lg * 2 * D * 4);
    x.b2p = (float*)c.take((size_t)T * x.b2_parts * D * 4);
    x.b1p = (float*)c.take((size_t)T * x.b1_parts * Hd * 4);
    if (w) *w = x;
    return c.off;
  }
  x.b2_parts = x.b1_parts = (int)rt;
  x.dV = c.take((size_t)T * B * D * e);
  x.dVt = c.take((size_t)T * D * Bp * e);
  x.W2t = c.take((size_t)T * Hd * D * e);
  x.dH = c.take((size_t)T * B * Hd * e);
  x.dU = c.take((size_t)T * B * Hd * e);
  x.dUt = c.take((size_t)T * Hd * Bp * e);
  x.Ht = c.take((size_t)T * Hd * Bp * e);
  x.St = c.take((size_t)T * D * Bp * e);
  x.W1t = c.take((size_t)T * D * Hd * e);
  x.dSf = (float*)c.take((size_t)T * B * D * 4);
  x.dY1 = (float*)c.take((size_t)B * T * D * 4);
  x.ln2p = (float*)c.take((size_t)lg * 2 * D * 4);
  x.ln1p = (float*)c.take((size_t)lg * 2 * D * 4);
  x.b2p = (float*)c.take((size_t)T * rt * D * 4);
  x.b1p = (float*)c.take((size_t)T * rt * Hd * 4);
  if (w) *w = x;
  return c.off;
}

rm_status check_train_shape(const rm_block_params* p, int64_t B, int T, int D, int hidden, int dt) {
  RM_TRY(check_block_params(p, dt));
  RM_TRY(check_block_dims(p, hidden, 0));
  if (p->kind != RM_BLOCK_DENSE || p->flags)
    return fail(RM_ERR_UNSUPPORTED, "training supports dense blocks (GELU FFN, Add & Norm after the mix) only");
  RM_TRY(check_block_shape(RM_BLOCK_DENSE, B, T, D, hidden, 0, dt));
  if (D > rm::ln_bwd_max_width())
    return fail(RM_ERR_UNSUPPORTED, "D=%d is wider than the backward row kernels support (%d)", D, rm::ln_bwd_max_width());
  if (B * T * (int64_t)hidden >= ((int64_t)1 << 31) || (int64_t)T * pad64(B) * hidden >= ((int64_t)1 << 31))
    return fail(RM_ERR_UNSUPPORTED, "B*T*hidden too large");
  return RM_OK;
}

}  // namespace

size_t rm_block_saved_bytes(int64_t B, int T, int D, int hidden, int dtype) {
  Carver c(nullptr);
  return saved_carve(c, B, T, D, hidden, dtype, nullptr);
}

rm_status rm_block_fwd_train(const void* x, const rm_block_params* p, void* x_out, void* saved, size_t saved_bytes,
                             int64_t B, int T, int D, int hidden, int dtype, void* ws, size_t ws_bytes, void* stream) {
  RM_TRY(check_train_shape(p, B, T, D, hidden, dtype));
  if (B == 0) return ok();
  RM_TRY(check_ptr(x, "x")); RM_TRY(check_ptr(x_out, "x_out"));
  if (x == x_out) return fail(RM_ERR_INVALID, "x_out must not alias x");
  RM_TRY(check_ptr(saved, "saved"));
  const size_t need_s = rm_block_saved_bytes(B, T, D, hidden, dtype);
  if (saved_bytes < need_s) return fail(RM_ERR_WORKSPACE, "saved buffer %zu bytes, need %zu", saved_bytes, need_s);
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_block_workspace_bytes(RM_BLOCK_DENSE, B, T, D, hidden, 0, dtype);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  Carver cs(saved);
  Saved sv;
  saved_carve(cs, B, T, D, hidden, dtype, &sv);
  Carver c(ws);
  BlockWs w;
  block_ws(c, RM_BLOCK_DENSE, B, T, D, hidden, 0, dtype, &w);
  const int64_t sb = D, sT = B * D;  // S is token-major
  audit("mix_ln1.x", x, B * T * D * (int64_t)elem_bytes(dtype));
  audit("mix_ln1.ln1_g", p->ln1_g, (int64_t)D * 4);
  audit("mix_ln1.ln1_b", p->ln1_b, (int64_t)D * 4);
  audit("ln2.ln2_g", p->ln2_g, (int64_t)D * 4);
  audit("ln2.ln2_b", p->ln2_b, (int64_t)D * 4);
  RM_TIMED("mix_ln1", st, RM_HIP(rm::launch_mix_ln(x, sv.S, p->ln1_g, p->ln1_b, B, T, D, dtype, true, st), "token mix + LayerNorm"));
  // keep U = W1 s + b1 (saved) and H = GELU(U): both from the product's
  // epilogue on the pipelined kernel, else a separate GELU pass
  rm::GemmArgs a1 = ffn1_args(sv.S, sb, sT, &p->pffn, sv.U, B, T, D, hidden, dtype);
  a1.epi = rm::kEpiBiasGeluDual;
  a1.C2 = sv.H;
  if (rm::gemm_pipe_eligible(a1)) {
    RM_TIMED("ffn1", st, RM_TRY(gemm_go("block W1 product + GELU", a1, st)));
  } else {
    a1.epi = rm::kEpiBias;
    RM_TIMED("ffn1", st, RM_TRY(gemm_go("block W1 product", a1, st)));
    RM_TIMED("gelu", st, RM_HIP(rm::launch_gelu_ew(sv.U, sv.H, B * T * (int64_t)hidden, dtype, st), "GELU"));
  }
  rm::GemmArgs a2 = ffn2_args(sv.H, &p->pffn, B, T, D, hidden, dtype);
  a2.epi = rm::kEpiBias;
  a2.C = sv.Z;
  RM_TIMED("ffn2", st, RM_TRY(gemm_go("block W2 product", a2, st)));
  RM_TIMED("ln2", st, RM_HIP(rm::launch_ln_rows(sv.Z, sv.S, sb, sT, T, x_out, p->ln2_g, p->ln2_b, B * T, D, dtype, st),
                             "residual + LayerNorm 2"));
  return ok();
}

size_t rm_block_bwd_workspace_bytes(int64_t B, int T, int D, int hidden, int dtype) {
  Carver c(nullptr);
  return bwd_carve(c, B, T, D, hidden, dtype, nullptr);
}

rm_status rm_block_bwd(const void* x, const rm_block_params* p, const void* saved, size_t saved_bytes, const void* d_out,
                       void* dx, const rm_block_grads* g, int64_t B, int T, int D, int hidden, int dtype, void* ws,
                       size_t ws_bytes, void* stream) {
  RM_TRY(check_train_shape(p, B, T, D, hidden, dtype));
  if (!g) return fail(RM_ERR_INVALID, "grads is NULL");
  RM_TRY(check_ptr(g->w1, "grads.w1")); RM_TRY(check_ptr(g->b1, "grads.b1"));
  RM_TRY(check_ptr(g->w2, "grads.w2")); RM_TRY(check_ptr(g->b2, "grads.b2"));
  RM_TRY(check_ptr(g->ln1_g, "grads.ln1_g")); RM_TRY(check_ptr(g->ln1_b, "grads.ln1_b"));
  RM_TRY(check_ptr(g->ln2_g, "grads.ln2_g")); RM_TRY(check_ptr(g->ln2_b, "grads.ln2_b"));
  hipStream_t st = (hipStream_t)stream;
  const int Hd = hidden;
  if (B == 0) {
    // an empty batch contributes nothing: every gradient is zero (a sum over
    // no partials, written by a kernel rather than a memset)
    const struct { float* p; int64_t n; } z[] = {{g->w1, (int64_t)T * Hd * D}, {g->b1, (int64_t)T * Hd},
                                                 {g->w2, (int64_t)T * D * Hd}, {g->b2, (int64_t)T * D},
                                                 {g->ln1_g, D}, {g->ln1_b, D}, {g->ln2_g, D}, {g->ln2_b, D}};
    for (const auto& v : z) RM_HIP(rm::launch_sum_parts(v.p, v.p, nullptr, 1, 0, v.n, v.n, st), "zero grads");
    return ok();
  }
  RM_TRY(check_ptr(x, "x")); RM_TRY(check_ptr(d_out, "d_out")); RM_TRY(check_ptr(dx, "dx"));
  if (dx == x || dx == d_out) return fail(RM_ERR_INVALID, "dx must not alias x or d_out");
  RM_TRY(check_ptr(saved, "saved"));
  const size_t need_s = rm_block_saved_bytes(B, T, D, hidden, dtype);
  if (saved_bytes < need_s) return fail(RM_ERR_WORKSPACE, "saved buffer %zu bytes, need %zu", saved_bytes, need_s);
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_block_bwd_workspace_bytes(B, T, D, hidden, dtype);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  Carver cs(const_cast<void*>(saved));
  Saved sv;
  saved_carve(cs, B, T, D, hidden, dtype, &sv);
  Carver c(ws);
  BwdWs w;
  bwd_carve(c, B, T, D, hidden, dtype, &w);
  const int dt = dtype;
  const int64_t Bp = pad64(B);
  const int lg = rm::ln_bwd_grid(B, T, D);
  audit("ln_bwd.x", x, B * T * D * (int64_t)elem_bytes(dt));
  audit("ln_bwd.d_out", d_out, B * T * D * (int64_t)elem_bytes(dt));
  audit("ln_bwd.ln2_g", p->ln2_g, (int64_t)D * 4);
  audit("ln_bwd.ln1_g", p->ln1_g, (int64_t)D * 4);
  // X' = LN2(Z + S): dV = dY2 (token-major), gamma2 / beta2 partials
  RM_TIMED("ln2_bwd", st, RM_HIP(rm::launch_ln_bwd(0, d_out, nullptr, nullptr, sv.Z, sv.S, p->ln2_g, w.dV, w.ln2p, B, T, D, dt, st), "LayerNorm 2 backward"));
  if (w.km) {
    // b2 partials: column sums of dV over 64-row blocks
    RM_TIMED("sums_dV", st, RM_HIP(rm::launch_colsum64(w.dV, w.b2p, T, B, D, dt, st), "dV column sums"));
    // dU = (dV W2) * GELU'(U) from the product's epilogue, with the b1 partials
    rm::GemmArgs g1 = bwd_dH_args(w.dV, p->pffn.w2, w.dU, B, T, D, Hd, dt);
    g1.epi = rm::kEpiGeluBwd;
    g1.aux = sv.U;
    g1.colsum = w.b1p;
    RM_TIMED("bwd_dH", st, RM_TRY(gemm_go("dH product + GELU backward", g1, st)));
    // dW2 = dV^T H and dW1 = dU^T S (fp32), both operands read as stored
    RM_TIMED("bwd_dW2", st, RM_TRY(gemm_go("dW2 product", bwd_dW_args(w.dV, D, sv.H, Hd, g->w2, B, T, dt), st)));
    RM_TIMED("bwd_dW1", st, RM_TRY(gemm_go("dW1 product", bwd_dW_args(w.dU, Hd, sv.S, D, g->w1, B, T, dt), st)));
  } else {
    // dV^T (rows padded to Bp) and the b2 partials
    RM_TIMED("tr_dV", st, RM_HIP(rm::launch_transpose(0, w.dV, nullptr, w.dVt, nullptr, nullptr, w.b2p, T, B, D, Bp, dt, st), "transpose dV"));
    // dH = dV W2: W2_t [D][Hd] is the product's W read K-major where the
    // kernel allows, else W2^T [T][Hd][D] first
    rm::GemmArgs g1 = bwd_dH_args(w.dV, p->pffn.w2, w.dH, B, T, D, Hd, dt);
    if (!rm::gemm_wt_eligible(g1)) {
      audit("tr_W2.W", p->pffn.w2, (int64_t)T * D * Hd * elem_bytes(dt));
      RM_TIMED("tr_W2", st, RM_HIP(rm::launch_transpose(0, p->pffn.w2, nullptr, w.W2t, nullptr, nullptr, nullptr, T, D, Hd, D, dt, st), "transpose W2"));
      g1.W = w.W2t;
      g1.w_kmajor = 0;
    }
    RM_TIMED("bwd_dH", st, RM_TRY(gemm_go("dH product", g1, st)));
    // dU = dH * GELU'(U), also transposed, with the b1 partials, and H^T
    // from the saved GELU(U)
    RM_TIMED("gelu_bwd", st, RM_HIP(rm::launch_transpose(2, w.dH, sv.U, w.dUt, w.dU, w.Ht, w.b1p, T, B, Hd, Bp, dt, st), "GELU backward"));
    // dW2 = dV^T H (fp32)
    rm::GemmArgs g2;
    g2.dt = dt; g2.epi = rm::kEpiBiasF32;
    g2.M = D; g2.N = Hd; g2.K = (int)Bp; g2.G = T;
    g2.A = w.dVt; g2.a_gs = (int64_t)D * Bp; g2.a_rs = Bp;
    g2.W = w.Ht; g2.b_gs = (int64_t)Hd * Bp;
    g2.C = g->w2; g2.c_gs = (int64_t)D * Hd; g2.c_rs = Hd;
    RM_TIMED("bwd_dW2", st, RM_TRY(gemm_go("dW2 product", g2, st)));
    // dW1 = dU^T S (fp32)
    RM_TIMED("tr_S", st, RM_HIP(rm::launch_transpose(0, sv.S, nullptr, w.St, nullptr, nullptr, nullptr, T, B, D, Bp, dt, st), "transpose S"));
    rm::GemmArgs g3;
    g3.dt = dt; g3.epi = rm::kEpiBiasF32;
    g3.M = Hd; g3.N = D; g3.K = (int)Bp; g3.G = T;
    g3.A = w.dUt; g3.a_gs = (int64_t)Hd * Bp; g3.a_rs = Bp;
    g3.W = w.St; g3.b_gs = (int64_t)D * Bp;
    g3.C = g->w1; g3.c_gs = (int64_t)Hd * D; g3.c_rs = D;
    RM_TIMED("bwd_dW1", st, RM_TRY(gemm_go("dW1 product", g3, st)));
  }
  // dS (W1 branch) = dU W1 (fp32, token-major): W1_t [Hd][D] read K-major
  // where the kernel allows, else W1^T first
  rm::GemmArgs g4 = bwd_dS_args(w.dU, p->pffn.w1, w.dSf, B, T, D, Hd, dt);
  if (!rm::gemm_wt_eligible(g4)) {
    audit("tr_W1.W", p->pffn.w1, (int64_t)T * Hd * D * elem_bytes(dt));
    RM_TIMED("tr_W1", st, RM_HIP(rm::launch_transpose(0, p->pffn.w1, nullptr, w.W1t, nullptr, nullptr, nullptr, T, Hd, D, Hd, dt, st), "transpose W1"));
    g4.W = w.W1t;
    g4.w_kmajor = 0;
  }
  RM_TIMED("bwd_dS", st, RM_TRY(gemm_go("dS product", g4, st)));
  // S = LN1(TM(X) + X) with dS = dV + dS_ffn; dX = dY1 + TM(dY1)
  RM_TIMED("ln1_bwd", st, RM_HIP(rm::launch_ln_bwd(1, nullptr, w.dV, w.dSf, x, nullptr, p->ln1_g, w.dY1, w.ln1p, B, T, D, dt, st), "LayerNorm 1 backward"));
  RM_TIMED("tm_add", st, RM_HIP(rm::launch_tm_add(w.dY1, dx, B, T, D, dt, st), "token mix backward"));
  // fixed-order sums of the partials
  RM_TIMED("sums_ln", st, RM_HIP(rm::launch_sum_parts(w.ln2p, g->ln2_g, g->ln2_b, 1, lg, 2 * (int64_t)D, D, st), "gamma2 / beta2"));
  RM_TIMED("sums_ln", st, RM_HIP(rm::launch_sum_parts(w.ln1p, g->ln1_g, g->ln1_b, 1, lg, 2 * (int64_t)D, D, st), "gamma1 / beta1"));
  RM_TIMED("sums_bias", st, RM_HIP(rm::launch_sum_parts(w.b2p, g->b2, nullptr, T, w.b2_parts, D, D, st), "b2"));
  RM_TIMED("sums_bias", st, RM_HIP(rm::launch_sum_parts(w.b1p, g->b1, nullptr, T, w.b1_parts, Hd, Hd, st), "b1"));
  return ok();
}

// ---------------------------------------------------------------------------
// MoE block training with the dense-training / sparse-inference routers

namespace {

struct MoeSaved {
  void* S;   // [T][B][D] token-major
  void* U;   // [T*E][B][He]: W1 product + b1 of every (token, expert), group-major
  void* H;   // [T*E][B][He]: GELU(U)
  void* Y;   // [B][T*E][D]: expert outputs
  float* Gt; // [B][T][E] training gates
  float* Gi; // [B][T][E] inference gates
  void* Z;   // [B][T][D]: sum_j G_train y_j
};
size_t moe_saved_carve(Carver& c, int64_t B, int T, int D, int E, int He, int dt, MoeSaved* w) {
  const size_t e = elem_bytes(dt);
  const int64_t TE = (int64_t)T * E;
  MoeSaved x;
  x.S = c.take((size_t)B * T * D * e);
  x.U = c.take((size_t)B * TE * He * e);
  x.H = c.take((size_t)B * TE * He * e);
  x.Y = c.take((size_t)B * TE * D * e);
  x.Gt = (float*)c.take((size_t)B * TE * 4);
  x.Gi = (float*)c.take((size_t)B * TE * 4);
  x.Z = c.take((size_t)B * T * D * e);
  if (w) *w = x;
  return c.off;
}

// The MoE backward's expert products over the T*E groups (dy, U, H
// group-major [T*E][B][.]; dU [B][T][E*He]): dH = dy W2 reads W2 K-major and,
// on the transpose-free path, applies GELU'(U) in its epilogue (writing dU
// and the b1 partials); dW2 = dy^T H and dW1 = dU^T S then read both operands
// as stored.
rm::GemmArgs moe_dH_args(const void* dy, const void* w2, void* C, int64_t B, int64_t TE, int D, int He, int dt) {
  rm::GemmArgs g;
  g.dt = dt; g.epi = rm::kEpiGeluBwd;
  g.M = (int)B; g.N = He; g.K = D; g.G = (int)TE;
  g.A = dy; g.a_gs = B * D; g.a_rs = D;
  g.W = w2; g.b_gs = (int64_t)He * D; g.w_kmajor = 1;
  g.C = C; g.c_gs = He; g.c_rs = TE * He;   // dU [B][T][E*He]
  g.aux_gs = B * He; g.aux_rs = He;          // U [T*E][B][He]
  return g;
}
rm::GemmArgs moe_dW2_args(const void* dy, const void* H, float* C, int64_t B, int64_t TE, int D, int He, int dt) {
  rm::GemmArgs g = bwd_dW_args(dy, D, H, He, C, B, (int)TE, dt);
  return g;
}
rm::GemmArgs moe_dW1_args(const void* dU, const void* S, float* C, int64_t B, int T, int E, int D, int He, int dt) {
  const int64_t TE = (int64_t)T * E;
  rm::GemmArgs g = bwd_dW_args(dU, He, S, D, C, B, (int)TE, dt);
  g.a_gs = He; g.a_rs = TE * He;  // dU [B][T][E*He]: group g's column block
  g.b_gdiv = E;                    // S per token
  return g;
}
// dS per token over the E experts' hidden units (dU [B][T][E*He]; W1 of
// token t, [E*He][D] as stored, is the K-major W)
rm::GemmArgs moe_dS_args(const void* dU, const void* w1, float* C, int64_t B, int T, int D, int E, int He, int dt) {
  rm::GemmArgs g;
  g.dt = dt; g.epi = rm::kEpiBiasF32;
  g.M = (int)B; g.N = D; g.K = E * He; g.G = T;
  g.A = dU; g.a_gs = (int64_t)E * He; g.a_rs = (int64_t)T * E * He;
  g.W = w1; g.b_gs = (int64_t)D * E * He; g.w_kmajor = 1;
  g.C = C; g.c_gs = B * D; g.c_rs = D;
  return g;
}
bool moe_bwd_kmajor(int64_t B, int T, int D, int E, int He, int dt) {
  const int64_t TE = (int64_t)T * E;
  return rm::gemm_kmajor_eligible(moe_dH_args(nullptr, nullptr, nullptr, B, TE, D, He, dt)) &&
         rm::gemm_kmajor_eligible(moe_dW2_args(nullptr, nullptr, nullptr, B, TE, D, He, dt)) &&
         rm::gemm_kmajor_eligible(moe_dW1_args(nullptr, nullptr, nullptr, B, T, E, D, He, dt));
}

// group-major [T*E][B][*]: dy, dH (so each (token, expert) slice is
// contiguous for its product and its transpose); dU [B][T][E*He] (one K axis
// over a token's experts for the dS product)
struct MoeTrainWs {
  bool km;  // moe_bwd_kmajor
  void *dV, *dy, *dz, *mask, *W2t, *dH, *dU, *dUt, *Ht, *dyt, *St, *W1tc, *dzt, *maskt;
  float *dSr, *dSf, *dY1, *ln2p, *ln1p, *b2p, *b1p, *brtp, *brip, *lpart;
  int b2_parts, b1_parts;  // partial sums per group of b2, b1
};
size_t moe_train_carve(Carver& c, int64_t B, int T, int D, int E, int He, int dt, MoeTrainWs* w) {
  const size_t e = elem_bytes(dt);
  const int64_t TE = (int64_t)T * E, Bp = pad64(B);
  const int64_t rt = rm::transpose_row_tiles(B, Bp);
  const int lg = rm::ln_bwd_grid(B, T, D);
  MoeTrainWs x{};
  x.km = moe_bwd_kmajor(B, T, D, E, He, dt);
  x.b2_parts = x.km ? rm::colsum64_parts(B) : (int)rt;
  x.b1_parts = x.km ? rm::gemm_colsum_parts((int)B) : (int)rt;
  x.dV = c.take((size_t)T * B * D * e);
  x.dy = c.take((size_t)B * TE * D * e);
  x.dz = c.take((size_t)B * TE * e);
  x.mask = c.take((size_t)B * TE * e);
  x.dU = c.take((size_t)B * TE * He * e);
  if (!x.km) {
    x.W2t = c.take((size_t)TE * He * D * e);
    x.dH = c.take((size_t)B * TE * He * e);
    x.dUt = c.take((size_t)TE * He * Bp * e);
    x.Ht = c.take((size_t)TE * He * Bp * e);
    x.dyt = c.take((size_t)TE * D * Bp * e);
  }
  x.St = c.take((size_t)T * D * Bp * e);
  if (!rm::gemm_wt_eligible(moe_dS_args(nullptr, nullptr, nullptr, B, T, D, E, He, dt)))
    x.W1tc = c.take((size_t)T * D * E * He * e);
  x.dzt = c.take((size_t)TE * Bp * e);
  x.maskt = c.take((size_t)TE * Bp * e);
  x.dSr = (float*)c.take((size_t)T * B * D * 4);
  x.dSf = (float*)c.take((size_t)T * B * D * 4);
  x.dY1 = (float*)c.take((size_t)B * T * D * 4);
  x.ln2p = (float*)c.take((size_t)lg * 2 * D * 4);
  x.ln1p = (float*)c.take((size_t)lg * 2 * D * 4);
  x.b2p = (float*)c.take((size_t)TE * x.b2_parts * D * 4);
  x.b1p = (float*)c.take((size_t)TE * x.b1_parts * He * 4);
  x.brtp = (float*)c.take((size_t)rt * TE * 4);
  x.brip = (float*)c.take((size_t)rt * TE * 4);
  x.lpart = (float*)c.take((size_t)rm::kSumParts * 4);
  if (w) *w = x;
  return c.off;
}

rm_status check_moe_train(const rm_block_params* p, const void* wr_train, const float* br_train, int64_t B, int T,
                          int D, int He, int E, int dt) {
  RM_TRY(check_block_params(p, dt));
  RM_TRY(check_block_dims(p, He, E));
  if (p->kind != RM_BLOCK_MOE || p->flags)
    return fail(RM_ERR_UNSUPPORTED, "MoE training needs an MoE block with the Add & Norm after the mix");
  RM_TRY(check_block_shape(RM_BLOCK_MOE, B, T, D, He, E, dt));
  RM_TRY(check_ptr(wr_train, "wr_train")); RM_TRY(check_ptr(br_train, "br_train"));
  if (D > rm::ln_bwd_max_width())
    return fail(RM_ERR_UNSUPPORTED, "D=%d is wider than the backward row kernels support (%d)", D, rm::ln_bwd_max_width());
  if (((int64_t)T * E) % 8) return fail(RM_ERR_UNSUPPORTED, "T*E=%lld must be a multiple of 8", (long long)T * E);
  const int64_t TE = (int64_t)T * E;
  if (B * TE * He >= ((int64_t)1 << 31) || TE * pad64(B) * He >= ((int64_t)1 << 31) || B * TE * D >= ((int64_t)1 << 31))
    return fail(RM_ERR_UNSUPPORTED, "B*T*E*hidden too large");
  return RM_OK;
}

}  // namespace

size_t rm_moe_saved_bytes(int64_t B, int T, int D, int He, int E, int dtype) {
  Carver c(nullptr);
  return moe_saved_carve(c, B, T, D, E, He, dtype, nullptr);
}

size_t rm_moe_train_workspace_bytes(int64_t B, int T, int D, int He, int E, int dtype) {
  Carver c(nullptr);
  return moe_train_carve(c, B, T, D, E, He, dtype, nullptr);
}

rm_status rm_moe_block_fwd_train(const void* x, const rm_block_params* p, const void* wr_train, const float* br_train,
                                 void* x_out, float* l_reg, void* saved, size_t saved_bytes, int64_t B, int T, int D,
                                 int He, int E, int dtype, void* ws, size_t ws_bytes, void* stream) {
  RM_TRY(check_moe_train(p, wr_train, br_train, B, T, D, He, E, dtype));
  RM_TRY(check_ptr(l_reg, "l_reg"));
  hipStream_t st = (hipStream_t)stream;
  if (B == 0) {
    RM_HIP(rm::launch_sum_parts(l_reg, l_reg, nullptr, 1, 0, 1, 1, st), "zero loss");
    return ok();
  }
  RM_TRY(check_ptr(x, "x")); RM_TRY(check_ptr(x_out, "x_out"));
  if (x == x_out) return fail(RM_ERR_INVALID, "x_out must not alias x");
  RM_TRY(check_ptr(saved, "saved"));
  const size_t need_s = rm_moe_saved_bytes(B, T, D, He, E, dtype);
  if (saved_bytes < need_s) return fail(RM_ERR_WORKSPACE, "saved buffer %zu bytes, need %zu", saved_bytes, need_s);
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_moe_train_workspace_bytes(B, T, D, He, E, dtype);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  const int dt = dtype;
  const int64_t TE = (int64_t)T * E;
  Carver cs(saved);
  MoeSaved sv;
  moe_saved_carve(cs, B, T, D, E, He, dt, &sv);
  Carver c(ws);
  MoeTrainWs w;
  moe_train_carve(c, B, T, D, E, He, dt, &w);
  // S = LN1(TM(X) + X), token-major
  RM_TIMED("mix_ln1", st, RM_HIP(rm::launch_mix_ln(x, sv.S, p->ln1_g, p->ln1_b, B, T, D, dt, true, st), "token mix + LayerNorm"));
  // both routers' gates; the sparsity loss sums the inference gates
  audit("mix_ln1.x", x, B * T * D * (int64_t)elem_bytes(dt));
  audit("mix_ln1.ln1_g", p->ln1_g, (int64_t)D * 4);
  audit("mix_ln1.ln1_b", p->ln1_b, (int64_t)D * 4);
  audit("router.wr_train", wr_train, (int64_t)T * E * D * elem_bytes(dt));
  audit("router.br_train", br_train, (int64_t)T * E * 4);
  audit("router.wr", p->moe.wr, (int64_t)T * E * D * elem_bytes(dt));
  audit("router.br", p->moe.br, (int64_t)T * E * 4);
  audit("ln2.ln2_g", p->ln2_g, (int64_t)D * 4);
  audit("ln2.ln2_b", p->ln2_b, (int64_t)D * 4);
  RM_TIMED("router", st, RM_HIP(rm::launch_moe_router(sv.S, D, B * D, wr_train, br_train, sv.Gt, B, T, D, E, dt, st), "training router"));
  RM_TIMED("router", st, RM_HIP(rm::launch_moe_router(sv.S, D, B * D, p->moe.wr, p->moe.br, sv.Gi, B, T, D, E, dt, st), "inference router"));
  RM_TIMED("l_reg", st, RM_HIP(rm::launch_sum_all(sv.Gi, l_reg, B * TE, w.lpart, st), "sparsity loss"));
  // every expert densely: U = S W1^T + b1 over T*E groups (S shared by a token's experts)
  rm::GemmArgs a1;
  a1.dt = dt; a1.epi = rm::kEpiBias;
  a1.M = (int)B; a1.N = He; a1.K = D; a1.G = (int)TE;
  a1.A = sv.S; a1.a_gs = B * D; a1.a_rs = D; a1.a_gdiv = E;
  a1.W = p->moe.w1; a1.b_gs = (int64_t)He * D;
  a1.C = sv.U; a1.c_gs = B * He; a1.c_rs = He;
  a1.bias = p->moe.b1; a1.bias_gs = He;
  a1.epi = rm::kEpiBiasGeluDual;  // U (saved) and H = GELU(U) from one epilogue where the kernel allows
  a1.C2 = sv.H;
  if (rm::gemm_pipe_eligible(a1)) {
    RM_TIMED("moe_ffn1", st, RM_TRY(gemm_go("expert W1 products + GELU", a1, st)));
  } else {
    a1.epi = rm::kEpiBias;
    RM_TIMED("moe_ffn1", st, RM_TRY(gemm_go("expert W1 products", a1, st)));
    RM_TIMED("gelu", st, RM_HIP(rm::launch_gelu_ew(sv.U, sv.H, B * TE * He, dt, st), "GELU"));
  }
  rm::GemmArgs a2;
  a2.dt = dt; a2.epi = rm::kEpiBias;
  a2.M = (int)B; a2.N = D; a2.K = He; a2.G = (int)TE;
  a2.A = sv.H; a2.a_gs = B * He; a2.a_rs = He;
  a2.W = p->moe.w2; a2.b_gs = (int64_t)D * He;
  a2.C = sv.Y; a2.c_gs = D; a2.c_rs = TE * D;
  a2.bias = p->moe.b2; a2.bias_gs = D;
  RM_TIMED("moe_ffn2", st, RM_TRY(gemm_go("expert W2 products", a2, st)));
  // Z = sum_j G_train y_j, then X' = LN2(Z + S)
  RM_TIMED("combine", st, RM_HIP(rm::launch_moe_combine_dense(sv.Y, sv.Gt, sv.Z, B * T, E, D, dt, st), "expert combine"));
  RM_TIMED("ln2", st, RM_HIP(rm::launch_ln_rows(sv.Z, sv.S, D, B * D, T, x_out, p->ln2_g, p->ln2_b, B * T, D, dt, st),
                             "residual + LayerNorm 2"));
  return ok();
}

rm_status rm_moe_block_bwd(const void* x, const rm_block_params* p, const void* wr_train, const float* br_train,
                           float lambda, const void* saved, size_t saved_bytes, const void* d_out, void* dx,
                           const rm_moe_grads* g, int64_t B, int T, int D, int He, int E, int dtype, void* ws,
                           size_t ws_bytes, void* stream) {
  RM_TRY(check_moe_train(p, wr_train, br_train, B, T, D, He, E, dtype));
  if (!g) return fail(RM_ERR_INVALID, "grads is NULL");
  const struct { float* p; const char* n; int64_t len; } outs[] = {
      {g->w1, "grads.w1", (int64_t)T * E * He * D}, {g->b1, "grads.b1", (int64_t)T * E * He},
      {g->w2, "grads.w2", (int64_t)T * E * D * He}, {g->b2, "grads.b2", (int64_t)T * E * D},
      {g->wr_train, "grads.wr_train", (int64_t)T * E * D}, {g->br_train, "grads.br_train", (int64_t)T * E},
      {g->wr_infer, "grads.wr_infer", (int64_t)T * E * D}, {g->br_infer, "grads.br_infer", (int64_t)T * E},
      {g->ln1_g, "grads.ln1_g", D}, {g->ln1_b, "grads.ln1_b", D}, {g->ln2_g, "grads.ln2_g", D}, {g->ln2_b, "grads.ln2_b", D}};
  for (const auto& o : outs) RM_TRY(check_ptr(o.p, o.n));
  hipStream_t st = (hipStream_t)stream;
  if (B == 0) {
    for (const auto& o : outs) RM_HIP(rm::launch_sum_parts(o.p, o.p, nullptr, 1, 0, o.len, o.len, st), "zero grads");
    return ok();
  }
  RM_TRY(check_ptr(x, "x")); RM_TRY(check_ptr(d_out, "d_out")); RM_TRY(check_ptr(dx, "dx"));
  if (dx == x || dx == d_out) return fail(RM_ERR_INVALID, "dx must not alias x or d_out");
  RM_TRY(check_ptr(saved, "saved"));
  const size_t need_s = rm_moe_saved_bytes(B, T, D, He, E, dtype);
  if (saved_bytes < need_s) return fail(RM_ERR_WORKSPACE, "saved buffer %zu bytes, need %zu", saved_bytes, need_s);
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_moe_train_workspace_bytes(B, T, D, He, E, dtype);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  const int dt = dtype;
  const int64_t TE = (int64_t)T * E, Bp = pad64(B);
  const int rt = rm::transpose_row_tiles(B, Bp);
  const int lg = rm::ln_bwd_grid(B, T, D);
  Carver cs(const_cast<void*>(saved));
  MoeSaved sv;
  moe_saved_carve(cs, B, T, D, E, He, dt, &sv);
  Carver c(ws);
  MoeTrainWs w;
  moe_train_carve(c, B, T, D, E, He, dt, &w);
  // X' = LN2(Z + S): dV = dY2 (token-major)
  RM_TIMED("ln2_bwd", st, RM_HIP(rm::launch_ln_bwd(0, d_out, nullptr, nullptr, sv.Z, sv.S, p->ln2_g, w.dV, w.ln2p, B, T, D, dt, st), "LayerNorm 2 backward"));
  // gates: dy = G_train dV, dz (training router), mask (inference router), router input gradient
  audit("ln_bwd.x", x, B * T * D * (int64_t)elem_bytes(dt));
  audit("ln_bwd.d_out", d_out, B * T * D * (int64_t)elem_bytes(dt));
  audit("ln_bwd.ln2_g", p->ln2_g, (int64_t)D * 4);
  audit("ln_bwd.ln1_g", p->ln1_g, (int64_t)D * 4);
  audit("moe_rows.wr_train", wr_train, (int64_t)T * E * D * elem_bytes(dt));
  audit("tr_W2.W", p->moe.w2, TE * D * He * elem_bytes(dt));
  audit("tr_W1.W", p->moe.w1, TE * He * D * elem_bytes(dt));
  RM_TIMED("moe_rows", st, RM_HIP(rm::launch_moe_bwd_rows(w.dV, sv.Y, sv.Gt, sv.Gi, wr_train, w.dy, w.dz, w.mask, w.dSr, B, T, E, D, dt, st), "gate backward"));
  // experts, densely over the T*E groups
  if (w.km) {
    // b2 partials from dy; dU = (dy W2) * GELU'(U) from the dH product's
    // epilogue with the b1 partials; dW2 = dy^T H and dW1 = dU^T S read their
    // operands as stored
    RM_TIMED("sums_dy", st, RM_HIP(rm::launch_colsum64(w.dy, w.b2p, (int)TE, B, D, dt, st), "dy column sums"));
    rm::GemmArgs g1 = moe_dH_args(w.dy, p->moe.w2, w.dU, B, TE, D, He, dt);
    g1.aux = sv.U;
    g1.colsum = w.b1p;
    RM_TIMED("bwd_dH", st, RM_TRY(gemm_go("expert dH products + GELU backward", g1, st)));
    RM_TIMED("bwd_dW2", st, RM_TRY(gemm_go("expert dW2 products", moe_dW2_args(w.dy, sv.H, g->w2, B, TE, D, He, dt), st)));
    RM_TIMED("tr_S", st, RM_HIP(rm::launch_transpose(0, sv.S, nullptr, w.St, nullptr, nullptr, nullptr, T, B, D, Bp, dt, st), "transpose S"));
    RM_TIMED("bwd_dW1", st, RM_TRY(gemm_go("expert dW1 products", moe_dW1_args(w.dU, sv.S, g->w1, B, T, E, D, He, dt), st)));
  } else {
    RM_TIMED("tr_W2", st, RM_HIP(rm::launch_transpose(0, p->moe.w2, nullptr, w.W2t, nullptr, nullptr, nullptr, (int)TE, D, He, D, dt, st), "transpose W2"));
    rm::GemmArgs g1;
    g1.dt = dt; g1.epi = rm::kEpiBias;
    g1.M = (int)B; g1.N = He; g1.K = D; g1.G = (int)TE;
    g1.A = w.dy; g1.a_gs = B * D; g1.a_rs = D;
    g1.W = w.W2t; g1.b_gs = (int64_t)He * D;
    g1.C = w.dH; g1.c_gs = B * He; g1.c_rs = He;
    RM_TIMED("bwd_dH", st, RM_TRY(gemm_go("expert dH products", g1, st)));
    // dH and U are group-major; dU also goes out [B][T][E*He] for the dS product
    RM_TIMED("gelu_bwd", st, RM_HIP(rm::launch_transpose(2, w.dH, sv.U, w.dUt, w.dU, w.Ht, w.b1p, (int)TE, B, He, Bp, dt, st, -1, -1, He, TE * He), "GELU backward"));
    RM_TIMED("tr_dy", st, RM_HIP(rm::launch_transpose(0, w.dy, nullptr, w.dyt, nullptr, nullptr, w.b2p, (int)TE, B, D, Bp, dt, st), "transpose dy"));
    rm::GemmArgs g2;
    g2.dt = dt; g2.epi = rm::kEpiBiasF32;
    g2.M = D; g2.N = He; g2.K = (int)Bp; g2.G = (int)TE;
    g2.A = w.dyt; g2.a_gs = (int64_t)D * Bp; g2.a_rs = Bp;
    g2.W = w.Ht; g2.b_gs = (int64_t)He * Bp;
    g2.C = g->w2; g2.c_gs = (int64_t)D * He; g2.c_rs = He;
    RM_TIMED("bwd_dW2", st, RM_TRY(gemm_go("expert dW2 products", g2, st)));
    RM_TIMED("tr_S", st, RM_HIP(rm::launch_transpose(0, sv.S, nullptr, w.St, nullptr, nullptr, nullptr, T, B, D, Bp, dt, st), "transpose S"));
    rm::GemmArgs g3;
    g3.dt = dt; g3.epi = rm::kEpiBiasF32;
    g3.M = He; g3.N = D; g3.K = (int)Bp; g3.G = (int)TE;
    g3.A = w.dUt; g3.a_gs = (int64_t)He * Bp; g3.a_rs = Bp;
    g3.W = w.St; g3.b_gs = (int64_t)D * Bp; g3.b_gdiv = E;
    g3.C = g->w1; g3.c_gs = (int64_t)He * D; g3.c_rs = D;
    RM_TIMED("bwd_dW1", st, RM_TRY(gemm_go("expert dW1 products", g3, st)));
  }
  // dS from the experts: per token one product over the E experts' hidden units
  // concatenated along K (dU is [B][T][E*He], W1 per token viewed as [E*He][D])
  rm::GemmArgs g4 = moe_dS_args(w.dU, p->moe.w1, w.dSf, B, T, D, E, He, dt);
  if (!rm::gemm_wt_eligible(g4)) {
    RM_TIMED("tr_W1", st, RM_HIP(rm::launch_transpose(0, p->moe.w1, nullptr, w.W1tc, nullptr, nullptr, nullptr, T, (int64_t)E * He, D, (int64_t)E * He, dt, st), "transpose W1"));
    g4.W = w.W1tc;
    g4.w_kmajor = 0;
  }
  RM_TIMED("bwd_dS", st, RM_TRY(gemm_go("expert dS products", g4, st)));
  // routers: dWr = dz^T S (training), lambda * mask^T S (inference); biases from the column sums
  RM_TIMED("tr_router", st, RM_HIP(rm::launch_transpose(0, w.dz, nullptr, w.dzt, nullptr, nullptr, w.brtp, 1, B, TE, Bp, dt, st), "transpose dz"));
  RM_TIMED("tr_router", st, RM_HIP(rm::launch_transpose(0, w.mask, nullptr, w.maskt, nullptr, nullptr, w.brip, 1, B, TE, Bp, dt, st), "transpose mask"));
  rm::GemmArgs g5;
  g5.dt = dt; g5.epi = rm::kEpiBiasF32;
  g5.M = E; g5.N = D; g5.K = (int)Bp; g5.G = T;
  g5.A = w.dzt; g5.a_gs = (int64_t)E * Bp; g5.a_rs = Bp;
  g5.W = w.St; g5.b_gs = (int64_t)D * Bp;
  g5.C = g->wr_train; g5.c_gs = (int64_t)E * D; g5.c_rs = D;
  RM_TIMED("bwd_router", st, RM_TRY(gemm_go("training router gradient", g5, st)));
  rm::GemmArgs g6 = g5;
  g6.A = w.maskt;
  g6.C = g->wr_infer;
  RM_TIMED("bwd_router", st, RM_TRY(gemm_go("inference router gradient", g6, st)));
  RM_TIMED("bwd_router", st, RM_HIP(rm::launch_scale(g->wr_infer, TE * D, lambda, st), "lambda"));
  // S = LN1(TM(X) + X) with dS = dY2 + experts + training router; dX = dY1 + TM(dY1)
  RM_TIMED("ln1_bwd", st, RM_HIP(rm::launch_ln_bwd(1, nullptr, w.dV, w.dSf, x, nullptr, p->ln1_g, w.dY1, w.ln1p, B, T, D, dt, st, w.dSr), "LayerNorm 1 backward"));
  RM_TIMED("tm_add", st, RM_HIP(rm::launch_tm_add(w.dY1, dx, B, T, D, dt, st), "token mix backward"));
  RM_TIMED("sums_ln", st, RM_HIP(rm::launch_sum_parts(w.ln2p, g->ln2_g, g->ln2_b, 1, lg, 2 * (int64_t)D, D, st), "gamma2 / beta2"));
  RM_TIMED("sums_ln", st, RM_HIP(rm::launch_sum_parts(w.ln1p, g->ln1_g, g->ln1_b, 1, lg, 2 * (int64_t)D, D, st), "gamma1 / beta1"));
  RM_TIMED("sums_bias", st, RM_HIP(rm::launch_sum_parts(w.b2p, g->b2, nullptr, (int)TE, w.b2_parts, D, D, st), "b2"));
  RM_TIMED("sums_bias", st, RM_HIP(rm::launch_sum_parts(w.b1p, g->b1, nullptr, (int)TE, w.b1_parts, He, He, st), "b1"));
  RM_TIMED("sums_bias", st, RM_HIP(rm::launch_sum_parts(w.brtp, g->br_train, nullptr, 1, rt, TE, TE, st), "training router bias"));
  RM_TIMED("sums_bias", st, RM_HIP(rm::launch_sum_parts(w.brip, g->br_infer, nullptr, 1, rt, TE, TE, st, lambda), "inference router bias"));
  return ok();
}

size_t rm_model_workspace_bytes(const rm_model_desc* m, int64_t B) {
  if (!m || (m->L > 0 && !m->blocks)) return 0;
  Carver c(nullptr);
  return model_ws(c, m, B, nullptr, nullptr, nullptr);
}

rm_status rm_model_fwd(const rm_model_desc* m, const void* in, void* x_out, float* pooled, float* logits, int64_t B,
                       void* ws, size_t ws_bytes, void* stream) {
  if (!m) return fail(RM_ERR_INVALID, "model descriptor is NULL");
  if (m->L < 0) return fail(RM_ERR_INVALID, "L=%d must not be negative", m->L);
  if (m->L > 0 && !m->blocks) return fail(RM_ERR_INVALID, "blocks is NULL");
  RM_TRY(check_shape(B, m->T, m->D, m->dtype));
  // every block is sized from its own descriptor
  for (int l = 0; l < m->L; ++l) {
    const rm_block_params& p = m->blocks[l];
    RM_TRY(check_block_params(&p, m->dtype));
    if (p.hidden <= 0) return fail(RM_ERR_INVALID, "block %d: hidden=%d must be set (> 0)", l, p.hidden);
    if (p.kind == RM_BLOCK_MOE ? p.E <= 0 : p.E != 0)
      return fail(RM_ERR_INVALID, "block %d: E=%d (MoE blocks need E > 0, other blocks E = 0)", l, p.E);
    const rm_status st = check_block_shape(p.kind, B, m->T, m->D, p.hidden, p.E, m->dtype);
    if (st != RM_OK) return fail(st, "block %d: %s", l, g_last_error.c_str());
  }
  if (m->F < 0) return fail(RM_ERR_INVALID, "F must not be negative");
  if (m->F > (int64_t)m->T * m->D) return fail(RM_ERR_UNSUPPORTED, "F=%lld floats do not fit in T*D", (long long)m->F);
  if ((pooled || logits) && !m->head_w) return fail(RM_ERR_INVALID, "pooled/logits requested without head_w");
  if (B == 0) return ok();
  RM_TRY(check_ptr(in, "in"));
  RM_TRY(check_ptr(x_out, "x_out", false));
  RM_TRY(check_ptr(pooled, "pooled", false));
  RM_TRY(check_ptr(logits, "logits", false));
  RM_TRY(check_ptr(m->head_w, "head_w", false));
  if ((pooled || logits) && !m->head_w) return fail(RM_ERR_INVALID, "pooled/logits requested without head_w");
  if (x_out && x_out == in) return fail(RM_ERR_INVALID, "x_out must not alias in");
  RM_TRY(check_ptr(ws, "ws"));
  const size_t need = rm_model_workspace_bytes(m, B);
  if (ws_bytes < need) return fail(RM_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);

  hipStream_t st = (hipStream_t)stream;
  Carver c(ws);
  void* buf[2];
  void* blk_region;
  model_ws(c, m, B, &buf[0], &buf[1], &blk_region);
  const int T = m->T, D = m->D, dt = m->dtype;
  const void* cur = in;
  int next = 0;
  // every block kind carves S first, so S sits at the same address for all
  // blocks and a boundary pass can leave the next block's S there
  bool s_given = false;
  if (m->F > 0 && m->L > 0 && !(m->blocks[0].flags & RM_BLOCK_NO_MIX_NORM) &&
      rm::mix_ln_emb_supported(T, D, m->F, dt)) {
    // block 0's token mix + LayerNorm 1 read the embedding in place: the
    // tokenized X0 never reaches HBM
    const rm_block_params& p0 = m->blocks[0];
    Carver bc(blk_region);
    BlockWs w0;
    block_ws(bc, p0.kind, B, T, D, p0.hidden, p0.E, dt, &w0);
    audit("mix_ln1_emb.emb", in, B * m->F * 4);
    audit("mix_ln1_emb.ln1_g", p0.ln1_g, (int64_t)D * 4);
    audit("mix_ln1_emb.ln1_b", p0.ln1_b, (int64_t)D * 4);
    RM_TIMED("tokenize_mix_ln1", st,
             RM_HIP(rm::launch_mix_ln_emb((const float*)in, m->F, w0.S, p0.ln1_g, p0.ln1_b, B, T, D, dt, st),
                    "pad-split tokenizer + token mix + LayerNorm"));
    s_given = true;
  } else if (m->F > 0) {
    audit("tokenize.emb", in, B * m->F * 4);
    RM_TIMED("tokenize", st, RM_HIP(rm::launch_tokenize_padsplit((const float*)in, B, m->F, T, D, dt, buf[0], st), "tokenize"));
    cur = buf[0];
    next = 1;
  }
  for (int l = 0; l < m->L; ++l) {
    void* dst = (l == m->L - 1 && x_out) ? x_out : buf[next];
    // this block's own layout in the shared region
    const rm_block_params& p = m->blocks[l];
    Carver bc(blk_region);
    BlockWs w;
    block_ws(bc, p.kind, B, T, D, p.hidden, p.E, dt, &w);
    const bool fuse = fusable_boundary(m, l);
    RM_TRY(run_block(cur, &p, dst, B, T, D, p.hidden, p.E, dt, w, st, s_given, fuse ? &m->blocks[l + 1] : nullptr));
    s_given = fuse;
    if (!fuse) {
      cur = dst;
      next ^= 1;
    }
  }
  if (x_out && cur != x_out) RM_HIP(hipMemcpyAsync(x_out, cur, (size_t)B * T * D * elem_bytes(dt), hipMemcpyDeviceToDevice, st), "copy x_out");
  audit("pool_logit.head_w", m->head_w, (int64_t)D * 4);
  if (m->head_w) RM_TIMED("pool_logit", st, RM_HIP(rm::launch_pool_logit(cur, m->head_w, m->head_c, pooled, logits, B, T, D, dt, st), "pool + logit"));
  return ok();
}

}  // extern "C"

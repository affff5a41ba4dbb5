// C ABI of the MoE layer library: argument validation, workspace layout and
// the launch sequence of the forward and backward passes.  Every check runs
// on the host before anything is launched; the library allocates nothing.
#include <mutex>
#include <vector>

#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline size_t esize(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

int check_desc(const moe_desc_t* d) {
  if (!d) return MOE_ERR_INVALID;
  if (d->num_tokens < 0 || d->d_model <= 0 || d->num_experts < 1 || d->num_experts > 256)
    return MOE_ERR_INVALID;
  if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->num_experts) return MOE_ERR_INVALID;
  if (d->d_ff <= 0 || d->d_model % 64 || d->d_ff % 64) return MOE_ERR_INVALID;
  if (d->num_shared < 0) return MOE_ERR_INVALID;
  if (d->num_shared > 0 && (d->d_ff_shared <= 0 || d->d_ff_shared % 64)) return MOE_ERR_INVALID;
  if (d->score != MOE_SOFTMAX && d->score != MOE_SIGMOID) return MOE_ERR_INVALID;
  if (d->renorm != 0 && d->renorm != 1) return MOE_ERR_INVALID;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (d->reserved != 0) return MOE_ERR_INVALID;
  // row indices are int32: every permuted row index must fit
  if (d->num_tokens * d->top_k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (d->d_model > 65536 || d->d_ff > 65536 || d->num_shared * d->d_ff_shared > 65536)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline int64_t shared_width(const moe_desc_t* d) { return d->num_shared * d->d_ff_shared; }
inline int64_t nblocks(const moe_desc_t* d) { return cdiv64(d->num_tokens, MOE_ROUTE_BLOCK); }

// A bump allocator over the caller's workspace (sizes only when base is null).
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  void* take(size_t n) {
    void* p = base ? base + off : nullptr;
    off += align_up(n);
    return p;
  }
};

GemmProblem gp(int layout, int epi, int ta, int tb, int tc, int64_t G, int64_t M, int64_t N,
               int64_t K, const int32_t* off, const void* A, const void* B, void* C, void* aux) {
  GemmProblem p;
  p.layout = layout;
  p.epilogue = epi;
  p.ta = ta;
  p.tb = tb;
  p.tc = tc;
  p.G = G;
  p.M_total = M;
  p.N = N;
  p.K = K;
  p.offsets = off;
  p.A = A;
  p.B = B;
  p.C = C;
  p.aux = aux;
  return p;
}

// The backward pass's weight-gradient products that may need split partials.
size_t backward_gemm_ws(const moe_desc_t* d) {
  const int dt = d->dtype;
  const int64_t T = d->num_tokens, D = d->d_model, E = d->num_experts, f = d->d_ff;
  const int64_t A = T * d->top_k, F = shared_width(d);
  size_t m = 0;
  auto upd = [&](const GemmProblem& p) {
    const size_t b = gemm_workspace_bytes(p);
    if (b > m) m = b;
  };
  const int rs = router_wgrad_splits((int)T, (int)D, (int)E);
  if (rs > 1 && (size_t)rs * E * D * sizeof(float) > m) m = (size_t)rs * E * D * sizeof(float);
  upd(gp(MOE_GEMM_TN, 0, dt, dt, dt, E, A, D, f, 0, 0, 0, 0, 0));
  upd(gp(MOE_GEMM_TN, 0, dt, dt, dt, E, A, 2 * f, D, 0, 0, 0, 0, 0));
  if (F > 0) {
    upd(gp(MOE_GEMM_TN, 0, dt, dt, dt, 1, T, D, F, 0, 0, 0, 0, 0));
    upd(gp(MOE_GEMM_TN, 0, dt, dt, dt, 1, T, 2 * F, D, 0, 0, 0, 0, 0));
  }
  return m;
}

struct FwdWs {
  int32_t* hist;
  int32_t* base;
  uint8_t* xq;  // fp8: token rows [T, d] and their scales [T]
  float* xs;
  uint8_t* hq;  // fp8: hidden rows, routed [A, f] then shared [T, F], and scales
  float* hs;
};
size_t fwd_ws(const moe_desc_t* d, bool fp8, void* ws, FwdWs* out) {
  Carve c(ws);
  const size_t nb = (size_t)d->num_experts * nblocks(d) * sizeof(int32_t);
  FwdWs w{};
  w.hist = (int32_t*)c.take(nb);
  w.base = (int32_t*)c.take(nb);
  if (fp8) {
    const size_t T = (size_t)d->num_tokens, A = T * (size_t)d->top_k;
    const size_t hrows = A > T ? A : T;
    const size_t hq = A * (size_t)d->d_ff > T * (size_t)shared_width(d) ? A * (size_t)d->d_ff
                                                                          : T * (size_t)shared_width(d);
    w.xq = (uint8_t*)c.take(T * (size_t)d->d_model);
    w.xs = (float*)c.take(T * sizeof(float));
    w.hq = (uint8_t*)c.take(hq);
    w.hs = (float*)c.take(hrows * sizeof(float));
  }
  if (out) *out = w;
  return c.off;
}

struct BwdWs {
  void* terms;
  void* dy_perm;   // [A, d]; reused for dx_perm once the down gradients are done
  void* dgu;       // [A, 2f]
  float* dlogits;  // [T, E]
  void* s_dgu;     // [T, 2F]
  void* dx_shared; // [T, d]
  int32_t* iota;   // [T] identity row map (shared experts)
  void* gemm;      // split partials
  size_t gemm_bytes;
  uint8_t* q;      // fp8: the quantised operand of each data gradient in turn
  float* qs;       // and its row scales
  uint8_t* q_dy;   // fp8: dy's codes [T, d] and scales [T] (the shared down data gradient)
  float* qs_dy;
  // fp8 weight gradients: the two operands' padded transposed codes, their
  // per-(group, column) scales, and the padded group offsets (routed, shared)
  uint8_t* wa;
  uint8_t* wb;
  float* wsa;
  float* wsb;
  int32_t* pad;
  int32_t* pad_s;
};
// bytes of the padded transposed codes of C columns over M rows in G groups
inline size_t colwise_bytes(int64_t G, int64_t M, int64_t C) { return (size_t)C * (size_t)(M + 63 * G); }
size_t bwd_ws(const moe_desc_t* d, bool fp8, void* ws, BwdWs* out, bool wgrad8 = false) {
  Carve c(ws);
  const int64_t T = d->num_tokens, D = d->d_model, f = d->d_ff, A = T * d->top_k;
  const int64_t F = shared_width(d);
  const size_t es = esize(d->dtype);
  BwdWs w;
  w.dy_perm = c.take((size_t)A * D * es);
  w.dgu = c.take((size_t)A * 2 * f * es);
  w.dlogits = (float*)c.take((size_t)T * d->num_experts * sizeof(float));
  w.terms = c.take(router_terms_ws_bytes(T, d->num_experts));
  w.s_dgu = F > 0 ? c.take((size_t)T * 2 * F * es) : nullptr;
  // the identity row map of the shared gate/up weight gradient when it runs
  // in one launch with the routed one, whose token rows are gathered
  w.iota = F > 0 ? (int32_t*)c.take((size_t)T * sizeof(int32_t)) : nullptr;
  w.dx_shared = F > 0 ? c.take((size_t)T * D * es) : nullptr;
  w.gemm_bytes = backward_gemm_ws(d);
  w.gemm = c.take(w.gemm_bytes);
  w.q = nullptr;
  w.qs = nullptr;
  w.q_dy = nullptr;
  w.qs_dy = nullptr;
  if (fp8) {
    // dY~ [A, d], dG|dU [A, 2f], dy [T, d], shared dG|dU [T, 2F]
    const size_t szs[] = {(size_t)A * D, (size_t)A * 2 * f, (size_t)T * D, (size_t)T * 2 * F};
    size_t qb = 0;
    for (size_t z : szs) qb = z > qb ? z : qb;
    w.q = (uint8_t*)c.take(qb);
    w.qs = (float*)c.take((size_t)(A > T ? A : T) * sizeof(float));
    w.q_dy = (uint8_t*)c.take((size_t)T * D);
    w.qs_dy = (float*)c.take((size_t)T * sizeof(float));
  }
  w.wa = w.wb = nullptr;
  w.wsa = w.wsb = nullptr;
  w.pad = w.pad_s = nullptr;
  if (fp8 && wgrad8) {
    const int64_t E = d->num_experts;
    // routed: dW_d (A' = dY~ [d], B' = H [f]), dW_gu (A' = dG|dU [2f], B' = x [d]);
    // shared: dW_sd (dy [d], H_s [F]), dW_sgu (dG|dU_s [2F], x [d])
    const size_t ra = D > 2 * f ? D : 2 * f, rb = D > f ? D : f;
    const size_t sa = F > 0 ? (size_t)(D > 2 * F ? D : 2 * F) : 0, sb = F > 0 ? (size_t)(D > F ? D : F) : 0;
    size_t qa = colwise_bytes(E, A, ra), qb = colwise_bytes(E, A, rb);
    if (F > 0) {
      qa = qa > colwise_bytes(1, T, sa) ? qa : colwise_bytes(1, T, sa);
      qb = qb > colwise_bytes(1, T, sb) ? qb : colwise_bytes(1, T, sb);
    }
    const size_t fa = (size_t)E * ra > sa ? (size_t)E * ra : sa, fb = (size_t)E * rb > sb ? (size_t)E * rb : sb;
    w.wa = (uint8_t*)c.take(qa);
    w.wb = (uint8_t*)c.take(qb);
    w.wsa = (float*)c.take(fa * sizeof(float));
    w.wsb = (float*)c.take(fb * sizeof(float));
    w.pad = (int32_t*)c.take((size_t)(E + 1) * sizeof(int32_t));
    w.pad_s = (int32_t*)c.take(2 * sizeof(int32_t));
  }
  if (out) *out = w;
  return c.off;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                         \
  do {                                        \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

// ---- per-stage event timing (off unless the caller enables it)
struct StageRec {
  int stage;
  hipEvent_t a, b;
};
constexpr size_t kMaxStageRecs = size_t(1) << 16;
std::mutex g_timing_mu;
uint32_t g_timing = 0;          // bit s: stage s is timed
std::vector<StageRec> g_recs;   // recorded, not yet read
std::vector<StageRec> g_spare;  // event pairs ready for reuse

// Returns an event pair already recorded on `st`, or {-1} when not timing.
StageRec stage_begin(int stage, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  StageRec r{-1, nullptr, nullptr};
  if (!((g_timing >> stage) & 1u) || g_recs.size() >= kMaxStageRecs) return r;
  if (!g_spare.empty()) {
    r = g_spare.back();
    g_spare.pop_back();
  } else if (hipEventCreate(&r.a) != hipSuccess) {
    return StageRec{-1, nullptr, nullptr};
  } else if (hipEventCreate(&r.b) != hipSuccess) {
    (void)hipEventDestroy(r.a);
    return StageRec{-1, nullptr, nullptr};
  }
  r.stage = stage;
  if (hipEventRecord(r.a, st) != hipSuccess) {
    g_spare.push_back(r);
    r.stage = -1;
  }
  return r;
}

void stage_end(StageRec r, hipStream_t st) {
  if (r.stage < 0) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  if (hipEventRecord(r.b, st) == hipSuccess)
    g_recs.push_back(r);
  else
    g_spare.push_back(r);
}

// A stage whose launch failed: its event pair goes back unrecorded.
void stage_abort(StageRec r) {
  if (r.stage < 0) return;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_spare.push_back(r);
}

// Runs the launches of one stage between its two events.
#define MOE_STAGE(stage, expr)                    \
  do {                                            \
    const StageRec _r = stage_begin((stage), st); \
    const hipError_t _e = (expr);                 \
    if (_e != hipSuccess) {                       \
      stage_abort(_r);                            \
      return MOE_ERR_HIP;                         \
    }                                             \
    stage_end(_r, st);                            \
  } while (0)

// ---- the device-resident scratch of moe_forward_no_workspace
// One copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address: its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept here.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

static __device__ __align__(256) char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device (looked up on the first
// call on that device).
int scratch_device_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID: invalid argument";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: pointer not 16-byte aligned";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape not supported by this build";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

int moe_abi_version(void) { return MOE_ABI_VERSION; }

size_t moe_route_hist_elems(const moe_desc_t* d) {
  if (check_desc(d) != MOE_OK) return 0;
  return (size_t)d->num_experts * (size_t)nblocks(d);
}

size_t moe_workspace_bytes(const moe_desc_t* d, int which) {
  if (check_desc(d) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_PERMUTE: return align_up((size_t)d->num_experts * nblocks(d) * sizeof(int32_t));
    case MOE_WS_FORWARD: return fwd_ws(d, false, nullptr, nullptr);
    case MOE_WS_BACKWARD: return bwd_ws(d, false, nullptr, nullptr);
    case MOE_WS_FORWARD_FP8: return fwd_ws(d, true, nullptr, nullptr);
    case MOE_WS_BACKWARD_FP8: return bwd_ws(d, true, nullptr, nullptr);
    case MOE_WS_BACKWARD_FP8_WGRAD: return bwd_ws(d, true, nullptr, nullptr, true);
    default: return 0;
  }
}

// The saved buffers of moe_forward in one allocation: each field 256-byte
// aligned, in struct order; fields the flags leave out stay NULL.
static size_t saved_layout(const moe_desc_t* d, int flags, char* base, moe_saved_t* out) {
  const int64_t T = d->num_tokens, D = d->d_model, E = d->num_experts, k = d->top_k;
  const int64_t f = d->d_ff, F = shared_width(d), A = T * k;
  const size_t es = d->dtype == MOE_BF16 ? 2 : 4;
  const bool training = flags & MOE_SAVED_TRAINING, copy = flags & MOE_SAVED_PERMUTED_COPY;
  size_t off = 0;
  auto take = [&](size_t bytes, bool want) -> void* {
    if (!want) return nullptr;
    void* p = base ? base + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return p;
  };
  moe_saved_t s;
  s.logits = (float*)take((size_t)T * E * 4, true);
  s.idx = (int32_t*)take((size_t)T * k * 4, true);
  s.gate = (float*)take((size_t)T * k * 4, true);
  s.counts = (int32_t*)take((size_t)E * 4, true);
  s.offsets = (int32_t*)take((size_t)(E + 1) * 4, true);
  s.pos = (int32_t*)take((size_t)A * 4, true);
  s.src = (int32_t*)take((size_t)A * 4, true);
  s.tok = (int32_t*)take((size_t)A * 4, true);
  s.x_perm = take((size_t)A * D * es, copy);
  s.preact = take((size_t)A * 2 * f * es, training);
  s.h = take((size_t)A * f * es, true);
  s.y_perm = take((size_t)A * D * es, true);
  s.s_preact = take((size_t)T * 2 * F * es, training && F > 0);
  s.s_h = take((size_t)T * F * es, F > 0);
  if (out) *out = s;
  return off;
}

size_t moe_saved_bytes(const moe_desc_t* d, int flags) {
  if (check_desc(d) != MOE_OK || (flags & ~3)) return 0;
  return saved_layout(d, flags, nullptr, nullptr);
}

int moe_saved_carve(const moe_desc_t* d, int flags, void* base, size_t bytes, moe_saved_t* out) {
  int s = check_desc(d);
  if (s) return s;
  if ((flags & ~3) || !base || !out) return MOE_ERR_INVALID;
  if (((uintptr_t)base & 255) != 0) return MOE_ERR_ALIGN;
  if (bytes < saved_layout(d, flags, nullptr, nullptr)) return MOE_ERR_WORKSPACE;
  saved_layout(d, flags, (char*)base, out);
  return MOE_OK;
}

static int check_gemm(int layout, int epi, int dtype, int64_t G, int64_t M, int64_t N, int64_t K) {
  if (layout < MOE_GEMM_NT || layout > MOE_GEMM_TN) return MOE_ERR_INVALID;
  if (epi == MOE_EPI_SWIGLU && layout != MOE_GEMM_NT) return MOE_ERR_INVALID;
  if (epi == MOE_EPI_DSWIGLU && layout != MOE_GEMM_NN) return MOE_ERR_INVALID;
  if (epi < MOE_EPI_NONE || epi > MOE_EPI_DSWIGLU) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (G < 1 || G > 256 || M < 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID;
  if (N % 64 || K % 64) return MOE_ERR_INVALID;
  if (epi == MOE_EPI_SWIGLU && (N % 128)) return MOE_ERR_INVALID;
  if (M >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_grouped_gemm_workspace_bytes(int layout, int dtype, int64_t G, int64_t M, int64_t N,
                                        int64_t K) {
  if (check_gemm(layout, MOE_EPI_NONE, dtype, G, M, N, K) != MOE_OK) return 0;
  return gemm_workspace_bytes(gp(layout, 0, dtype, dtype, dtype, G, M, N, K, 0, 0, 0, 0, 0));
}

int moe_route(const moe_desc_t* d, const float* logits, const float* bias, int32_t* idx,
              float* gate, int32_t* block_hist, void* stream) {
  int s = check_desc(d);
  if (s) return s;
  if (d->num_tokens > 0 && (!logits || !idx || !gate || !block_hist)) return MOE_ERR_INVALID;
  if (!aligned16(logits) || !aligned16(idx) || !aligned16(gate) || !aligned16(block_hist) ||
      !aligned16(bias))
    return MOE_ERR_ALIGN;
  return hip_status(launch_route(logits, d->score == MOE_SIGMOID ? bias : nullptr,
                                 (int)d->num_tokens, (int)d->num_experts, (int)d->top_k,
                                 d->score, d->renorm, idx, gate, block_hist,
                                 (hipStream_t)stream));
}

int moe_permute(const moe_desc_t* d, const void* x, const int32_t* idx,
                const int32_t* block_hist, int32_t* counts, int32_t* offsets, int32_t* pos,
                int32_t* src, int32_t* tok, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  int s = check_desc(d);
  if (s) return s;
  if (!counts || !offsets) return MOE_ERR_INVALID;
  if (d->num_tokens > 0 && (!idx || !block_hist || !pos || !src || !ws || (x_perm && !x)))
    return MOE_ERR_INVALID;
  const void* ptrs[] = {x, idx, block_hist, counts, offsets, pos, src, tok, x_perm, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  if (ws_bytes < moe_workspace_bytes(d, MOE_WS_PERMUTE)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_permute(x, d->dtype, idx, block_hist, (int)d->num_tokens,
                                   (int)d->d_model, (int)d->num_experts, (int)d->top_k,
                                   (int32_t*)ws, counts, offsets, pos, src, tok, x_perm,
                                   (hipStream_t)stream));
}

int moe_grouped_gemm(int layout, int epi, int dtype, int64_t G, int64_t M, int64_t N, int64_t K,
                     const int32_t* off, const void* A, const void* B, void* C, void* aux,
                     void* ws, size_t ws_bytes, void* stream) {
  int s = check_gemm(layout, epi, dtype, G, M, N, K);
  if (s) return s;
  if ((!off && G != 1) || !B || !C) return MOE_ERR_INVALID;
  if (M > 0 && !A) return MOE_ERR_INVALID;
  if (epi == MOE_EPI_DSWIGLU && !aux) return MOE_ERR_INVALID;
  const void* ptrs[] = {off, A, B, C, aux, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  GemmProblem p = gp(layout, epi, dtype, dtype, dtype, G, M, N, K, off, A, B, C, aux);
  if (ws_bytes < gemm_workspace_bytes(p) || (gemm_workspace_bytes(p) && !ws))
    return MOE_ERR_WORKSPACE;
  return hip_status(launch_grouped_gemm(p, ws, ws_bytes, (hipStream_t)stream));
}

int moe_grouped_gemm_gather(int layout, int epi, int64_t G, int64_t M, int64_t N, int64_t K,
                            const int32_t* off, const void* A, const void* B, void* C, void* aux,
                            const int32_t* rows, int64_t src_rows, void* stream) {
  int s = check_gemm(layout, epi, MOE_BF16, G, M, N, K);
  if (s) return s;
  if ((!off && G != 1) || !B || !C || src_rows < 0) return MOE_ERR_INVALID;
  if (M > 0 && (!A || !rows)) return MOE_ERR_INVALID;
  const void* ptrs[] = {off, A, B, C, aux, rows};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  if (layout == MOE_GEMM_NN || epi == MOE_EPI_DSWIGLU || (layout == MOE_GEMM_TN && epi != MOE_EPI_NONE))
    return MOE_ERR_UNSUPPORTED;
  // row byte offsets of the token matrix are 32-bit in the kernel
  if (src_rows * K * 2 > (int64_t(1) << 32)) return MOE_ERR_UNSUPPORTED;
  GemmProblem p = gp(layout, epi, MOE_BF16, MOE_BF16, MOE_BF16, G, M, N, K, off, A, B, C, aux);
  // M = 0: any non-null device pointer selects the gathered kernel (with no
  // routed rows the map is never read)
  p.rows = rows ? rows : (off ? off : (const int32_t*)C);
  if (!gemm_big_supported(p)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_grouped_gemm(p, nullptr, 0, (hipStream_t)stream));
}

int moe_combine(const moe_desc_t* d, const void* y_perm, const float* gate, const int32_t* pos,
                const void* shared_y, void* y, void* stream) {
  int s = check_desc(d);
  if (s) return s;
  if (d->num_tokens > 0 && (!y_perm || !gate || !pos || !y)) return MOE_ERR_INVALID;
  const void* ptrs[] = {y_perm, gate, pos, shared_y, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  return hip_status(launch_combine(d->dtype, y_perm, gate, pos, shared_y, y,
                                   (int)d->num_tokens, (int)d->d_model, (int)d->top_k,
                                   (hipStream_t)stream));
}

// Layers whose routed gate/up products can read the token rows through the
// row map (saved.x_perm == NULL): the persistent kernel takes the forward
// product and, for training, the weight gradient; row byte offsets fit 32 bits.
static int gather_supported(const moe_desc_t* d, bool training) {
  const int64_t T = d->num_tokens, D = d->d_model, E = d->num_experts, f = d->d_ff;
  if (d->dtype != MOE_BF16 || T * D * 2 > (int64_t(1) << 32)) return MOE_ERR_UNSUPPORTED;
  static const int32_t dummy = 0;
  GemmProblem fw = gp(MOE_GEMM_NT, MOE_EPI_SWIGLU, MOE_BF16, MOE_BF16, MOE_BF16, E, T * d->top_k, 2 * f, D,
                      0, 0, 0, 0, 0);
  GemmProblem wg = gp(MOE_GEMM_TN, MOE_EPI_NONE, MOE_BF16, MOE_BF16, MOE_BF16, E, T * d->top_k, 2 * f, D,
                      0, 0, 0, 0, 0);
  fw.rows = wg.rows = &dummy;
  if (!gemm_big_supported(fw) || (training && !gemm_big_supported(wg))) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The fp8 layer calls: bf16 layers whose SwiGLU products pair 128 gate with
// 128 up columns per tile, and whose token rows (gathered as fp8 codes) have
// 32-bit byte offsets.
static int fp8_layer_supported(const moe_desc_t* d) {
  if (d->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (d->d_ff % 128 || shared_width(d) % 128) return MOE_ERR_UNSUPPORTED;
  if (d->num_tokens * d->d_model > (int64_t(1) << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The forward pass of moe_forward (w8 NULL) or moe_forward_fp8 on the
// workspace ws (ws_bytes of it).
static int forward_impl(const moe_desc_t* d, const moe_weights_t* w, const moe_fp8_weights_t* w8,
                        const void* x, void* y, const moe_saved_t* sv, void* ws, size_t ws_bytes,
                        void* stream) {
  int s = check_desc(d);
  if (s) return s;
  if (!w || !sv) return MOE_ERR_INVALID;
  const int64_t T = d->num_tokens, D = d->d_model, E = d->num_experts, k = d->top_k;
  const int64_t f = d->d_ff, F = shared_width(d), A = T * k;
  const int dt = d->dtype;
  const bool fp8 = w8 != nullptr;
  if (!w->w_router) return MOE_ERR_INVALID;
  if (fp8) {
    s = fp8_layer_supported(d);
    if (s) return s;
    if (!w8->gateup_q || !w8->gateup_s || !w8->down_q || !w8->down_s) return MOE_ERR_INVALID;
    if (F > 0 && (!w8->s_gateup_q || !w8->s_gateup_s || !w8->s_down_q || !w8->s_down_s))
      return MOE_ERR_INVALID;
    const void* p8[] = {w8->gateup_q, w8->gateup_s, w8->down_q, w8->down_s, w8->s_gateup_q,
                        w8->s_gateup_s, w8->s_down_q, w8->s_down_s};
    for (const void* p : p8)
      if (!aligned16(p)) return MOE_ERR_ALIGN;
  } else {
    if (!w->w_gateup || !w->w_down) return MOE_ERR_INVALID;
    if (F > 0 && (!w->s_gateup || !w->s_down)) return MOE_ERR_INVALID;
  }
  if (!sv->counts || !sv->offsets) return MOE_ERR_INVALID;
  // no permuted copy of the tokens: the gate/up products gather them (with
  // no tokens there is nothing to gather); the fp8 products always gather
  // the quantised token rows
  const bool gather = T > 0 && (fp8 || !sv->x_perm);
  if (T > 0 && (!x || !y || !sv->logits || !sv->idx || !sv->gate || !sv->pos || !sv->src ||
                (gather && !sv->tok) || !sv->h || !sv->y_perm || !ws || (F > 0 && !sv->s_h)))
    return MOE_ERR_INVALID;
  const void* ptrs[] = {x, y, w->w_router, w->bias, w->w_gateup, w->w_down, w->s_gateup,
                        w->s_down, sv->logits, sv->idx, sv->gate, sv->counts, sv->offsets,
                        sv->pos, sv->src, sv->tok, sv->x_perm, sv->preact, sv->h, sv->y_perm,
                        sv->s_preact, sv->s_h, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  if (gather && !fp8) {
    s = gather_supported(d, sv->preact != nullptr);
    if (s) return s;
  }
  if (ws_bytes < moe_workspace_bytes(d, fp8 ? MOE_WS_FORWARD_FP8 : MOE_WS_FORWARD)) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (T == 0) {
    MOE_TRY(launch_fill_i32(sv->counts, E, 0, st));
    MOE_TRY(launch_fill_i32(sv->offsets, E + 1, 0, st));
    return MOE_OK;
  }
  FwdWs fw;
  fwd_ws(d, fp8, ws, &fw);
  // 1. router logits in fp32, 2. scores, top-k, gates, per-block histogram
  // (one kernel when a workgroup holds all E logits of its tokens)
  const float* rbias = d->score == MOE_SIGMOID ? w->bias : nullptr;
  if (router_route_fused(dt, (int)D, (int)E)) {
    MOE_STAGE(MOE_STAGE_ROUTER, launch_router_route(x, w->w_router, (int)T, (int)D, (int)E, sv->logits, rbias,
                                                    (int)k, d->score, d->renorm, sv->idx, sv->gate, fw.hist, st));
  } else {
    MOE_STAGE(MOE_STAGE_ROUTER, launch_router_logits(x, dt, w->w_router, (int)T, (int)D, (int)E, sv->logits, st));
    MOE_STAGE(MOE_STAGE_ROUTE, launch_route(sv->logits, rbias, (int)T, (int)E, (int)k, d->score, d->renorm,
                                            sv->idx, sv->gate, fw.hist, st));
  }
  // 3. permutation into expert-contiguous rows
  MOE_STAGE(MOE_STAGE_PERMUTE, launch_permute(x, dt, sv->idx, fw.hist, (int)T, (int)D, (int)E, (int)k, fw.base,
                         sv->counts, sv->offsets, sv->pos, sv->src, sv->tok, sv->x_perm, st));
  if (fp8) {
    // 4. token rows in e4m3 (one scale per token), gate/up product on the
    // routed rows gathered through tok, SwiGLU; 5. hidden rows in e4m3, down
    // product; 6. the same for the shared experts (no gather)
    MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, launch_quantize_fp8(x, dt, T, (int)D, fw.xq, fw.xs, st));
    MOE_STAGE(MOE_STAGE_GATE_UP, launch_gemm_fp8(MOE_EPI_SWIGLU, E, A, 2 * f, D, sv->offsets, fw.xq, fw.xs,
                                                 w8->gateup_q, w8->gateup_s, sv->h, sv->preact, sv->tok, st));
    MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, launch_quantize_fp8(sv->h, dt, A, (int)f, fw.hq, fw.hs, st));
    MOE_STAGE(MOE_STAGE_DOWN, launch_gemm_fp8(MOE_EPI_NONE, E, A, D, f, sv->offsets, fw.hq, fw.hs, w8->down_q,
                                              w8->down_s, sv->y_perm, nullptr, nullptr, st));
    if (F > 0) {
      MOE_STAGE(MOE_STAGE_SHARED_GATE_UP,
                launch_gemm_fp8(MOE_EPI_SWIGLU, 1, T, 2 * F, D, nullptr, fw.xq, fw.xs, w8->s_gateup_q,
                                w8->s_gateup_s, sv->s_h, sv->s_preact, nullptr, st));
      MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, launch_quantize_fp8(sv->s_h, dt, T, (int)F, fw.hq, fw.hs, st));
      MOE_STAGE(MOE_STAGE_SHARED_DOWN, launch_gemm_fp8(MOE_EPI_NONE, 1, T, D, F, nullptr, fw.hq, fw.hs,
                                                       w8->s_down_q, w8->s_down_s, y, nullptr, nullptr, st));
    }
  } else {
    // 4. gate/up grouped GEMM with the SwiGLU activation (rows of x_perm, or of
    // x gathered through tok)
    GemmProblem gu = gp(MOE_GEMM_NT, MOE_EPI_SWIGLU, dt, dt, dt, E, A, 2 * f, D, sv->offsets,
                        gather ? x : sv->x_perm, w->w_gateup, sv->h, sv->preact);
    gu.rows = gather ? sv->tok : nullptr;
    MOE_STAGE(MOE_STAGE_GATE_UP, launch_grouped_gemm(gu, nullptr, 0, st));
    // 5. down grouped GEMM
    MOE_STAGE(MOE_STAGE_DOWN, launch_grouped_gemm(gp(MOE_GEMM_NT, MOE_EPI_NONE, dt, dt, dt, E, A, D, f, sv->offsets,
                                   sv->h, w->w_down, sv->y_perm, nullptr),
                                nullptr, 0, st));
    // 6. shared experts on every token; their output lands in y
    if (F > 0) {
      MOE_STAGE(MOE_STAGE_SHARED_GATE_UP, launch_grouped_gemm(gp(MOE_GEMM_NT, MOE_EPI_SWIGLU, dt, dt, dt, 1, T, 2 * F, D,
                                     nullptr, x, w->s_gateup, sv->s_h, sv->s_preact),
                                  nullptr, 0, st));
      MOE_STAGE(MOE_STAGE_SHARED_DOWN, launch_grouped_gemm(gp(MOE_GEMM_NT, MOE_EPI_NONE, dt, dt, dt, 1, T, D, F,
                                     nullptr, sv->s_h, w->s_down, y, nullptr),
                                  nullptr, 0, st));
    }
  }
  // 7. weighted combine (+ shared output)
  MOE_STAGE(MOE_STAGE_COMBINE, launch_combine(dt, sv->y_perm, sv->gate, sv->pos, F > 0 ? y : nullptr, y, (int)T,
                         (int)D, (int)k, st));
  return MOE_OK;
}

int moe_forward(const moe_desc_t* d, const moe_weights_t* w, const void* x, void* y,
                const moe_saved_t* sv, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(d, w, nullptr, x, y, sv, ws, ws_bytes, stream);
}

int moe_forward_fp8(const moe_desc_t* d, const moe_weights_t* w, const moe_fp8_weights_t* w8,
                    const void* x, void* y, const moe_saved_t* sv, void* ws, size_t ws_bytes,
                    void* stream) {
  if (!w8) return MOE_ERR_INVALID;
  return forward_impl(d, w, w8, x, y, sv, ws, ws_bytes, stream);
}

int moe_forward_no_workspace(const moe_desc_t* d, const moe_weights_t* w, const void* x, void* y,
                             const moe_saved_t* sv, void* stream) {
  const int s = check_desc(d);
  if (s) return s;
  const size_t need = fwd_ws(d, false, nullptr, nullptr);
  if (need > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  const int r = scratch_device_ptr(&ws);
  if (r) return r;
  return forward_impl(d, w, nullptr, x, y, sv, ws, MOE_STATIC_SCRATCH_BYTES, stream);
}

// The backward pass of moe_backward (w8 NULL) or moe_backward_fp8.
static int backward_impl(const moe_desc_t* d, const moe_weights_t* w, const moe_fp8_weights_t* w8,
                         int grad_format, int wgrad_fp8, const void* x, const moe_saved_t* sv, const void* dy,
                         void* dx,
                         const moe_grads_t* g, const moe_router_terms_t* terms, float* losses,
                         void* ws, size_t ws_bytes, void* stream) {
  int s = check_desc(d);
  if (s) return s;
  if (losses && !terms) return MOE_ERR_INVALID;
  if (terms) {
    const float cs[3] = {terms->aux_coeff, terms->seq_aux_coeff, terms->z_coeff};
    for (float c : cs)
      if (!(c >= 0.0f) || c > 3.0e38f) return MOE_ERR_INVALID;  // also rejects NaN
    if (terms->seq_len < 0 || (terms->seq_len > 0 && d->num_tokens % terms->seq_len))
      return MOE_ERR_INVALID;
    if (!aligned16(losses)) return MOE_ERR_ALIGN;
  }
  if (!w || !sv || !g) return MOE_ERR_INVALID;
  const int64_t T = d->num_tokens, D = d->d_model, E = d->num_experts, k = d->top_k;
  const int64_t f = d->d_ff, F = shared_width(d), A = T * k;
  const int dt = d->dtype;
  const bool fp8 = w8 != nullptr;
  if (grad_format != MOE_E4M3 && grad_format != MOE_E5M2) return MOE_ERR_INVALID;
  if (wgrad_fp8 != 0 && wgrad_fp8 != 1) return MOE_ERR_INVALID;
  const bool wg8 = fp8 && wgrad_fp8;
  const int gf = grad_format == MOE_E5M2 ? FP8_E5M2 : FP8_E4M3;
  if (!w->w_router || !w->w_gateup || !w->w_down) return MOE_ERR_INVALID;
  if (!g->d_w_router || !g->d_w_gateup || !g->d_w_down) return MOE_ERR_INVALID;
  if (F > 0 && (!w->s_gateup || !w->s_down || !g->d_s_gateup || !g->d_s_down))
    return MOE_ERR_INVALID;
  if (fp8) {
    s = fp8_layer_supported(d);
    if (s) return s;
    if (!w8->gateup_tq || !w8->gateup_ts || !w8->down_tq || !w8->down_ts) return MOE_ERR_INVALID;
    if (F > 0 && (!w8->s_gateup_tq || !w8->s_gateup_ts || !w8->s_down_tq || !w8->s_down_ts))
      return MOE_ERR_INVALID;
    const void* p8[] = {w8->gateup_tq, w8->gateup_ts, w8->down_tq, w8->down_ts, w8->s_gateup_tq,
                        w8->s_gateup_ts, w8->s_down_tq, w8->s_down_ts};
    for (const void* p : p8)
      if (!aligned16(p)) return MOE_ERR_ALIGN;
  }
  if (F > 0 && T > 0 && (!sv->s_h || !sv->s_preact)) return MOE_ERR_INVALID;
  if (!sv->offsets) return MOE_ERR_INVALID;
  const bool gather = T > 0 && !sv->x_perm;
  if (T > 0 && (!x || !dy || !dx || !sv->logits || !sv->idx || !sv->gate || !sv->pos ||
                (gather && !sv->tok) || !sv->preact || !sv->h || !sv->y_perm || !ws))
    return MOE_ERR_INVALID;
  const void* ptrs[] = {x, dy, dx, w->w_router, w->w_gateup, w->w_down, w->s_gateup, w->s_down,
                        sv->logits, sv->idx, sv->gate, sv->offsets, sv->pos, sv->tok, sv->x_perm,
                        sv->preact, sv->h, sv->y_perm, sv->s_preact, sv->s_h, g->d_w_router,
                        g->d_w_gateup, g->d_w_down, g->d_s_gateup, g->d_s_down, ws};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  if (gather) {
    s = gather_supported(d, true);
    if (s) return s;
  }
  if (ws_bytes < moe_workspace_bytes(d, wg8 ? MOE_WS_BACKWARD_FP8_WGRAD
                                            : (fp8 ? MOE_WS_BACKWARD_FP8 : MOE_WS_BACKWARD)))
    return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  BwdWs bw;
  bwd_ws(d, fp8, ws, &bw, wg8);
  // an fp8 weight gradient: both operands quantised column-wise over each
  // group's rows (stored transposed and padded), then the scaled product
  auto quant_w = [&](const void* src, const int32_t* rows, const int32_t* offs, int G, int64_t M, int64_t C,
                     int32_t* pad, uint8_t* q, float* sc) -> hipError_t {
    return launch_quantize_fp8_colwise(src, dt, rows, offs, G, M, C, pad, q, sc, st);
  };
  // 1. combine backward + router backward (dlogits); fp8 (k <= 8): the
  // same kernel also writes the e4m3 copies of dY~ and dy
  const bool fused_q = fp8 && k <= 8;
  if (fused_q) {
    MOE_STAGE(MOE_STAGE_COMBINE_BWD, launch_combine_bwd_fp8(dy, sv->y_perm, sv->gate, sv->pos, sv->idx, sv->logits,
                                                            d->score, d->renorm, (int)T, (int)D, (int)E, (int)k,
                                                            bw.dy_perm, bw.dlogits, bw.q, bw.qs, bw.q_dy, bw.qs_dy,
                                                            st, gf));
  } else {
    MOE_STAGE(MOE_STAGE_COMBINE_BWD, launch_combine_bwd(dt, dy, sv->y_perm, sv->gate, sv->pos, sv->idx, sv->logits,
                               d->score, d->renorm, (int)T, (int)D, (int)E, (int)k, bw.dy_perm,
                               bw.dlogits, st));
  }
  // 1b. router training terms: their gradients join the router gradient
  if (terms && T > 0 && !sv->counts) return MOE_ERR_INVALID;
  // terms_grad: some term adds gradient; the kernels also run for the loss
  // values alone
  const bool terms_grad = terms && (terms->aux_coeff > 0.0f || terms->seq_aux_coeff > 0.0f ||
                                    terms->z_coeff > 0.0f);
  if (terms_grad || losses) {
    MOE_STAGE(MOE_STAGE_ROUTER_TERMS,
              launch_router_terms(sv->logits, sv->idx, sv->counts, (int)T, (int)E, (int)k, d->score,
                                  terms->aux_coeff, terms->seq_aux_coeff, terms->z_coeff,
                                  terms->seq_len, bw.dlogits, losses, bw.terms, st));
  }
  // 2. down data gradient fused with the SwiGLU derivative -> dG | dU (fp8:
  // dY~ in e4m3 per row against W_d quantised along d, stored transposed)
  if (fp8) {
    if (!fused_q)
      MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, launch_quantize_fp8(bw.dy_perm, dt, A, (int)D, bw.q, bw.qs, st, gf));
    MOE_STAGE(MOE_STAGE_DOWN_DGRAD, launch_gemm_fp8(MOE_EPI_DSWIGLU, E, A, f, D, sv->offsets, bw.q, bw.qs,
                                                    w8->down_tq, w8->down_ts, bw.dgu, sv->preact, nullptr, st, gf));
  } else {
    MOE_STAGE(MOE_STAGE_DOWN_DGRAD, launch_grouped_gemm(gp(MOE_GEMM_NN, MOE_EPI_DSWIGLU, dt, dt, dt, E, A, D, f,
                                   sv->offsets, bw.dy_perm, w->w_down, bw.dgu, sv->preact),
                                nullptr, 0, st));
  }
  // the shared experts' down data gradient (-> their dG | dU)
  auto shared_down_dgrad = [&]() -> int {
    if (fp8) {
      if (!fused_q)
        MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, launch_quantize_fp8(dy, dt, T, (int)D, bw.q_dy, bw.qs_dy, st, gf));
      MOE_STAGE(MOE_STAGE_SHARED_DOWN_DGRAD,
                launch_gemm_fp8(MOE_EPI_DSWIGLU, 1, T, F, D, nullptr, bw.q_dy, bw.qs_dy, w8->s_down_tq,
                                w8->s_down_ts, bw.s_dgu, sv->s_preact, nullptr, st, gf));
    } else {
      MOE_STAGE(MOE_STAGE_SHARED_DOWN_DGRAD, launch_grouped_gemm(gp(MOE_GEMM_NN, MOE_EPI_DSWIGLU, dt, dt, dt, 1, T, D, F,
                                     nullptr, dy, w->s_down, bw.s_dgu, sv->s_preact),
                                  nullptr, 0, st));
    }
    return MOE_OK;
  };
  // bf16 weight gradients with shared experts: each routed weight gradient
  // and its shared counterpart run as one launch of the persistent kernel,
  // the shared experts' few long tiles first (so their down data gradient
  // runs before the weight gradients)
  GemmProblem dw_r = gp(MOE_GEMM_TN, MOE_EPI_NONE, dt, dt, dt, E, A, D, f, sv->offsets, bw.dy_perm, sv->h,
                        g->d_w_down, nullptr);
  GemmProblem guw = gp(MOE_GEMM_TN, MOE_EPI_NONE, dt, dt, dt, E, A, 2 * f, D, sv->offsets, bw.dgu,
                       gather ? x : sv->x_perm, g->d_w_gateup, nullptr);
  guw.rows = gather ? sv->tok : nullptr;
  const GemmProblem dw_s = gp(MOE_GEMM_TN, MOE_EPI_NONE, dt, dt, dt, 1, T, D, F, nullptr, dy, sv->s_h,
                              g->d_s_down, nullptr);
  GemmProblem guw_s = gp(MOE_GEMM_TN, MOE_EPI_NONE, dt, dt, dt, 1, T, 2 * F, D, nullptr, bw.s_dgu, x,
                         g->d_s_gateup, nullptr);
  guw_s.rows = gather ? bw.iota : nullptr;
  const bool paired = !wg8 && F > 0 && T > 0 && gemm_big_pair_supported(dw_r, dw_s) &&
                      gemm_big_pair_supported(guw, guw_s);
  if (paired) {
    s = shared_down_dgrad();
    if (s) return s;
  }
  // 3. down weight gradient, 4. gate/up weight gradient (token rows of
  // x_perm, or of x through tok)
  if (paired) {
    MOE_STAGE(MOE_STAGE_DOWN_WGRAD, launch_gemm_big_pair(dw_r, dw_s, st));
    if (gather) MOE_TRY(launch_iota(bw.iota, T, st));
    MOE_STAGE(MOE_STAGE_GATE_UP_WGRAD, launch_gemm_big_pair(guw, guw_s, st));
  } else if (wg8) {
    MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, quant_w(bw.dy_perm, nullptr, sv->offsets, (int)E, A, D, bw.pad, bw.wa, bw.wsa));
    MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, quant_w(sv->h, nullptr, sv->offsets, (int)E, A, f, bw.pad, bw.wb, bw.wsb));
    MOE_STAGE(MOE_STAGE_DOWN_WGRAD, launch_gemm_fp8_wgrad(E, D, f, bw.pad, bw.wa, bw.wsa, bw.wb, bw.wsb,
                                                          g->d_w_down, st));
    MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, quant_w(bw.dgu, nullptr, sv->offsets, (int)E, A, 2 * f, bw.pad, bw.wa, bw.wsa));
    MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, quant_w(gather ? x : sv->x_perm, gather ? sv->tok : nullptr, sv->offsets,
                                              (int)E, A, D, bw.pad, bw.wb, bw.wsb));
    MOE_STAGE(MOE_STAGE_GATE_UP_WGRAD, launch_gemm_fp8_wgrad(E, 2 * f, D, bw.pad, bw.wa, bw.wsa, bw.wb, bw.wsb,
                                                             g->d_w_gateup, st));
  } else {
    MOE_STAGE(MOE_STAGE_DOWN_WGRAD, launch_grouped_gemm(dw_r, bw.gemm, bw.gemm_bytes, st));
    MOE_STAGE(MOE_STAGE_GATE_UP_WGRAD, launch_grouped_gemm(guw, bw.gemm, bw.gemm_bytes, st));
  }
  // 5. gate/up data gradient (written over dy_perm, which is no longer needed;
  // fp8: dG | dU in e4m3 per row against W_gu quantised along 2f, transposed)
  void* dx_perm = bw.dy_perm;
  if (fp8) {
    MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, launch_quantize_fp8(bw.dgu, dt, A, (int)(2 * f), bw.q, bw.qs, st, gf));
    MOE_STAGE(MOE_STAGE_GATE_UP_DGRAD, launch_gemm_fp8(MOE_EPI_NONE, E, A, D, 2 * f, sv->offsets, bw.q, bw.qs,
                                                       w8->gateup_tq, w8->gateup_ts, dx_perm, nullptr, nullptr, st,
                                                       gf));
  } else {
    MOE_STAGE(MOE_STAGE_GATE_UP_DGRAD, launch_grouped_gemm(gp(MOE_GEMM_NN, MOE_EPI_NONE, dt, dt, dt, E, A, 2 * f, D,
                                   sv->offsets, bw.dgu, w->w_gateup, dx_perm, nullptr),
                                nullptr, 0, st));
  }
  // 6. shared experts
  if (F > 0) {
    if (!paired) {
      s = shared_down_dgrad();
      if (s) return s;
    }
    if (paired) {
      // the weight gradients ran with the routed ones
    } else if (wg8) {
      MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, quant_w(dy, nullptr, nullptr, 1, T, D, bw.pad_s, bw.wa, bw.wsa));
      MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, quant_w(sv->s_h, nullptr, nullptr, 1, T, F, bw.pad_s, bw.wb, bw.wsb));
      MOE_STAGE(MOE_STAGE_SHARED_DOWN_WGRAD, launch_gemm_fp8_wgrad(1, D, F, bw.pad_s, bw.wa, bw.wsa, bw.wb, bw.wsb,
                                                                   g->d_s_down, st));
      MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, quant_w(bw.s_dgu, nullptr, nullptr, 1, T, 2 * F, bw.pad_s, bw.wa, bw.wsa));
      MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, quant_w(x, nullptr, nullptr, 1, T, D, bw.pad_s, bw.wb, bw.wsb));
      MOE_STAGE(MOE_STAGE_SHARED_GATE_UP_WGRAD, launch_gemm_fp8_wgrad(1, 2 * F, D, bw.pad_s, bw.wa, bw.wsa, bw.wb,
                                                                      bw.wsb, g->d_s_gateup, st));
    } else {
      MOE_STAGE(MOE_STAGE_SHARED_DOWN_WGRAD, launch_grouped_gemm(gp(MOE_GEMM_TN, MOE_EPI_NONE, dt, dt, dt, 1, T, D, F,
                                                                    nullptr, dy, sv->s_h, g->d_s_down, nullptr),
                                                                 bw.gemm, bw.gemm_bytes, st));
      MOE_STAGE(MOE_STAGE_SHARED_GATE_UP_WGRAD,
                launch_grouped_gemm(gp(MOE_GEMM_TN, MOE_EPI_NONE, dt, dt, dt, 1, T, 2 * F, D, nullptr, bw.s_dgu, x,
                                       g->d_s_gateup, nullptr),
                                    bw.gemm, bw.gemm_bytes, st));
    }
    if (fp8) {
      MOE_STAGE(MOE_STAGE_FP8_QUANTIZE, launch_quantize_fp8(bw.s_dgu, dt, T, (int)(2 * F), bw.q, bw.qs, st, gf));
      MOE_STAGE(MOE_STAGE_SHARED_GATE_UP_DGRAD,
                launch_gemm_fp8(MOE_EPI_NONE, 1, T, D, 2 * F, nullptr, bw.q, bw.qs, w8->s_gateup_tq,
                                w8->s_gateup_ts, bw.dx_shared, nullptr, nullptr, st, gf));
    } else {
      MOE_STAGE(MOE_STAGE_SHARED_GATE_UP_DGRAD, launch_grouped_gemm(gp(MOE_GEMM_NN, MOE_EPI_NONE, dt, dt, dt, 1, T, 2 * F, D,
                                     nullptr, bw.s_dgu, w->s_gateup, bw.dx_shared, nullptr),
                                  nullptr, 0, st));
    }
  }
  // 7. router weight gradient (fp32)
  MOE_STAGE(MOE_STAGE_ROUTER_WGRAD, launch_router_wgrad(bw.dlogits, x, dt, (int)T, (int)D, (int)E, (float*)bw.gemm,
                              g->d_w_router, st));
  // 8. input gradient: permuted rows + shared + router terms
  // the router term of dx runs over all experts when every logit can carry
  // gradient: a softmax without renormalisation, or any router with the
  // balance or z-loss terms on
  const int dense_router = ((d->score == MOE_SOFTMAX && !d->renorm) || terms_grad) ? 1 : 0;
  MOE_STAGE(MOE_STAGE_UNPERMUTE_SUM, launch_unpermute_sum(dt, dx_perm, sv->pos, F > 0 ? bw.dx_shared : nullptr, bw.dlogits,
                               sv->idx, w->w_router, dense_router, (int)T, (int)D, (int)E, (int)k,
                               dx, st));
  return MOE_OK;
}

int moe_backward(const moe_desc_t* d, const moe_weights_t* w, const void* x,
                 const moe_saved_t* sv, const void* dy, void* dx, const moe_grads_t* g,
                 const moe_router_terms_t* terms, float* losses, void* ws, size_t ws_bytes,
                 void* stream) {
  return backward_impl(d, w, nullptr, MOE_E4M3, 0, x, sv, dy, dx, g, terms, losses, ws, ws_bytes, stream);
}

int moe_backward_fp8(const moe_desc_t* d, const moe_weights_t* w, const moe_fp8_weights_t* w8,
                     int grad_format, int wgrad_fp8, const void* x, const moe_saved_t* sv, const void* dy,
                     void* dx, const moe_grads_t* g, const moe_router_terms_t* terms, float* losses, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!w8) return MOE_ERR_INVALID;
  return backward_impl(d, w, w8, grad_format, wgrad_fp8, x, sv, dy, dx, g, terms, losses, ws, ws_bytes,
                       stream);
}

int moe_fp8_weights_quantize(const moe_desc_t* d, const moe_weights_t* w, const moe_fp8_weights_t* w8,
                             int parts, void* stream) {
  int s = check_desc(d);
  if (s) return s;
  if (!w || !w8 || parts < 1 || parts > 3) return MOE_ERR_INVALID;
  s = fp8_layer_supported(d);
  if (s) return s;
  const int64_t D = d->d_model, E = d->num_experts, f = d->d_ff, F = shared_width(d);
  const int dt = d->dtype;
  const bool fwd = parts & MOE_FP8_FORWARD_LAYOUT, bwd = parts & MOE_FP8_BACKWARD_LAYOUT;
  if (!w->w_gateup || !w->w_down || (F > 0 && (!w->s_gateup || !w->s_down))) return MOE_ERR_INVALID;
  if (fwd && (!w8->gateup_q || !w8->gateup_s || !w8->down_q || !w8->down_s ||
              (F > 0 && (!w8->s_gateup_q || !w8->s_gateup_s || !w8->s_down_q || !w8->s_down_s))))
    return MOE_ERR_INVALID;
  if (bwd && (!w8->gateup_tq || !w8->gateup_ts || !w8->down_tq || !w8->down_ts ||
              (F > 0 && (!w8->s_gateup_tq || !w8->s_gateup_ts || !w8->s_down_tq || !w8->s_down_ts))))
    return MOE_ERR_INVALID;
  const void* ptrs[] = {w->w_gateup, w->w_down, w->s_gateup, w->s_down, w8->gateup_q, w8->gateup_s,
                        w8->down_q, w8->down_s, w8->gateup_tq, w8->gateup_ts, w8->down_tq, w8->down_ts,
                        w8->s_gateup_q, w8->s_gateup_s, w8->s_down_q, w8->s_down_s, w8->s_gateup_tq,
                        w8->s_gateup_ts, w8->s_down_tq, w8->s_down_ts};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  if (fwd) {
    MOE_TRY(launch_quantize_fp8(w->w_gateup, dt, E * 2 * f, (int)D, w8->gateup_q, w8->gateup_s, st));
    MOE_TRY(launch_quantize_fp8(w->w_down, dt, E * D, (int)f, w8->down_q, w8->down_s, st));
    if (F > 0) {
      MOE_TRY(launch_quantize_fp8(w->s_gateup, dt, 2 * F, (int)D, w8->s_gateup_q, w8->s_gateup_s, st));
      MOE_TRY(launch_quantize_fp8(w->s_down, dt, D, (int)F, w8->s_down_q, w8->s_down_s, st));
    }
  }
  if (bwd) {
    MOE_TRY(launch_quantize_fp8_transposed(w->w_gateup, dt, E, 2 * f, D, w8->gateup_tq, w8->gateup_ts, st));
    MOE_TRY(launch_quantize_fp8_transposed(w->w_down, dt, E, D, f, w8->down_tq, w8->down_ts, st));
    if (F > 0) {
      MOE_TRY(launch_quantize_fp8_transposed(w->s_gateup, dt, 1, 2 * F, D, w8->s_gateup_tq, w8->s_gateup_ts, st));
      MOE_TRY(launch_quantize_fp8_transposed(w->s_down, dt, 1, D, F, w8->s_down_tq, w8->s_down_ts, st));
    }
  }
  return MOE_OK;
}

int moe_quantize_fp8(int64_t rows, int64_t cols, int dtype, int format, const void* x, uint8_t* q,
                     float* scale, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 64 || cols > (int64_t(1) << 24)) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (format != MOE_E4M3 && format != MOE_E5M2) return MOE_ERR_INVALID;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scale) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return MOE_ERR_ALIGN;
  MOE_TRY(launch_quantize_fp8(x, dtype, rows, (int)cols, q, scale, (hipStream_t)stream,
                              format == MOE_E5M2 ? FP8_E5M2 : FP8_E4M3));
  return MOE_OK;
}

int moe_quantize_fp8_transposed(int64_t G, int64_t rows, int64_t cols, int dtype, const void* x,
                                uint8_t* q, float* scale, void* stream) {
  if (G < 0 || G > 65535 || rows < 0 || cols <= 0 || rows % 64 || cols % 64) return MOE_ERR_INVALID;
  if (rows > (int64_t(1) << 24) || cols > (int64_t(1) << 22)) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (G == 0 || rows == 0) return MOE_OK;
  if (!x || !q || !scale) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale)) return MOE_ERR_ALIGN;
  MOE_TRY(launch_quantize_fp8_transposed(x, dtype, G, rows, cols, q, scale, (hipStream_t)stream));
  return MOE_OK;
}

size_t moe_quantize_fp8_tensorwise_workspace_bytes(int64_t rows) {
  return rows < 0 ? 0 : quantize_fp8_tensorwise_ws_bytes(rows);
}

int moe_quantize_fp8_tensorwise(int64_t rows, int64_t cols, int dtype, const void* x, uint8_t* q,
                                float* scale, void* ws, size_t ws_bytes, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 64 || cols > (int64_t(1) << 24)) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scale || !ws) return MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(q) || !aligned16(scale) || !aligned16(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < quantize_fp8_tensorwise_ws_bytes(rows)) return MOE_ERR_WORKSPACE;
  MOE_TRY(launch_quantize_fp8_tensorwise(x, dtype, rows, (int)cols, q, scale, (float*)ws,
                                         (hipStream_t)stream));
  return MOE_OK;
}

int moe_grouped_gemm_fp8(int epi, int a_format, int64_t G, int64_t M, int64_t N, int64_t K,
                         const int32_t* offsets, const uint8_t* A, const float* a_scale,
                         const uint8_t* B, const float* b_scale, void* C, void* aux, void* stream) {
  if (epi != MOE_EPI_NONE && epi != MOE_EPI_SWIGLU && epi != MOE_EPI_DSWIGLU) return MOE_ERR_INVALID;
  if (a_format != MOE_E4M3 && a_format != MOE_E5M2) return MOE_ERR_INVALID;
  // e5m2 codes are the gradient operand of a data gradient: no SwiGLU epilogue
  if (a_format == MOE_E5M2 && epi == MOE_EPI_SWIGLU) return MOE_ERR_UNSUPPORTED;
  if (G < 1 || G > 256 || M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64) return MOE_ERR_INVALID;
  if (epi == MOE_EPI_DSWIGLU && M > 0 && !aux) return MOE_ERR_INVALID;
  if (epi == MOE_EPI_SWIGLU && (N / 2) % 128) return MOE_ERR_INVALID;
  if (M >= (int64_t(1) << 31) || N > 65536 || K > 65536) return MOE_ERR_UNSUPPORTED;
  if (!offsets && G != 1) return MOE_ERR_INVALID;
  if (M > 0 && (!A || !a_scale || !B || !b_scale || !C)) return MOE_ERR_INVALID;
  const void* ptrs[] = {offsets, A, a_scale, B, b_scale, C, aux};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  if (M == 0) return MOE_OK;
  MOE_TRY(launch_gemm_fp8(epi, G, M, N, K, offsets, A, a_scale, B, b_scale, C, aux, nullptr,
                          (hipStream_t)stream, a_format == MOE_E5M2 ? FP8_E5M2 : FP8_E4M3));
  return MOE_OK;
}

int moe_grouped_gemm_fp8_gather(int epi, int64_t G, int64_t M, int64_t N, int64_t K,
                                const int32_t* offsets, const uint8_t* A, const float* a_scale,
                                const uint8_t* B, const float* b_scale, void* C, void* aux,
                                const int32_t* rows, int64_t src_rows, void* stream) {
  if (epi != MOE_EPI_NONE && epi != MOE_EPI_SWIGLU) return MOE_ERR_INVALID;
  if (G < 1 || G > 256 || M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64 || src_rows < 0)
    return MOE_ERR_INVALID;
  if (epi == MOE_EPI_SWIGLU && (N / 2) % 128) return MOE_ERR_INVALID;
  if (M >= (int64_t(1) << 31) || N > 65536 || K > 65536) return MOE_ERR_UNSUPPORTED;
  // row byte offsets of the gathered codes are 32-bit in the kernel
  if (src_rows * K > (int64_t(1) << 32)) return MOE_ERR_UNSUPPORTED;
  if (!offsets && G != 1) return MOE_ERR_INVALID;
  if (M > 0 && (!A || !a_scale || !B || !b_scale || !C || !rows)) return MOE_ERR_INVALID;
  const void* ptrs[] = {offsets, A, a_scale, B, b_scale, C, aux, rows};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  if (M == 0) return MOE_OK;
  MOE_TRY(launch_gemm_fp8(epi, G, M, N, K, offsets, A, a_scale, B, b_scale, C, aux, rows,
                          (hipStream_t)stream));
  return MOE_OK;
}

size_t moe_quantize_fp8_colwise_bytes(int64_t G, int64_t M, int64_t C) {
  if (G < 1 || G > 256 || M < 0 || C <= 0) return 0;
  return colwise_bytes(G, M, C);
}

int moe_quantize_fp8_colwise(int64_t G, int64_t M, int64_t C, int dtype, const int32_t* offsets,
                             const int32_t* rows, int64_t src_rows, const void* x, int32_t* pad_offsets,
                             uint8_t* q, float* scale, void* stream) {
  if (G < 1 || G > 256 || M < 0 || C <= 0 || C % 64 || C > 65536 || src_rows < 0) return MOE_ERR_INVALID;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID;
  if (M >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  if (!offsets && G != 1) return MOE_ERR_INVALID;
  if (!pad_offsets || !q || !scale || (M > 0 && !x) || (rows && M > 0 && src_rows == 0)) return MOE_ERR_INVALID;
  const void* ptrs[] = {offsets, rows, x, pad_offsets, q, scale};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  MOE_TRY(launch_quantize_fp8_colwise(x, dtype, rows, offsets, (int)G, M, C, pad_offsets, q, scale,
                                      (hipStream_t)stream));
  return MOE_OK;
}

int moe_grouped_gemm_fp8_wgrad(int64_t G, int64_t N, int64_t K, const int32_t* pad_offsets, const uint8_t* A,
                               const float* a_scale, const uint8_t* B, const float* b_scale, void* C,
                               void* stream) {
  if (G < 1 || G > 256 || N <= 0 || K <= 0 || N % 64 || K % 64) return MOE_ERR_INVALID;
  if (N > 65536 || K > 65536) return MOE_ERR_UNSUPPORTED;
  if (!pad_offsets || !A || !a_scale || !B || !b_scale || !C) return MOE_ERR_INVALID;
  const void* ptrs[] = {pad_offsets, A, a_scale, B, b_scale, C};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_ALIGN;
  MOE_TRY(launch_gemm_fp8_wgrad(G, N, K, pad_offsets, A, a_scale, B, b_scale, C, (hipStream_t)stream));
  return MOE_OK;
}

int moe_bias_update(const moe_desc_t* d, const int32_t* counts, float rate, float* bias,
                    void* stream) {
  int s = check_desc(d);
  if (s) return s;
  if (!(rate == rate) || rate > 3.0e38f || rate < -3.0e38f) return MOE_ERR_INVALID;
  if (d->num_tokens == 0) return MOE_OK;
  if (!counts || !bias) return MOE_ERR_INVALID;
  if (!aligned16(counts) || !aligned16(bias)) return MOE_ERR_ALIGN;
  MOE_TRY(launch_bias_update(counts, (int)d->num_tokens, (int)d->num_experts, (int)d->top_k, rate, bias,
                             (hipStream_t)stream));
  return MOE_OK;
}

int moe_mfma_ceiling(int kind, int64_t iters, float* out, double* flop_per_launch, void* stream) {
  if (kind < MOE_MFMA_BF16_32X32X16 || kind > MOE_MFMA_E4M3_16X16X128 || iters < 1 || iters > (int64_t(1) << 30))
    return MOE_ERR_INVALID;
  if (!out || !flop_per_launch) return MOE_ERR_INVALID;
  if (!aligned16(out)) return MOE_ERR_ALIGN;
  // multiply-adds of one instruction of each kind
  static const double macs[4] = {32.0 * 32 * 16, 16.0 * 16 * 32, 32.0 * 32 * 64, 16.0 * 16 * 128};
  const int grid = mfma_rate_grid();
  *flop_per_launch = 2.0 * macs[kind] * 8.0 * (double)iters * (double)grid * 8.0;
  MOE_TRY(launch_mfma_rate(kind, iters, out, (hipStream_t)stream));
  return MOE_OK;
}

int moe_hbm_ceiling(const void* src, void* dst, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 || bytes > (int64_t(1) << 40)) return MOE_ERR_INVALID;
  if (bytes == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_INVALID;
  if (!aligned16(src) || !aligned16(dst)) return MOE_ERR_ALIGN;
  MOE_TRY(launch_stream_copy(src, dst, bytes / 16, (hipStream_t)stream));
  return MOE_OK;
}

int moe_stage_timing_mask(uint32_t mask) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (const StageRec& r : g_recs) g_spare.push_back(r);
  g_recs.clear();
  g_timing = mask & ((1u << MOE_NUM_STAGES) - 1u);
  return MOE_OK;
}

int moe_stage_timing(int enable) { return moe_stage_timing_mask(enable ? ~0u : 0u); }

int moe_stage_times(double* ms, int64_t* launches) {
  if (!ms || !launches) return MOE_ERR_INVALID;
  for (int i = 0; i < MOE_NUM_STAGES; ++i) {
    ms[i] = 0.0;
    launches[i] = 0;
  }
  std::lock_guard<std::mutex> lk(g_timing_mu);
  int status = MOE_OK;
  for (const StageRec& r : g_recs) {
    float t = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
      status = MOE_ERR_HIP;
    } else {
      ms[r.stage] += t;
      launches[r.stage] += 1;
    }
    g_spare.push_back(r);
  }
  g_recs.clear();
  return status;
}

}  // extern "C"

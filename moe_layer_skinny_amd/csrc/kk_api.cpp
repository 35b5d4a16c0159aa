// Host side of the C ABI (include/kk.h): argument validation, plan selection, workspace
// layout, the context (auxiliary stream + fork/join events), HIP graph capture/replay and
// optional per-kernel event timing.  All device work is in kk_gemv.hip / kk_mfma.hip.
//
// "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly", sections "Recovering
// time between operators" (per-batch kernel choice, the shared expert on another stream,
// fewer launches) and "Faster code needs targeted validation" (the chosen path must be
// visible to callers and tests: no silent fallback to another implementation).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/kk.h"
#include "kk_internal.h"

namespace {

thread_local std::string g_err;

kk_status fail(kk_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

kk_status hip_fail(hipError_t e, const char* what) {
  return fail(KK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxBatch = 64;
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 512;
constexpr int kMaxOprojSplits = 8;   // o-proj K chunks (7 on the split-K path)
constexpr int kMaxRouterSplits = 10;  // router logit partial slots (up to 10)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace carve-up (offsets in bytes from ws, each 256-byte aligned).
struct Layout {
  size_t h32, u32, logit_part, topk_idx, topk_gate, offsets, perm, inv_perm, act, n_act, vg, n_vg,
      status, A, As, Y, ys, oproj_part, total;
};

kk::Shape to_shape(const kk_config& c) {
  return kk::Shape{c.hidden, c.oproj_in, c.n_experts, c.top_k, c.inter, c.shared_inter, c.dtype,
                   c.routed_scale};
}

Layout make_layout(const kk_config& c, int Bm) {
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  const size_t slots = (size_t)Bm * c.top_k;
  L.h32 = take((size_t)Bm * c.hidden * 4);
  L.u32 = take((size_t)Bm * c.hidden * 4);  // normalised h (split-K path with a norm)
  L.logit_part = take((size_t)kMaxRouterSplits * Bm * c.n_experts * 4);  // [splits][Bm][E]
  L.topk_idx = take(slots * 4);
  L.topk_gate = take(slots * 4);
  L.offsets = take((size_t)(c.n_experts + 1) * 4);
  L.perm = take(slots * 4);
  L.inv_perm = take(slots * 4);
  L.act = take((size_t)std::max(c.n_experts, 64) * 4);  // read 64 lanes at a time
  L.n_act = take(16);
  L.vg = take((size_t)(c.n_experts + 64) * 4);  // pieces of <= 16 positions (<= E + B*k/16)
  L.n_vg = take(16);
  L.status = take(16);  // check of caller-supplied routing tables (kk_moe_decode)
  L.A = take(slots * c.inter * 4);
  L.As = take((size_t)Bm * c.shared_inter * 4);
  L.Y = take(slots * c.hidden * 4);
  L.ys = take((size_t)Bm * c.hidden * 4);
  // o-proj partials of the split-K path; reused afterwards by the gate/up partials (K chunks,
  // or the shared expert's split-K product)
  L.oproj_part = take(std::max((size_t)kMaxOprojSplits * Bm * c.hidden,
                               kk::mfma_scratch_floats(to_shape(c), Bm)) * 4);
  L.total = o;
  return L;
}


bool misaligned(const void* p, size_t a = 16) { return ((uintptr_t)p) % a != 0; }

kk_status validate_cfg(const kk_config* c, int32_t max_batch) {
  if (!c) return fail(KK_ERR_INVALID_ARG, "config is NULL");
  if (max_batch < 1 || max_batch > kMaxBatch)
    return fail(KK_ERR_INVALID_ARG, "max_batch %d outside 1..%d", max_batch, kMaxBatch);
  if (c->dtype != KK_F32 && c->dtype != KK_BF16)
    return fail(KK_ERR_INVALID_ARG, "dtype %d is neither KK_F32 nor KK_BF16", c->dtype);
  if (c->hidden <= 0 || c->oproj_in <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->inter <= 0 ||
      c->shared_inter <= 0)
    return fail(KK_ERR_INVALID_ARG, "every dimension must be positive");
  if (c->top_k > c->n_experts)
    return fail(KK_ERR_INVALID_ARG, "top_k %d > n_experts %d", c->top_k, c->n_experts);
  if (!(c->routed_scale > 0.f) || c->routed_scale != c->routed_scale)
    return fail(KK_ERR_INVALID_ARG, "routed_scale must be a positive number");
  if (!(c->norm_eps >= 0.f && c->norm_eps <= 3.4e38f))
    return fail(KK_ERR_INVALID_ARG, "norm_eps must be a finite number >= 0");
  if (c->top_k > kMaxTopK)
    return fail(KK_ERR_UNSUPPORTED, "top_k %d > %d", c->top_k, kMaxTopK);
  if (c->n_experts > kMaxExperts)
    return fail(KK_ERR_UNSUPPORTED, "n_experts %d > %d", c->n_experts, kMaxExperts);
  const int esz = c->dtype == KK_BF16 ? 2 : 4;
  if ((c->hidden * esz) % 16 || (c->oproj_in * esz) % 16 || (c->inter * esz) % 16 ||
      (c->shared_inter * esz) % 16)
    return fail(KK_ERR_INVALID_ARG, "rows must be whole 16-byte chunks (H, Ko, I, Is multiple of %d)",
                16 / esz);
  kk::Shape s = to_shape(*c);
  if (c->dtype == KK_BF16) {
    if (!(s.H == 7168 && (s.Ko == 7168 || s.Ko == 448) && (s.I == 2048 || s.I == 128) && s.I == s.Is))
      return fail(KK_ERR_UNSUPPORTED,
                  "bf16 shapes supported: H=7168, Ko in {448,7168}, I=Is in {128,2048}");
  } else {
    if (!(s.H == 256 && s.Ko == 256 && s.I == 128 && s.Is == 128))
      return fail(KK_ERR_UNSUPPORTED, "fp32 shapes supported: H=Ko=256, I=Is=128");
    if (max_batch > 2) return fail(KK_ERR_UNSUPPORTED, "fp32 layers run batch <= 2 only");
  }
  return KK_OK;
}

const char* kernel_names[] = {"oproj_gemv",  "router_logits_shared", "router_logits",
                              "gateup_gemv_shared", "gateup_gemv_routed", "topk_gateup_gemv_routed",
                              "down_combine_gemv", "moe_prep",    "combine",    "oproj_mfma",
                              "oproj_reduce", "router_mfma", "gateup_mfma", "down_mfma",
                              "topk_rows",   "tables", "topk_tables", "oproj_reduce_norm",
                              "norm_rows", "prefetch", "oproj_router_gemv",
                              "topk_shared_gateup_gemv", "oproj_router_mfma", "shared_mfma"};
enum KName {
  K_OPROJ, K_LOGITS_SHARED, K_LOGITS, K_GU_SHARED, K_GU_ROUTED, K_TOPK_GU, K_DOWN, K_PREP,
  K_COMBINE, K_OPROJ_MFMA, K_OPROJ_REDUCE, K_ROUTER_MFMA, K_GU_MFMA, K_DOWN_MFMA, K_TOPK_ROWS,
  K_TABLES, K_TOPK_TABLES, K_OPROJ_REDUCE_NORM, K_NORM_ROWS, K_PREFETCH, K_OPROJ_ROUTER,
  K_TOPK_SHARED_GU, K_OPROJ_ROUTER_MFMA, K_SHARED_MFMA
};

struct TimingRec {
  int name;
  hipEvent_t a, b;
};

struct GraphEntry {
  int B;
  uint32_t flags;
  int path;  // the plan the step was captured with (KK_FORCE_PLAN may change it)
  const void *x, *r, *out, *idx, *gate, *ws;
  hipStream_t stream;
  hipGraphExec_t exec;
  unsigned long long uses;
};

// A captured chain of layers (kept by its first context).
struct ChainGraph {
  std::vector<uintptr_t> key;  // context serials, x[], out[], plan paths, resid, ws, stream
  int B;
  uint32_t flags;
  hipGraphExec_t exec;
  unsigned long long uses;
};

}  // namespace

struct kk_ctx {
  unsigned long long serial;  // never reused: chain graphs of other contexts key on it
  kk_config cfg;
  kk::Shape shape;
  kk::Weights w;
  kk::Norm norm;  // gamma == nullptr: no norm
  void* mr = nullptr;  // router-o-proj product W_r W_o (GEMV path without a norm), owned
  int max_batch;
  int device;
  kk::Device dev;
  Layout L;
  hipStream_t aux = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  std::vector<GraphEntry> graphs;
  std::vector<ChainGraph> chains;
  unsigned long long clock = 0;
  bool timing = false;
  long long wall_khz = 0;        // constant-rate device clock, for the delay test hook
  long long delay_ticks[2] = {0, 0};  // main stream / auxiliary stream delays (test hook)
  std::vector<TimingRec> trecs;
  std::vector<hipEvent_t> tpool;
  void* scratch = nullptr;            // this device's static scratch (kk_layer_decode_static)
  hipError_t scratch_err = hipSuccess;
  bool no_alloc = false;              // inside kk_layer_decode_static: no timing events
};

namespace {

int forced_path() {
  const char* f = std::getenv("KK_FORCE_PLAN");
  if (!f || !*f) return -1;
  if (!std::strcmp(f, "gemv")) return KK_PATH_GEMV;
  if (!std::strcmp(f, "mfma") || !std::strcmp(f, "splitk")) return KK_PATH_SPLITK_MFMA;
  return -2;
}

// Whether batch B on the GEMV path runs the three-launch step (the router from r and x in the
// o-proj's launch): with a 448-wide o-proj slice at both batches; at full width only for two
// tokens, where the removed router launch gains more than the 11 MB product costs (one token:
// 158.5 against 157.8 us per step, two: 282 against 291).
bool gemv_fused(const kk_ctx* c, int B) {
  return c->mr != nullptr && (c->shape.Ko < c->shape.H || B == 2);
}

// Whether batch B on the split-K path runs the o-proj and the router as one launch (a layer with
// the router-o-proj product and a 448-wide o-proj slice: at full width the product's split-K
// units would cost about what the saved launches gain).
bool mfma_fused(const kk_ctx* c, int B) { return c->mr != nullptr && c->shape.Ko < c->shape.H; }

kk_status plan_for(const kk_ctx* c, int B, kk_plan* p) {
  std::memset(p, 0, sizeof *p);
  const int f = forced_path();
  if (f == -2) return fail(KK_ERR_INVALID_ARG, "KK_FORCE_PLAN must be 'gemv' or 'mfma'");
  p->forced = f >= 0;
  p->path = f >= 0 ? f : (B <= 2 ? KK_PATH_GEMV : KK_PATH_SPLITK_MFMA);
  p->streams = 1;
  if (p->path == KK_PATH_GEMV) {
    if (!kk::gemv_supported(c->shape, B))
      return fail(KK_ERR_UNSUPPORTED, "GEMV path has no kernels for batch %d of this shape", B);
    const size_t lds_down = kk::down_combine_gemv_lds(c->shape, c->dev, B, true);
    if ((long)lds_down > c->dev.max_lds)
      return fail(KK_ERR_UNSUPPORTED, "GEMV down-projection needs %zu B of LDS (device: %d)",
                  lds_down, c->dev.max_lds);
    p->oproj_splitk = 1;
    if (gemv_fused(c, B)) {
      // o-proj + router logits (from x and r), top-k + shared gate/up + routed gate/up,
      // routed + shared down + combine
      p->router_splitk = kk::router_fused_splits(c->shape);
      p->kernels_per_step = 3;
    } else {
      // oproj, router logits + shared gate/up, top-k + shared down + routed gate/up,
      // routed down + combine
      p->router_splitk = kk::router_gemv_splits(c->shape);
      p->kernels_per_step = 4;
    }
    return KK_OK;
  }
  if (!kk::mfma_supported(c->shape, B))
    return fail(KK_ERR_UNSUPPORTED, "split-K MFMA path has no kernels for batch %d of this shape",
                B);
  p->oproj_splitk = kk::mfma_oproj_splits(c->shape);
  p->router_splitk = kk::mfma_router_splits(c->shape);
  // oproj, reduce, router logits, top-k rows + tables (one launch up to 16 tokens), gate/up,
  // down, combine; a gate/up over K chunks adds the SwiGLU launch that sums them, and over 32
  // tokens an unsplit gate/up adds the shared expert's split-K launch and its SwiGLU
  const bool split = kk::mfma_gateup_split(c->shape, B);
  p->kernels_per_step = (B > 16 ? 8 : 7) + (split ? 1 : 0) + (B > 32 && !split ? 2 : 0);
  // (a small intermediate up to 16 tokens: the down-projection sums the K chunks itself)
  if (kk::mfma_swiglu_in_down(c->shape, B)) p->kernels_per_step -= 1;
  if (mfma_fused(c, B)) {
    // o-proj (with the residual) + router logits from x and r in one launch: no reduce and
    // no router launch
    p->router_splitk = kk::mfma_fused_splits(c->shape);
    p->kernels_per_step -= 2;
  }
  return KK_OK;
}

hipEvent_t pool_event(kk_ctx* c) {
  if (!c->tpool.empty()) {
    hipEvent_t e = c->tpool.back();
    c->tpool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

// Runs one launch, bracketed by timing events when enabled (never inside a capture).
template <typename F>
hipError_t timed(kk_ctx* c, int name, hipStream_t s, F&& launch) {
  if (!c->timing || c->no_alloc || capturing(s)) return launch();
  TimingRec r{name, pool_event(c), pool_event(c)};
  if (r.a) (void)hipEventRecord(r.a, s);
  hipError_t e = launch();
  if (r.b) (void)hipEventRecord(r.b, s);
  if (r.a && r.b) c->trecs.push_back(r);
  return e;
}

struct WsPtrs {
  float* h32;
  float* u32;
  float* logit_part;
  int32_t* topk_idx;
  float* topk_gate;
  int32_t* offsets;
  int32_t* perm;
  int32_t* inv_perm;
  int32_t* act;
  int32_t* n_act;
  int32_t* vg;
  int32_t* n_vg;
  int32_t* status;
  float* A;
  float* As;
  float* Y;
  float* ys;
  float* oproj_part;
};

WsPtrs carve(const Layout& L, void* ws) {
  char* b = (char*)ws;
  return WsPtrs{(float*)(b + L.h32),     (float*)(b + L.u32),        (float*)(b + L.logit_part), (int32_t*)(b + L.topk_idx),
                (float*)(b + L.topk_gate), (int32_t*)(b + L.offsets),  (int32_t*)(b + L.perm),
                (int32_t*)(b + L.inv_perm), (int32_t*)(b + L.act),    (int32_t*)(b + L.n_act),
                (int32_t*)(b + L.vg),       (int32_t*)(b + L.n_vg),  (int32_t*)(b + L.status),
                (float*)(b + L.A),         (float*)(b + L.As),         (float*)(b + L.Y),
                (float*)(b + L.ys),         (float*)(b + L.oproj_part)};
}

kk_status check_common(const kk_ctx* c, int B, void* ws) {
  if (!c) return fail(KK_ERR_INVALID_ARG, "context is NULL");
  if (B < 1 || B > c->max_batch)
    return fail(KK_ERR_INVALID_ARG, "batch %d outside 1..%d (max_batch of this context)", B,
                c->max_batch);
  if (!ws) return fail(KK_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", c->L.total);
  if (misaligned(ws, 256)) return fail(KK_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != c->device)
    return fail(KK_ERR_INVALID_ARG, "current device %d is not the context's device %d", dev,
                c->device);
  return KK_OK;
}

#define KK_PTR(p, name)                                                            \
  do {                                                                             \
    if (!(p)) return fail(KK_ERR_INVALID_ARG, "%s is NULL", name);                 \
    if (misaligned(p)) return fail(KK_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

#define KK_HIP(expr, what)                      \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// ---- step pieces ------------------------------------------------------------------------
// With u32 (and a norm): the split-K path's reduce also writes u32 = norm(h32); the GEMV path
// leaves the norm to the launches that read u.
kk_status enqueue_oproj(kk_ctx* c, int B, const void* x, const void* r, float* h32, void* h_out,
                        float* part, float* u32, int path, hipStream_t s) {
  if (path == KK_PATH_GEMV) {
    KK_HIP(timed(c, K_OPROJ, s,
                 [&] {
                   return kk::launch_oproj_gemv(c->shape, c->dev, B, x, r, c->w.w_o, h32, h_out, s);
                 }),
           "oproj launch");
    return KK_OK;
  }
  KK_HIP(timed(c, K_OPROJ_MFMA, s,
               [&] { return kk::launch_oproj_mfma(c->shape, c->dev, B, x, part, c->w.w_o, s); }),
         "oproj launch");
  if (u32 && c->norm.gamma) {
    KK_HIP(timed(c, K_OPROJ_REDUCE_NORM, s,
                 [&] { return kk::launch_norm_rows(c->shape, B, part, r, h32, h_out, c->norm, u32, s); }),
           "oproj reduce + norm launch");
    return KK_OK;
  }
  KK_HIP(timed(c, K_OPROJ_REDUCE, s,
               [&] { return kk::launch_oproj_reduce(c->shape, B, part, r, h32, h_out, s); }),
         "oproj reduce launch");
  return KK_OK;
}

// Split-K path on its own (router / experts from a caller's h32): u32 = norm(h32) when the
// context has a norm; returns the rows the path should read (u32 or h32).
const float* enqueue_norm_from_h32(kk_ctx* c, int B, const float* h32, float* u32, hipStream_t s,
                                   kk_status* st) {
  *st = KK_OK;
  if (!c->norm.gamma) return h32;
  hipError_t e = timed(c, K_NORM_ROWS, s, [&] {
    return kk::launch_norm_rows(c->shape, B, nullptr, nullptr, const_cast<float*>(h32), nullptr,
                                c->norm, u32, s);
  });
  if (e != hipSuccess) *st = hip_fail(e, "norm launch");
  return u32;
}

// Top-k rows and routing tables from logit partials: one launch up to 16 tokens, else one
// wave-per-token launch and a tables launch.
kk_status enqueue_topk(kk_ctx* c, int B, const float* logit_part, int splits,
                       const kk::Routing& rt, hipStream_t s) {
  if (B <= 16) {
    KK_HIP(timed(c, K_TOPK_TABLES, s,
                 [&] {
                   return kk::launch_topk_tables(c->shape, B, logit_part, splits, c->w.bias, rt, s);
                 }),
           "top-k launch");
    return KK_OK;
  }
  KK_HIP(timed(c, K_TOPK_ROWS, s,
               [&] { return kk::launch_topk_rows(c->shape, B, logit_part, splits, c->w.bias, rt, s); }),
         "top-k launch");
  KK_HIP(timed(c, K_TABLES, s, [&] { return kk::launch_tables(c->shape, B, rt, s); }),
         "routing tables launch");
  return KK_OK;
}

// MFMA path: router logits from u (h32 or its normalised rows), then the top-k and tables.
kk_status enqueue_router_mfma(kk_ctx* c, int B, const float* u, const kk::Routing& rt,
                              float* logit_part, hipStream_t s) {
  KK_HIP(timed(c, K_ROUTER_MFMA, s,
               [&] { return kk::launch_router_mfma(c->shape, c->dev, B, u, c->w.w_r, logit_part, s); }),
         "router logits launch");
  return enqueue_topk(c, B, logit_part, kk::mfma_router_splits(c->shape), rt, s);
}

// MFMA path, KK_TWO_STREAM: the shared expert's gate/up and down-projection on the auxiliary
// stream from u (forked here, joined before the combine), the same kernels as in the grouped
// launches restricted to the shared group, so the bits are the same.  They read no routing table
// and write only As / ys and the shared positions of the gate/up scratch.
kk_status fork_shared_mfma(kk_ctx* c, int B, const float* u, const kk::Routing& rt,
                           const WsPtrs& p, hipStream_t s) {
  KK_HIP(hipEventRecord(c->ev_fork, s), "fork event");
  KK_HIP(hipStreamWaitEvent(c->aux, c->ev_fork, 0), "aux wait");
  KK_HIP(kk::launch_delay(c->delay_ticks[1], c->aux), "delay launch");
  KK_HIP(timed(c, K_SHARED_MFMA, c->aux,
               [&] {
                 hipError_t e = kk::launch_gateup_mfma(c->shape, c->dev, B, u, c->w.w13, c->w.ws13,
                                                       rt, p.A, p.As, p.oproj_part, c->aux,
                                                       kk::kGroupsSharedOnly);
                 if (e != hipSuccess) return e;
                 return kk::launch_down_mfma(c->shape, c->dev, B, p.A, p.As, c->w.w2, c->w.ws2, rt,
                                             p.Y, p.ys, p.oproj_part, c->aux,
                                             kk::kGroupsSharedOnly);
               }),
         "shared expert launches");
  KK_HIP(hipEventRecord(c->ev_join, c->aux), "join event");
  return KK_OK;
}

// MFMA path: grouped gate/up (from u) and down over the active experts plus the shared one
// (the active experts only when two_stream: the shared expert was forked), combine (onto h32).
kk_status enqueue_experts_mfma(kk_ctx* c, int B, const float* u, const float* h32,
                               const kk::Routing& rt, const WsPtrs& p, void* out, hipStream_t s,
                               bool two_stream = false) {
  const int sel = two_stream ? kk::kGroupsRoutedOnly : kk::kGroupsEvery;
  KK_HIP(timed(c, K_GU_MFMA, s,
               [&] {
                 // (the o-proj partials are consumed by now: their region is scratch)
                 return kk::launch_gateup_mfma(c->shape, c->dev, B, u, c->w.w13, c->w.ws13, rt,
                                               p.A, p.As, p.oproj_part, s, sel);
               }),
         "gate/up launch");
  KK_HIP(timed(c, K_DOWN_MFMA, s,
               [&] {
                 return kk::launch_down_mfma(c->shape, c->dev, B, p.A, p.As, c->w.w2, c->w.ws2, rt,
                                             p.Y, p.ys, p.oproj_part, s, sel);
               }),
         "down launch");
  if (two_stream) KK_HIP(hipStreamWaitEvent(s, c->ev_join, 0), "join wait");
  KK_HIP(timed(c, K_COMBINE, s,
               [&] { return kk::launch_combine(c->shape, B, h32, p.Y, p.ys, rt, out, s); }),
         "combine launch");
  return KK_OK;
}

// GEMV path: router logit partials (with ws13: and the shared expert's gate/up).
kk_status enqueue_logits(kk_ctx* c, int B, const float* h32, const kk::Routing& rt,
                         float* logit_part, const void* ws13, float* As, hipStream_t s) {
  KK_HIP(timed(c, ws13 ? K_LOGITS_SHARED : K_LOGITS, s,
               [&] {
                 return kk::launch_router_logits(c->shape, c->dev, B, h32, c->w.w_r, logit_part,
                                                 ws13, rt, As, c->norm, s);
               }),
         "router logits launch");
  return KK_OK;
}

kk_status enqueue_shared_gateup(kk_ctx* c, int B, const float* h32, const kk::Routing& rt,
                                float* As, hipStream_t s) {
  KK_HIP(timed(c, K_GU_SHARED, s,
               [&] {
                 kk::GateupExtras x;
                 x.norm = c->norm;
                 return kk::launch_gateup_gemv(c->shape, c->dev, B, h32, c->w.ws13, true, rt, As,
                                               x, s);
               }),
         "shared gate/up launch");
  return KK_OK;
}

// Routed gate/up (with the shared expert's down-projection in its first moments; with
// logit_part: after running the top-k itself), then the routed down-projection and the
// combine, on s.
kk_status enqueue_routed_and_combine(kk_ctx* c, int B, const float* h32, const kk::Routing& rt,
                                     const WsPtrs& p, const float* logit_part, void* out,
                                     hipStream_t s) {
  kk::GateupExtras x;
  if (logit_part) {
    x.part = logit_part;
    x.splits = kk::router_gemv_splits(c->shape);
    x.bias = c->w.bias;
  }
  x.ws2 = c->w.ws2;
  x.As = p.As;
  x.ys = p.ys;
  x.norm = c->norm;
  KK_HIP(timed(c, logit_part ? K_TOPK_GU : K_GU_ROUTED, s,
               [&] {
                 return kk::launch_gateup_gemv(c->shape, c->dev, B, h32, c->w.w13, false, rt, p.A,
                                               x, s);
               }),
         "routed gate/up launch");
  KK_HIP(timed(c, K_DOWN, s,
               [&] {
                 return kk::launch_down_combine_gemv(c->shape, c->dev, B, p.A, p.ys, c->w.w2, h32,
                                                     rt, out, nullptr, nullptr, s);
               }),
         "down + combine launch");
  return KK_OK;
}

// Prefetch of the next layer's first weights on `owner`'s auxiliary stream, forked from s
// after this layer's o-proj (the join is left to the caller).
struct PrefetchNext {
  kk_ctx* owner;
  const kk_ctx* next;
};

kk_status enqueue_prefetch(const PrefetchNext& pf, hipStream_t s) {
  kk_ctx* o = pf.owner;
  const kk::Shape& sh = pf.next->shape;
  const size_t eb = sh.dtype == 1 ? 2 : 4;
  KK_HIP(hipEventRecord(o->ev_fork, s), "prefetch fork event");
  KK_HIP(hipStreamWaitEvent(o->aux, o->ev_fork, 0), "prefetch fork wait");
  KK_HIP(kk::launch_delay(o->delay_ticks[1], o->aux), "delay launch");
  const struct {
    const void* p;
    size_t bytes;
  } parts[] = {{pf.next->w.w_o, eb * sh.H * sh.Ko},
               {pf.next->w.w_r, eb * sh.E * sh.H},
               {pf.next->w.ws13, eb * 2 * sh.Is * sh.H}};
  for (const auto& q : parts)
    KK_HIP(timed(o, K_PREFETCH, o->aux,
                 [&] { return kk::launch_prefetch(o->dev, q.p, q.bytes, o->aux); }),
           "prefetch launch");
  KK_HIP(hipEventRecord(o->ev_join, o->aux), "prefetch join event");
  return KK_OK;
}

// GEMV step in three launches, for a layer with the router-o-proj product at the batches
// gemv_fused picks: o-proj + router logits from x and r; the top-k in every block of the routed gate/up launch,
// covered by the shared expert's gate/up (or, two_stream, that gate/up on the auxiliary stream,
// joined before the last launch); routed and shared down-projection with the combine.
kk_status enqueue_layer_gemv3(kk_ctx* c, int B, const void* x, const void* r, void* out,
                              const kk::Routing& rt, const WsPtrs& p, hipStream_t s,
                              bool two_stream, const PrefetchNext* pf) {
  KK_HIP(timed(c, K_OPROJ_ROUTER, s,
               [&] {
                 return kk::launch_oproj_router_gemv(c->shape, c->dev, B, x, r, c->w.w_o, c->w.w_r,
                                                     c->mr, p.h32, nullptr, p.logit_part, s);
               }),
         "o-proj + router launch");
  if (pf) {
    kk_status st = enqueue_prefetch(*pf, s);
    if (st != KK_OK) return st;
  }
  kk::GateupExtras gx;
  gx.part = p.logit_part;
  gx.splits = kk::router_fused_splits(c->shape);
  gx.bias = c->w.bias;
  if (two_stream) {
    KK_HIP(hipEventRecord(c->ev_fork, s), "fork event");
    KK_HIP(hipStreamWaitEvent(c->aux, c->ev_fork, 0), "aux wait");
    KK_HIP(kk::launch_delay(c->delay_ticks[1], c->aux), "delay launch");
    kk_status st = enqueue_shared_gateup(c, B, p.h32, rt, p.As, c->aux);
    if (st != KK_OK) return st;
    KK_HIP(hipEventRecord(c->ev_join, c->aux), "join event");
  } else {
    gx.ws13 = c->w.ws13;
    gx.As_out = p.As;
  }
  KK_HIP(timed(c, two_stream ? K_TOPK_GU : K_TOPK_SHARED_GU, s,
               [&] {
                 return kk::launch_gateup_gemv(c->shape, c->dev, B, p.h32, c->w.w13, false, rt, p.A,
                                               gx, s);
               }),
         "routed gate/up launch");
  if (two_stream) KK_HIP(hipStreamWaitEvent(s, c->ev_join, 0), "join wait");
  KK_HIP(timed(c, K_DOWN, s,
               [&] {
                 return kk::launch_down_combine_gemv(c->shape, c->dev, B, p.A, p.ys, c->w.w2, p.h32,
                                                     rt, out, c->w.ws2, p.As, s);
               }),
         "down + combine launch");
  return KK_OK;
}

kk_status enqueue_layer(kk_ctx* c, int B, const void* x, const void* r, void* out, int32_t* idx,
                        float* gate, void* ws, hipStream_t s, bool two_stream, int path,
                        const PrefetchNext* pf = nullptr, const Layout* lay = nullptr) {
  WsPtrs p = carve(lay ? *lay : c->L, ws);
  kk::Routing rt{idx ? idx : p.topk_idx, gate ? gate : p.topk_gate, p.offsets, p.perm,
                 p.inv_perm, p.act, p.n_act, p.vg, p.n_vg};
  KK_HIP(kk::launch_delay(c->delay_ticks[0], s), "delay launch");
  if (path == KK_PATH_GEMV && gemv_fused(c, B)) return enqueue_layer_gemv3(c, B, x, r, out, rt, p, s, two_stream, pf);
  if (path == KK_PATH_SPLITK_MFMA && mfma_fused(c, B)) {
    KK_HIP(timed(c, K_OPROJ_ROUTER_MFMA, s,
                 [&] {
                   return kk::launch_oproj_router_mfma(c->shape, c->dev, B, x, r, c->w.w_o, c->w.w_r,
                                                       c->mr, p.h32, p.oproj_part, p.logit_part, s);
                 }),
           "o-proj + router launch");
    if (pf) {
      kk_status st = enqueue_prefetch(*pf, s);
      if (st != KK_OK) return st;
    }
    kk_status st = two_stream ? fork_shared_mfma(c, B, p.h32, rt, p, s) : KK_OK;
    if (st != KK_OK) return st;
    st = enqueue_topk(c, B, p.logit_part, kk::mfma_fused_splits(c->shape), rt, s);
    if (st != KK_OK) return st;
    return enqueue_experts_mfma(c, B, p.h32, p.h32, rt, p, out, s, two_stream);
  }
  kk_status st = enqueue_oproj(c, B, x, r, p.h32, nullptr, p.oproj_part, p.u32, path, s);
  if (st != KK_OK) return st;
  if (pf && (st = enqueue_prefetch(*pf, s)) != KK_OK) return st;
  if (path == KK_PATH_SPLITK_MFMA) {
    const float* u = c->norm.gamma ? p.u32 : p.h32;
    if (two_stream && (st = fork_shared_mfma(c, B, u, rt, p, s)) != KK_OK) return st;
    st = enqueue_router_mfma(c, B, u, rt, p.logit_part, s);
    if (st != KK_OK) return st;
    return enqueue_experts_mfma(c, B, u, p.h32, rt, p, out, s, two_stream);
  }
  if (!two_stream) {
    // the shared expert's gate/up streams with the router logits, its down-projection
    // with the top-k at the start of the routed gate/up launch
    st = enqueue_logits(c, B, p.h32, rt, p.logit_part, c->w.ws13, p.As, s);
    if (st != KK_OK) return st;
    return enqueue_routed_and_combine(c, B, p.h32, rt, p, p.logit_part, out, s);
  }
  // shared expert's gate/up on the auxiliary stream, joined before the routed gate/up
  KK_HIP(hipEventRecord(c->ev_fork, s), "fork event");
  KK_HIP(hipStreamWaitEvent(c->aux, c->ev_fork, 0), "aux wait");
  KK_HIP(kk::launch_delay(c->delay_ticks[1], c->aux), "delay launch");
  st = enqueue_shared_gateup(c, B, p.h32, rt, p.As, c->aux);
  if (st != KK_OK) return st;
  KK_HIP(hipEventRecord(c->ev_join, c->aux), "join event");
  st = enqueue_logits(c, B, p.h32, rt, p.logit_part, nullptr, nullptr, s);
  if (st != KK_OK) return st;
  KK_HIP(hipStreamWaitEvent(s, c->ev_join, 0), "join wait");
  return enqueue_routed_and_combine(c, B, p.h32, rt, p, p.logit_part, out, s);
}

void destroy_graphs(kk_ctx* c) {
  for (auto& g : c->graphs) (void)hipGraphExecDestroy(g.exec);
  c->graphs.clear();
  for (auto& g : c->chains) (void)hipGraphExecDestroy(g.exec);
  c->chains.clear();
}

// The layers in order on s; with prefetch, each layer but the last forks the next layer's
// weight prefetch after its o-proj, and s joins the auxiliary stream at the end.
kk_status enqueue_chain(kk_ctx* const* ctx, int L, int B, const void* const* x, const void* resid,
                        void* const* out, void* ws, hipStream_t s, bool prefetch) {
  for (int l = 0; l < L; ++l) {
    kk_plan plan;
    kk_status st = plan_for(ctx[l], B, &plan);
    if (st != KK_OK) return st;
    const PrefetchNext pf{ctx[0], l + 1 < L ? ctx[l + 1] : nullptr};
    st = enqueue_layer(ctx[l], B, x[l], l == 0 ? resid : out[l - 1], out[l], nullptr, nullptr, ws,
                       s, false, plan.path, prefetch && l + 1 < L ? &pf : nullptr);
    if (st != KK_OK) return st;
  }
  if (prefetch && L > 1) KK_HIP(hipStreamWaitEvent(s, ctx[0]->ev_join, 0), "prefetch join wait");
  return KK_OK;
}

}  // namespace

extern "C" {

const char* kk_status_string(kk_status s) {
  switch (s) {
    case KK_OK: return "KK_OK";
    case KK_ERR_INVALID_ARG: return "KK_ERR_INVALID_ARG";
    case KK_ERR_UNSUPPORTED: return "KK_ERR_UNSUPPORTED";
    case KK_ERR_WORKSPACE: return "KK_ERR_WORKSPACE";
    case KK_ERR_HIP: return "KK_ERR_HIP";
  }
  return "KK_ERR_UNKNOWN";
}

const char* kk_last_error(void) { return g_err.c_str(); }

kk_status kk_validate(const kk_config* cfg, int32_t max_batch) {
  try {
    return validate_cfg(cfg, max_batch);
  } catch (...) {
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_validate");
  }
}

size_t kk_workspace_bytes(const kk_config* cfg, int32_t max_batch) {
  if (validate_cfg(cfg, max_batch) != KK_OK) return 0;
  return make_layout(*cfg, max_batch).total;
}

kk_status kk_create(const kk_config* cfg, const kk_weights* w, int32_t max_batch, kk_ctx** out) {
  try {
    if (!out) return fail(KK_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    kk_status st = validate_cfg(cfg, max_batch);
    if (st != KK_OK) return st;
    if (!w) return fail(KK_ERR_INVALID_ARG, "weights is NULL");
    KK_PTR(w->w_o, "w_o");
    KK_PTR(w->w_r, "w_r");
    KK_PTR(w->router_bias, "router_bias");
    KK_PTR(w->w13, "w13");
    KK_PTR(w->w2, "w2");
    KK_PTR(w->ws13, "ws13");
    KK_PTR(w->ws2, "ws2");
    if (w->norm_weight && misaligned(w->norm_weight))
      return fail(KK_ERR_INVALID_ARG, "norm_weight is not 16-byte aligned");
    static std::atomic<unsigned long long> serials{0};
    kk_ctx* c = new kk_ctx();
    c->serial = ++serials;
    c->cfg = *cfg;
    c->shape = to_shape(*cfg);
    c->w = kk::Weights{w->w_o, w->w_r, w->router_bias, w->w13, w->w2, w->ws13, w->ws2};
    c->norm.gamma = w->norm_weight;
    c->norm.eps = cfg->norm_eps;
    c->max_batch = max_batch;
    c->L = make_layout(*cfg, max_batch);
    auto bail = [&](hipError_t e, const char* what) {
      kk_destroy(c);
      return hip_fail(e, what);
    };
    hipError_t e = hipGetDevice(&c->device);
    if (e != hipSuccess) return bail(e, "hipGetDevice");
    int ncu = 0, lds = 0;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, c->device);
    if (e != hipSuccess) return bail(e, "CU count");
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, c->device);
    if (e != hipSuccess) return bail(e, "LDS size");
    c->dev = kk::Device{ncu, lds};
    int wall = 0;
    if (hipDeviceGetAttribute(&wall, hipDeviceAttributeWallClockRate, c->device) == hipSuccess)
      c->wall_khz = wall;
    e = hipStreamCreateWithFlags(&c->aux, hipStreamNonBlocking);
    if (e != hipSuccess) return bail(e, "aux stream");
    e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming);
    if (e != hipSuccess) return bail(e, "fork event");
    e = hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming);
    if (e != hipSuccess) return bail(e, "join event");
    // the router-o-proj product for the fused o-proj + router launch of a layer without a norm
    // (the router reads h itself): E x Ko per plane, 0.69 MB for a 448-wide o-proj slice (used
    // by both paths), 11 MB for a full-width input (GEMV path, two tokens)
    if (kk::router_fused_applies(c->shape) && !c->norm.gamma) {
      e = hipMalloc(&c->mr, kk::router_oproj_product_bytes(c->shape));
      if (e != hipSuccess) return bail(e, "router-o-proj product allocation");
      e = kk::launch_router_oproj_product(c->shape, c->w.w_r, c->w.w_o, c->mr, nullptr);
      if (e != hipSuccess) return bail(e, "router-o-proj product launch");
    }
    // the static scratch of kk_layer_decode_static: its address on this device, looked up once
    // per device (a failure only disables that entry point)
    c->scratch_err = kk::scratch_init(c->device);
    if (c->scratch_err == hipSuccess) c->scratch = kk::scratch_ptr(c->device);
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return bail(e, "create sync");
    *out = c;
    return KK_OK;
  } catch (...) {
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_create");
  }
}

kk_status kk_destroy(kk_ctx* c) {
  if (!c) return KK_OK;
  if (c->aux) (void)hipStreamSynchronize(c->aux);
  destroy_graphs(c);
  if (c->mr) (void)hipFree(c->mr);
  for (auto& r : c->trecs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto ev : c->tpool) (void)hipEventDestroy(ev);
  if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
  if (c->ev_join) (void)hipEventDestroy(c->ev_join);
  if (c->aux) (void)hipStreamDestroy(c->aux);
  delete c;
  return KK_OK;
}

kk_status kk_query_plan(const kk_ctx* c, int32_t B, kk_plan* out) {
  if (!c || !out) return fail(KK_ERR_INVALID_ARG, "NULL argument");
  if (B < 1 || B > c->max_batch) return fail(KK_ERR_INVALID_ARG, "batch %d outside 1..%d", B, c->max_batch);
  return plan_for(c, B, out);
}

kk_status kk_oproj_residual(kk_ctx* c, int32_t B, const void* x, const void* resid, float* h32,
                            void* h_out, void* ws, kk_stream stream) {
  try {
    kk_status st = check_common(c, B, ws);
    if (st != KK_OK) return st;
    KK_PTR(x, "x");
    KK_PTR(resid, "resid");
    KK_PTR(h32, "h32");
    if (h_out && misaligned(h_out)) return fail(KK_ERR_INVALID_ARG, "h_out is not 16-byte aligned");
    kk_plan plan;
    if ((st = plan_for(c, B, &plan)) != KK_OK) return st;
    WsPtrs p = carve(c->L, ws);
    return enqueue_oproj(c, B, x, resid, h32, h_out, p.oproj_part, nullptr, plan.path,
                         (hipStream_t)stream);
  } catch (...) {
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_oproj_residual");
  }
}

kk_status kk_router_topk(kk_ctx* c, int32_t B, const float* h32, int32_t* topk_idx,
                         float* topk_gate, int32_t* expert_offsets, int32_t* perm, void* ws,
                         kk_stream stream) {
  try {
    kk_status st = check_common(c, B, ws);
    if (st != KK_OK) return st;
    KK_PTR(h32, "h32");
    KK_PTR(topk_idx, "topk_idx");
    KK_PTR(topk_gate, "topk_gate");
    KK_PTR(expert_offsets, "expert_offsets");
    KK_PTR(perm, "perm");
    kk_plan plan;
    if ((st = plan_for(c, B, &plan)) != KK_OK) return st;
    WsPtrs p = carve(c->L, ws);
    kk::Routing rt{topk_idx, topk_gate, expert_offsets, perm, p.inv_perm, p.act, p.n_act, p.vg,
                   p.n_vg};
    if (plan.path == KK_PATH_SPLITK_MFMA) {
      const float* u = enqueue_norm_from_h32(c, B, h32, p.u32, (hipStream_t)stream, &st);
      if (st != KK_OK) return st;
      return enqueue_router_mfma(c, B, u, rt, p.logit_part, (hipStream_t)stream);
    }
    // GEMV path on its own: logits, then the top-k rows and the tables
    hipStream_t s = (hipStream_t)stream;
    st = enqueue_logits(c, B, h32, rt, p.logit_part, nullptr, nullptr, s);
    if (st != KK_OK) return st;
    return enqueue_topk(c, B, p.logit_part, kk::router_gemv_splits(c->shape), rt, s);
  } catch (...) {
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_router_topk");
  }
}

kk_status kk_moe_decode(kk_ctx* c, int32_t B, const float* h32, const int32_t* topk_idx,
                        const float* topk_gate, const int32_t* expert_offsets, const int32_t* perm,
                        void* out, void* ws, kk_stream stream) {
  try {
    kk_status st = check_common(c, B, ws);
    if (st != KK_OK) return st;
    KK_PTR(h32, "h32");
    KK_PTR(topk_idx, "topk_idx");
    KK_PTR(topk_gate, "topk_gate");
    KK_PTR(expert_offsets, "expert_offsets");
    KK_PTR(perm, "perm");
    KK_PTR(out, "out");
    kk_plan plan;
    if ((st = plan_for(c, B, &plan)) != KK_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    WsPtrs p = carve(c->L, ws);
    kk::Routing rt{(int32_t*)topk_idx, (float*)topk_gate, (int32_t*)expert_offsets,
                   (int32_t*)perm, p.inv_perm, p.act, p.n_act, p.vg, p.n_vg, p.status};
    KK_HIP(timed(c, K_PREP, s, [&] { return kk::launch_moe_prep(c->shape, B, rt, s); }),
           "moe prep launch");
    if (plan.path == KK_PATH_SPLITK_MFMA) {
      const float* u = enqueue_norm_from_h32(c, B, h32, p.u32, s, &st);
      if (st != KK_OK) return st;
      return enqueue_experts_mfma(c, B, u, h32, rt, p, out, s);
    }
    st = enqueue_shared_gateup(c, B, h32, rt, p.As, s);
    if (st != KK_OK) return st;
    return enqueue_routed_and_combine(c, B, h32, rt, p, nullptr, out, s);
  } catch (...) {
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_moe_decode");
  }
}

kk_status kk_routing_status(kk_ctx* c, const void* ws, kk_stream stream) {
  try {
    if (!c) return fail(KK_ERR_INVALID_ARG, "context is NULL");
    if (!ws) return fail(KK_ERR_WORKSPACE, "workspace is NULL");
    if (misaligned(ws, 256)) return fail(KK_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != c->device)
      return fail(KK_ERR_INVALID_ARG, "current device %d is not the context's device %d", dev,
                  c->device);
    hipStream_t s = (hipStream_t)stream;
    int32_t bits = 0;
    KK_HIP(hipMemcpyAsync(&bits, (const char*)ws + c->L.status, sizeof bits, hipMemcpyDeviceToHost,
                          s),
           "status read");
    KK_HIP(hipStreamSynchronize(s), "status sync");
    if (bits == 0) return KK_OK;
    std::string why;
    const struct {
      int bit;
      const char* text;
    } reasons[] = {
        {kk::kRoutingOffsets, "expert_offsets not non-decreasing from 0 to B*k, or an expert with "
                              "more than B slots"},
        {kk::kRoutingPermRange, "a perm entry outside 0..B*k-1"},
        {kk::kRoutingPermDup, "perm lists a slot twice (not a permutation)"},
        {kk::kRoutingOrder, "an expert's slots are not in ascending token order"},
        {kk::kRoutingIdx, "topk_idx of a slot names another expert than the perm range it is in"}};
    for (const auto& r : reasons)
      if (bits & r.bit) why += std::string(why.empty() ? "" : "; ") + r.text;
    return fail(KK_ERR_INVALID_ARG,
                "kk_moe_decode was given invalid routing tables (%s); its routed part was left out",
                why.c_str());
  } catch (...) {
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_routing_status");
  }
}

kk_status kk_layer_decode(kk_ctx* c, int32_t B, const void* x, const void* resid, void* out,
                          int32_t* topk_idx, float* topk_gate, void* ws, kk_stream stream,
                          uint32_t flags) {
  try {
    kk_status st = check_common(c, B, ws);
    if (st != KK_OK) return st;
    KK_PTR(x, "x");
    KK_PTR(resid, "resid");
    KK_PTR(out, "out");
    if (topk_idx && misaligned(topk_idx)) return fail(KK_ERR_INVALID_ARG, "topk_idx misaligned");
    if (topk_gate && misaligned(topk_gate)) return fail(KK_ERR_INVALID_ARG, "topk_gate misaligned");
    if (flags & ~(KK_GRAPH | KK_TWO_STREAM))
      return fail(KK_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
    const bool two = (flags & KK_TWO_STREAM) != 0;
    kk_plan plan0;
    if ((st = plan_for(c, B, &plan0)) != KK_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    if (!(flags & KK_GRAPH))
      return enqueue_layer(c, B, x, resid, out, topk_idx, topk_gate, ws, s, two, plan0.path);
    if (!s) return fail(KK_ERR_INVALID_ARG, "KK_GRAPH needs a non-null stream");
    ++c->clock;
    for (auto& g : c->graphs) {
      if (g.B == B && g.flags == flags && g.path == plan0.path && g.x == x && g.r == resid &&
          g.out == out && g.idx == topk_idx && g.gate == topk_gate && g.ws == ws && g.stream == s) {
        g.uses = c->clock;
        KK_HIP(hipGraphLaunch(g.exec, s), "graph launch");
        return KK_OK;
      }
    }
    if (c->graphs.size() >= 16) {  // evict the least recently used graph
      size_t lru = 0;
      for (size_t i = 1; i < c->graphs.size(); ++i)
        if (c->graphs[i].uses < c->graphs[lru].uses) lru = i;
      (void)hipGraphExecDestroy(c->graphs[lru].exec);
      c->graphs.erase(c->graphs.begin() + lru);
    }
    KK_HIP(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "begin capture");
    st = enqueue_layer(c, B, x, resid, out, topk_idx, topk_gate, ws, s, two, plan0.path);
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(s, &graph);
    if (st != KK_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return st;
    }
    if (e != hipSuccess) return hip_fail(e, "end capture");
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(e, "graph instantiate");
    c->graphs.push_back(
        GraphEntry{B, flags, plan0.path, x, resid, out, topk_idx, topk_gate, ws, s, exec, c->clock});
    KK_HIP(hipGraphLaunch(exec, s), "graph launch");
    return KK_OK;
  } catch (...) {
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_layer_decode");
  }
}

kk_status kk_layer_decode_static(kk_ctx* c, int32_t B, const void* x, const void* resid, void* out,
                                 int32_t* topk_idx, float* topk_gate, kk_stream stream,
                                 uint32_t flags) {
  try {
    if (!c) return fail(KK_ERR_INVALID_ARG, "context is NULL");
    if (flags & ~KK_TWO_STREAM)
      return fail(KK_ERR_INVALID_ARG, "kk_layer_decode_static takes only KK_TWO_STREAM (flags 0x%x)",
                  flags);
    if (B < 1 || B > c->max_batch)
      return fail(KK_ERR_INVALID_ARG, "batch %d outside 1..%d (max_batch of this context)", B,
                  c->max_batch);
    if (!c->scratch)
      return hip_fail(c->scratch_err != hipSuccess ? c->scratch_err : hipErrorInvalidValue,
                      "static scratch unavailable on this device");
    // the regions this batch needs, in the same order as a workspace of max_batch B
    const Layout Ls = make_layout(c->cfg, B);
    if (Ls.total > kk::kScratchBytes)
      return fail(KK_ERR_WORKSPACE, "batch %d of this shape needs %zu bytes of scratch; the static "
                  "scratch holds %zu", B, Ls.total, kk::kScratchBytes);
    kk_status st = check_common(c, B, c->scratch);
    if (st != KK_OK) return st;
    KK_PTR(x, "x");
    KK_PTR(resid, "resid");
    KK_PTR(out, "out");
    if (topk_idx && misaligned(topk_idx)) return fail(KK_ERR_INVALID_ARG, "topk_idx misaligned");
    if (topk_gate && misaligned(topk_gate)) return fail(KK_ERR_INVALID_ARG, "topk_gate misaligned");
    const bool two = (flags & KK_TWO_STREAM) != 0;
    kk_plan plan;
    if ((st = plan_for(c, B, &plan)) != KK_OK) return st;
    c->no_alloc = true;
    st = enqueue_layer(c, B, x, resid, out, topk_idx, topk_gate, c->scratch, (hipStream_t)stream,
                       two, plan.path, nullptr, &Ls);
    c->no_alloc = false;
    return st;
  } catch (...) {
    c->no_alloc = false;
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_layer_decode_static");
  }
}

kk_status kk_chain_decode(kk_ctx* const* ctx, int32_t L, int32_t B, const void* const* x,
                          const void* resid, void* const* out, void* ws, kk_stream stream,
                          uint32_t flags) {
  try {
    if (!ctx || !x || !out) return fail(KK_ERR_INVALID_ARG, "ctx, x and out arrays must be non-NULL");
    if (L < 1 || L > 1024) return fail(KK_ERR_INVALID_ARG, "layer count %d outside 1..1024", L);
    if (flags & ~(KK_GRAPH | KK_PREFETCH))
      return fail(KK_ERR_INVALID_ARG, "unknown flags 0x%x for a chain", flags);
    KK_PTR(resid, "resid");
    for (int l = 0; l < L; ++l) {
      kk_status st = check_common(ctx[l], B, ws);
      if (st != KK_OK) return st;
      if (std::memcmp(&ctx[l]->cfg, &ctx[0]->cfg, sizeof(kk_config)) != 0)
        return fail(KK_ERR_INVALID_ARG, "context %d has another kk_config than context 0", l);
      for (int j = 0; j < l; ++j)
        if (ctx[j] == ctx[l]) return fail(KK_ERR_INVALID_ARG, "context %d repeats context %d", l, j);
      KK_PTR(x[l], "x[l]");
      KK_PTR(out[l], "out[l]");
    }
    hipStream_t s = (hipStream_t)stream;
    const bool prefetch = (flags & KK_PREFETCH) != 0;
    if (!(flags & KK_GRAPH)) return enqueue_chain(ctx, L, B, x, resid, out, ws, s, prefetch);
    if (!s) return fail(KK_ERR_INVALID_ARG, "KK_GRAPH needs a non-null stream");
    kk_ctx* c0 = ctx[0];
    std::vector<uintptr_t> key;
    key.reserve(4 * L + 3);
    for (int l = 0; l < L; ++l) key.push_back((uintptr_t)ctx[l]->serial);
    for (int l = 0; l < L; ++l) key.push_back((uintptr_t)x[l]);
    for (int l = 0; l < L; ++l) key.push_back((uintptr_t)out[l]);
    for (int l = 0; l < L; ++l) {  // the plans the chain is captured with
      kk_plan plan;
      kk_status st = plan_for(ctx[l], B, &plan);
      if (st != KK_OK) return st;
      key.push_back((uintptr_t)plan.path);
    }
    key.push_back((uintptr_t)resid);
    key.push_back((uintptr_t)ws);
    key.push_back((uintptr_t)s);
    ++c0->clock;
    for (auto& g : c0->chains) {
      if (g.B == B && g.flags == flags && g.key == key) {
        g.uses = c0->clock;
        KK_HIP(hipGraphLaunch(g.exec, s), "chain graph launch");
        return KK_OK;
      }
    }
    if (c0->chains.size() >= 8) {  // evict the least recently used chain graph
      size_t lru = 0;
      for (size_t i = 1; i < c0->chains.size(); ++i)
        if (c0->chains[i].uses < c0->chains[lru].uses) lru = i;
      (void)hipGraphExecDestroy(c0->chains[lru].exec);
      c0->chains.erase(c0->chains.begin() + lru);
    }
    KK_HIP(hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal), "begin capture");
    kk_status st = enqueue_chain(ctx, L, B, x, resid, out, ws, s, prefetch);
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamEndCapture(s, &graph);
    if (st != KK_OK) {
      if (graph) (void)hipGraphDestroy(graph);
      return st;
    }
    if (e != hipSuccess) return hip_fail(e, "end capture");
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(e, "graph instantiate");
    c0->chains.push_back(ChainGraph{std::move(key), B, flags, exec, c0->clock});
    KK_HIP(hipGraphLaunch(exec, s), "chain graph launch");
    return KK_OK;
  } catch (...) {
    return fail(KK_ERR_INVALID_ARG, "internal error in kk_chain_decode");
  }
}

kk_status kk_set_stream_delay(kk_ctx* c, int32_t which, float microseconds) {
  if (!c) return fail(KK_ERR_INVALID_ARG, "context is NULL");
  if (which != 0 && which != 1) return fail(KK_ERR_INVALID_ARG, "which must be 0 (main) or 1 (auxiliary)");
  if (!(microseconds >= 0.f && microseconds <= 10000.f))
    return fail(KK_ERR_INVALID_ARG, "delay must be 0..10000 microseconds");
  if (microseconds > 0.f && c->wall_khz <= 0)
    return fail(KK_ERR_UNSUPPORTED, "the device reports no constant-rate clock");
  c->delay_ticks[which] = (long long)((double)microseconds * (double)c->wall_khz / 1000.0);
  return KK_OK;
}

kk_status kk_set_kernel_timing(kk_ctx* c, int32_t enable) {
  if (!c) return fail(KK_ERR_INVALID_ARG, "context is NULL");
  c->timing = enable != 0;
  return KK_OK;
}

kk_status kk_read_kernel_timing(kk_ctx* c, const char** names, float* ms, int32_t cap,
                                int32_t* count) {
  if (!c || !count) return fail(KK_ERR_INVALID_ARG, "NULL argument");
  int n = 0;
  for (auto& r : c->trecs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(KK_ERR_HIP, "timing event sync");
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) t = -1.f;
    if (n < cap) {
      if (names) names[n] = kernel_names[r.name];
      if (ms) ms[n] = t;
    }
    ++n;
    c->tpool.push_back(r.a);
    c->tpool.push_back(r.b);
  }
  c->trecs.clear();
  *count = n;
  return KK_OK;
}

}  // extern "C"

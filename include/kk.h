/*
 * kk.h -- C ABI of the MI355X (gfx950) MoE decode-layer step.
 *
 * One small-batch (1..64 token) decode step of the weight-bandwidth-bound part of a
 * Kimi-K3-style layer:
 *   h   = r + x W_o^T                       attention output projection + residual
 *   u   = h, or with a norm weight w:        u = w * h / sqrt(mean(h^2) + norm_eps)
 *   l   = u W_r^T, s = sigmoid(l)            router scores
 *   S_t = top-k of (s + b)                   selection (bias steers selection only)
 *   g   = s[S_t] / sum s[S_t] * routed_scale renormalised gates
 *   out = h + sum_j g_j SwiGLU_{S_t,j}(u) + SwiGLU_shared(u)
 * Sources: "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly", section
 * "Recovering time between operators" (o-proj fused with residual processing; router
 * scores; selected experts; the shared expert on another stream; small-matrix kernels at
 * batch 1-2 and split-K at larger batch); "vLLM Hyper-Optimizes Kimi K3 on NVIDIA GB300 for
 * Blazing-FAST Inference", section "What's Optimized" (per-batch kernel choice, shared
 * expert in parallel on a separate stream).  The pages print no formula; the math above
 * is the plain reading of the operations they name (sigmoid + bias router, renormalised
 * gates, gated SwiGLU with gate rows before up rows).  The "residual processing" fused with
 * the o-proj is read as the residual add, optionally followed by an RMSNorm whose output
 * feeds the router and the experts while h stays the residual stream.
 *
 * Layouts (all row-major, "out-major": each output row contiguous along its reduction dim)
 *   w_o  [H][Ko]     w_r [E][H]     router_bias [E] (fp32)
 *   w13  [E][2I][H]  rows 0..I-1 gate (W1), rows I..2I-1 up (W3)
 *   w2   [E][H][I]   ws13 [2Is][H]  ws2 [H][Is]  norm_weight [H] (optional)
 *   x [B][Ko], resid [B][H], out [B][H]  in the config dtype; h32 [B][H] fp32.
 *   topk_idx [B][k] int32, ascending expert index within each token; topk_gate [B][k] fp32
 *   in the same order.  Slot of (token t, position j) = t*k + j.
 *   expert_offsets [E+1] int32: exclusive prefix sum of per-expert slot counts.
 *   perm [B*k] int32: slots ordered by (expert, token).
 *
 * Ownership: the caller owns every buffer (weights, activations, outputs, workspace).
 * Weights passed to kk_create must stay alive and unchanged until kk_destroy.  The
 * context owns an auxiliary HIP stream, events, cached HIP graphs and, for a bf16 layer without
 * a norm, one device buffer: the router-o-proj product W_r W_o (two bf16 planes [2][E][Ko]; at
 * E = 384 0.69 MB for a 448-wide o-proj input slice, 11 MB for a 7168-wide input), computed by
 * kk_create from the weights and freed by kk_destroy.  Every device pointer must be 16-byte aligned; ws must be
 * 256-byte aligned.
 *
 * Concurrency: every op is asynchronous on the caller's stream; no host synchronisation.
 * One host thread and one stream at a time per context (the ops share the context's
 * auxiliary stream and events).
 *
 * Errors: arguments are validated on the host before anything is enqueued; a failure
 * returns a status and sets kk_last_error() (thread-local text).  A shape outside the
 * supported set returns KK_ERR_UNSUPPORTED -- there is no slower fallback.  A failed HIP
 * launch returns KK_ERR_HIP; device faults surface at the caller's next synchronisation.
 * No op writes the weights.
 */
#ifndef KK_H_
#define KK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KK_OK = 0,
  KK_ERR_INVALID_ARG = 1,
  KK_ERR_UNSUPPORTED = 2,
  KK_ERR_WORKSPACE = 3,
  KK_ERR_HIP = 4
} kk_status;

typedef enum { KK_F32 = 0, KK_BF16 = 1 } kk_dtype;

typedef enum {
  KK_PATH_GEMV = 0,       /* batch 1-2: bf16/fp32 weight rows streamed with 128-bit loads */
  KK_PATH_SPLITK_MFMA = 1 /* batch 3-64: MFMA tiles, split-K with an fp32 second stage */
} kk_path;

/* kk_layer_decode flags */
#define KK_GRAPH 1u      /* capture the step once per (B, buffers, stream, flags), replay it */
#define KK_TWO_STREAM 2u /* the shared expert on the context's auxiliary stream (kept for
                            comparison; same output bits): batch 1-2 its gate/up instead of
                            inside the top-k launch, batch 3-64 its gate/up and down-projection
                            (forked after the o-proj, joined before the combine) instead of as
                            the last group of the grouped launches */
#define KK_PREFETCH 4u   /* kk_chain_decode: after layer l's o-proj, the first context's
                            auxiliary stream reads layer l+1's o-proj, router and shared gate/up
                            weights once, so that layer finds them in the memory-side cache */

typedef struct {
  int32_t hidden;       /* H  */
  int32_t oproj_in;     /* Ko */
  int32_t n_experts;    /* E  */
  int32_t top_k;        /* k  */
  int32_t inter;        /* I  (routed SwiGLU intermediate) */
  int32_t shared_inter; /* Is (shared SwiGLU intermediate) */
  int32_t dtype;        /* kk_dtype of weights, x, resid and out */
  float routed_scale;   /* multiplies the renormalised gates; 1.0 */
  float norm_eps;       /* RMSNorm epsilon (>= 0; used only with kk_weights.norm_weight) */
} kk_config;

typedef struct {
  const void* w_o;
  const void* w_r;
  const float* router_bias;
  const void* w13;
  const void* w2;
  const void* ws13;
  const void* ws2;
  const void* norm_weight; /* [H] in the config dtype, or NULL: no norm (u = h) */
} kk_weights;

typedef struct {
  int32_t path;             /* kk_path chosen for this batch */
  int32_t forced;           /* 1 if the KK_FORCE_PLAN environment variable chose it */
  int32_t oproj_splitk;     /* K splits of the o-proj (1 on the GEMV path) */
  int32_t router_splitk;    /* K splits of the router logits */
  int32_t kernels_per_step; /* kernel launches of one default kk_layer_decode step */
  int32_t streams;          /* streams the default step uses (1; 2 with KK_TWO_STREAM) */
} kk_plan;

typedef struct kk_ctx kk_ctx;
typedef void* kk_stream; /* a hipStream_t; NULL = the null stream */

/* Supported set today: max_batch 1..64; E <= 512 with k <= min(E, 16); bf16: H = 7168,
 * Ko in {448, 7168}, I and Is in {128, 2048}; fp32: H = Ko = 256, I = Is = 128 and
 * batch <= 2.  Host-only: enqueues nothing and touches no device. */
kk_status kk_validate(const kk_config* cfg, int32_t max_batch);

/* Bytes of workspace every op needs for any B <= max_batch (0 if cfg is invalid). */
size_t kk_workspace_bytes(const kk_config* cfg, int32_t max_batch);

/* Creates a context on the current HIP device; weights are referenced, not copied.  For a bf16
 * layer without a norm it also allocates the router-o-proj product (0.69 MB for a 448-wide
 * o-proj slice, 11 MB for a 7168-wide input) and computes it with one kernel on the null
 * stream, synchronised before returning;
 * an allocation or launch failure returns KK_ERR_HIP and no context. */
kk_status kk_create(const kk_config* cfg, const kk_weights* w, int32_t max_batch, kk_ctx** out);
kk_status kk_destroy(kk_ctx* ctx);

/* Which path and how many launches a step of batch B uses (no device work). */
kk_status kk_query_plan(const kk_ctx* ctx, int32_t B, kk_plan* out);

/* h32 = resid + x W_o^T (fp32); h_out (nullable) = the same rounded RNE to the config
 * dtype. "Recovering time between operators": o-proj fused with residual processing. */
kk_status kk_oproj_residual(kk_ctx* ctx, int32_t B, const void* x, const void* resid, float* h32,
                            void* h_out, void* ws, kk_stream stream);

/* Router: logits from fp32 h32 (normalised first when the context has a norm weight), sigmoid scores, selection keys (s + b, fp64), top-k,
 * renormalised gates, and the token->expert permutation with expert offsets (prefix sum).
 * "Recovering time between operators": router scores in MoE preparation. */
kk_status kk_router_topk(kk_ctx* ctx, int32_t B, const float* h32, int32_t* topk_idx,
                         float* topk_gate, int32_t* expert_offsets, int32_t* perm, void* ws,
                         kk_stream stream);

/* Routed experts (each selected expert's weights read once), the shared expert, and the
 * combine out = h32 + sum g y + y_shared (RNE to the config dtype), all on `stream`; the
 * experts read u = h32, or h32 normalised when the context has a norm weight.
 * Routing tables as written by kk_router_topk for the same B.  A device-side check runs before
 * any weight is read: expert_offsets non-decreasing from 0 to B*k with at most B slots per
 * expert, perm a permutation of the B*k slots, each expert's slots in ascending token order,
 * and topk_idx of every slot naming the expert whose perm range holds it.  Tables that fail
 * leave the routed part out (out = h32 + y_shared, no out-of-bounds access) and record why in
 * ws: kk_routing_status reports it.  (The call itself returns as soon as the work is enqueued.)
 * "Recovering time between operators": selected experts; shared expert on another stream.
 * "Faster code needs targeted validation": a path that silently falls back gives no evidence,
 * so the caller can always tell a dropped MoE part from a computed one. */
kk_status kk_moe_decode(kk_ctx* ctx, int32_t B, const float* h32, const int32_t* topk_idx,
                        const float* topk_gate, const int32_t* expert_offsets, const int32_t* perm,
                        void* out, void* ws, kk_stream stream);

/* Result of the table check of the last kk_moe_decode that used workspace ws: waits for
 * `stream` (a host synchronisation; enqueue nothing that changes ws in between), then returns
 * KK_OK when the tables were a valid routing, else KK_ERR_INVALID_ARG with kk_last_error()
 * naming each rule they broke (that call's routed part was left out of its output).  Other ops
 * do not update the record.  "Faster code needs targeted validation": no silent fallback. */
kk_status kk_routing_status(kk_ctx* ctx, const void* ws, kk_stream stream);

/* The whole step: o-proj + residual (+ norm), router logits, top-k || shared expert gate/up,
 * routed gate/up, down-projection with the combine (batch 1-2: four launches on `stream`, the
 * norm recomputed inside the launches that read u; three with the router-o-proj product, for a
 * 448-wide o-proj slice and for a full-width input at batch 2; the split-K MFMA path for larger
 * batches, the norm fused into the o-proj's reduce: see
 * kk_query_plan for the launch count).  topk_idx / topk_gate are optional
 * copies of the routing (nullable).  With KK_GRAPH the step is captured into a HIP graph on
 * first use for these (B, pointers, stream, flags, planned path) and replayed afterwards.
 * "Recovering time between operators": the o-proj fused with the residual processing, router
 * scores in the MoE preparation, the selected experts and the shared expert, with the kernel
 * choice depending on the batch (small-matrix kernels at batch 1-2, split-K above). */
kk_status kk_layer_decode(kk_ctx* ctx, int32_t B, const void* x, const void* resid, void* out,
                          int32_t* topk_idx, float* topk_gate, void* ws, kk_stream stream,
                          uint32_t flags);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): kk_layer_decode without a workspace argument.  The
 * step's intermediates live in a static device array of the library (64 MiB per GPU, held from
 * the library's first use on that GPU until the process ends; its address is looked up once per
 * device by kk_create); the call itself allocates nothing.  A batch whose intermediates exceed
 * the array returns KK_ERR_WORKSPACE (every supported shape fits up to 64 tokens).  flags: 0 or
 * KK_TWO_STREAM (no KK_GRAPH).  Output bits equal kk_layer_decode's for the same inputs.  All
 * calls on one GPU share its array and keep no state in it between calls (every region a step
 * reads is written earlier in that step), so calls that overlap in time on one GPU, from any
 * context or stream, race and give undefined output: serialise them. */
kk_status kk_layer_decode_static(kk_ctx* ctx, int32_t B, const void* x, const void* resid,
                                 void* out, int32_t* topk_idx, float* topk_gate,
                                 kk_stream stream, uint32_t flags);

/* Consecutive layers, each with its own context and weights: layer l reads x[l] [B][Ko] and the
 * residual stream r_l (resid for l = 0, out[l-1] after it) and writes out[l] [B][H]; every
 * layer's output is kept.  All L contexts must have the same kk_config, max_batch >= B and
 * the current device; ws (kk_workspace_bytes of the largest max_batch among them) is used by
 * the layers in turn.  x, out: host arrays of L device pointers; no out[l] may overlap an
 * x[j], resid or another out.  Flags: KK_GRAPH (the whole chain is captured once per
 * (contexts, B, pointers, stream, flags) and replayed; the graphs are kept by ctx[0]) and
 * KK_PREFETCH.  "What's Optimized" (a side kernel preloads the next operation's weights into
 * cache) and "Recovering time between operators" (an auxiliary stream loads weights before
 * their consumer starts, in the idle intervals of the current work). */
kk_status kk_chain_decode(kk_ctx* const* ctx, int32_t L, int32_t B, const void* const* x,
                          const void* resid, void* const* out, void* ws, kk_stream stream,
                          uint32_t flags);
/* Test hook for stream hazards: a one-wave kernel that waits `microseconds` (0..10000; 0
 * removes it) of the device's constant-rate clock is enqueued before every later step's work on
 * the caller's stream (which = 0, ahead of the o-proj) or on the auxiliary stream right after it
 * waits for the fork (which = 1: the KK_TWO_STREAM shared expert, the KK_PREFETCH reads).  A
 * missing cross-stream wait then shows as changed output bits.  Every delay kernel ends after
 * its time (or after about a second of sleeps at most).  "Faster code needs targeted
 * validation": reads moved before a synchronisation wait escape ordinary functional tests. */
kk_status kk_set_stream_delay(kk_ctx* ctx, int32_t which, float microseconds);

/* Per-kernel timing of eager (non-graph) launches: when enabled, every kernel the context
 * launches is bracketed by HIP events on its own stream.  kk_read_kernel_timing waits for
 * the recorded events and returns up to `cap` (name, milliseconds) records of the launches
 * since the last read, clearing them.  Names stay valid until kk_destroy. */
kk_status kk_set_kernel_timing(kk_ctx* ctx, int32_t enable);
kk_status kk_read_kernel_timing(kk_ctx* ctx, const char** names, float* ms, int32_t cap,
                                int32_t* count);

const char* kk_status_string(kk_status s);
const char* kk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KK_H_ */

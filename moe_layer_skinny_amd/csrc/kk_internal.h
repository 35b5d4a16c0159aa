// Internal interface between the host API (kk_api.cpp) and the kernels (kk_gemv.hip,
// kk_mfma.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kk {

struct Shape {
  int H, Ko, E, k, I, Is;
  int dtype;  // 0 fp32, 1 bf16
  float routed_scale;
};

struct Weights {
  const void* w_o;
  const void* w_r;
  const float* bias;
  const void* w13;
  const void* w2;
  const void* ws13;
  const void* ws2;
};

// Routing tables on the device.  topk_* and offsets/perm may be caller buffers.
struct Routing {
  int32_t* topk_idx;   // [B][k]
  float* topk_gate;    // [B][k]
  int32_t* offsets;    // [E+1]
  int32_t* perm;       // [B*k]  position -> slot
  int32_t* inv_perm;   // [B*k]  slot -> position
  int32_t* act;        // [E]    active experts, ascending
  int32_t* n_act;      // [1]
  // optional: the active experts cut into pieces of at most 16 positions, in expert order;
  // entry = (index into act) << 2 | piece (positions offsets[e] + 16 piece ..)
  int32_t* vg = nullptr;    // [E + 64]
  int32_t* n_vg = nullptr;  // [1]
  // check of caller-supplied tables (kk_moe_decode): 0 valid, else kRouting* bits
  int32_t* status = nullptr;  // [1]
};

// Bits of Routing::status: what made caller-supplied tables invalid.
constexpr int kRoutingOffsets = 1;    // offsets not non-decreasing from 0 to B*k, or an
                                      // expert with more than B positions
constexpr int kRoutingPermRange = 2;  // a perm entry outside 0..B*k-1
constexpr int kRoutingPermDup = 4;    // a slot listed twice in perm (not a permutation)
constexpr int kRoutingOrder = 8;      // an expert's slots not in ascending token order
                                      // (or one token twice)
constexpr int kRoutingIdx = 16;       // topk_idx of a slot names another expert than the
                                      // range of perm it sits in

// RMSNorm between the residual add and the router / experts:
// u = h * gamma / sqrt(mean(h^2) + eps); gamma == nullptr: none, u = h.
struct Norm {
  const void* gamma = nullptr;  // [H] in the config dtype
  float eps = 0.f;
};

// Launch configuration facts gathered once per context.
struct Device {
  int num_cu;
  int max_lds;  // bytes of LDS one block may use
};

// ---- GEMV path (batch 1..2) ----------------------------------------------------------
// Each returns hipSuccess or the launch error.  `unsupported` is set when no kernel
// instance exists for the shape (checked by kk_validate before any launch).
bool gemv_supported(const Shape& s, int B);

hipError_t launch_oproj_gemv(const Shape& s, const Device& d, int B, const void* x, const void* r,
                             const void* w_o, float* h32, void* h_out, hipStream_t st);

// The router-o-proj product mr = W_r W_o of a layer ([planes][E][Ko] in the weight dtype:
// bf16 as hi + lo planes, fp32 as one), computed once (fp64 accumulation).
bool router_fused_applies(const Shape& s);  // bf16 GEMV shapes with H = 7168, Ko 448 or 7168
int router_oproj_planes(const Shape& s);
size_t router_oproj_product_bytes(const Shape& s);
hipError_t launch_router_oproj_product(const Shape& s, const void* w_r, const void* w_o, void* mr,
                                       hipStream_t st);
// o-proj + residual and the router logit partials in one launch, the router reading x and r
// (logit = W_r . r + mr . x): part[router_fused_splits(s)][B][E].
int router_fused_splits(const Shape& s);
hipError_t launch_oproj_router_gemv(const Shape& s, const Device& d, int B, const void* x,
                                    const void* r, const void* w_o, const void* w_r, const void* mr,
                                    float* h32, void* h_out, float* part, hipStream_t st);

// Router logit partials part[s][t][e] = h32[t][slice s] . W_r[e][slice s]; with ws13 !=
// nullptr the same launch computes the shared expert's gate/up,
// As[t][i] = silu(Ws1[i] . u_t) * (Ws3[i] . u_t).  The top-k runs in the routed gate/up
// launch (GateupExtras::part) or, on its own, in launch_topk_rows + launch_tables.
// With a norm every block stages u = norm(h32) in its LDS from h32.
hipError_t launch_router_logits(const Shape& s, const Device& d, int B, const float* h32,
                                const void* w_r, float* partials, const void* ws13,
                                const Routing& rt, float* As, const Norm& nm, hipStream_t st);
int router_gemv_splits(const Shape& s);

// Optional work of the routed gate/up launch.
struct GateupExtras {
  const float* part = nullptr;  // logit partials [splits][B][E]: run the top-k in the launch
  int splits = 0;               // and write the routing tables (rt) from its block 0
  const float* bias = nullptr;
  const void* ws2 = nullptr;    // shared expert's down-projection ys = Ws2 . As in the launch
  const float* As = nullptr;
  float* ys = nullptr;
  const void* ws13 = nullptr;   // or its gate/up As_out = SwiGLU(Ws13 . u) in the launch
  float* As_out = nullptr;
  Norm norm;                    // stage u = norm(u) (every block from the rows it reads)
};

// Routed gate/up over the active experts (act/n_act) or the shared expert (shared=true):
// A[position][i] = silu(W1[i] . u_t) * (W3[i] . u_t), t = token of the position.
hipError_t launch_gateup_gemv(const Shape& s, const Device& d, int B, const float* u,
                              const void* w13, bool shared, const Routing& rt, float* A,
                              const GateupExtras& extras, hipStream_t st);

// Down projection of the active experts fused with the weighted combine (GEMV path):
// out[t][n] = RNE(h32[t][n] + sum_j gate[t][j] Y[inv_perm[t*k+j]][n] + ys[t][n]) with
// Y[p][n] = W2_e[n] . A[p] kept on chip and ys the shared expert's output: with ws2 != nullptr
// computed in the same launch from As (ys unused), else read from ys.
size_t down_combine_gemv_lds(const Shape& s, const Device& d, int B, bool shared_down);
hipError_t launch_down_combine_gemv(const Shape& s, const Device& d, int B, const float* A,
                                    const float* ys, const void* w2, const float* h32,
                                    const Routing& rt, void* out, const void* ws2,
                                    const float* As, hipStream_t st);
// Weighted combine of Y / ys written by the grouped MFMA down-projection.
hipError_t launch_combine(const Shape& s, int B, const float* h32, const float* Y, const float* ys,
                          const Routing& rt, void* out, hipStream_t st);

// Large-batch router tail: one wave per token writes its top-k row, then one block builds
// the routing tables from all rows.
hipError_t launch_topk_rows(const Shape& s, int B, const float* part, int splits,
                            const float* bias, const Routing& rt, hipStream_t st);
hipError_t launch_tables(const Shape& s, int B, const Routing& rt, hipStream_t st);
// Both in one launch, for up to 16 tokens.
hipError_t launch_topk_tables(const Shape& s, int B, const float* part, int splits,
                              const float* bias, const Routing& rt, hipStream_t st);

// One wave that waits `ticks` of the constant-rate device clock (bounded; nothing if <= 0).
hipError_t launch_delay(long long ticks, hipStream_t st);

// Reads `bytes` (a multiple of 16) at p once with cache-allocating loads and discards them.
hipError_t launch_prefetch(const Device& d, const void* p, size_t bytes, hipStream_t st);

// act / n_act / inv_perm from caller-provided offsets + perm (standalone kk_moe_decode), after
// checking the tables; invalid tables give n_act = 0 (routed part left out) and the reason in
// rt.status.
hipError_t launch_moe_prep(const Shape& s, int B, const Routing& rt, hipStream_t st);

// ---- static scratch (kk_scratch.hip) ----------------------------------------------------
// Size of the per-device static scratch array of the entry point that allocates nothing.
constexpr size_t kScratchBytes = (size_t)64 << 20;
// Looks up the array's device address on `device` (which must be current) once, and keeps it.
hipError_t scratch_init(int device);
// The address scratch_init found for `device`, or nullptr.
void* scratch_ptr(int device);

// ---- split-K MFMA path (batch 3..64) ---------------------------------------------------
bool mfma_supported(const Shape& s, int B);
int mfma_oproj_splits(const Shape& s);
int mfma_router_splits(const Shape& s);
// o-proj partials part[sp][t][n] over the K slices, then h32 = r + sum (and h_out).
hipError_t launch_oproj_mfma(const Shape& s, const Device& d, int B, const void* x, float* part,
                             const void* w_o, hipStream_t st);
// Split-K path, layers with the router-o-proj product (bf16, Ko = 448): the o-proj
// (h32 = r + W_o x directly) and the router logit partials from r and x in one launch,
// part[mfma_fused_splits(s)][B][E].
int mfma_fused_splits(const Shape& s);
hipError_t launch_oproj_router_mfma(const Shape& s, const Device& d, int B, const void* x,
                                    const void* r, const void* w_o, const void* w_r,
                                    const void* mr, float* h32, float* oproj_part,
                                    float* logit_part, hipStream_t st);
hipError_t launch_oproj_reduce(const Shape& s, int B, const float* part, const void* r,
                               float* h32, void* h_out, hipStream_t st);
// One block per token: u32 = norm(h) with h = r + sum of the o-proj partials (also written to
// h32 / h_out) when part != nullptr, else h read from h32.
hipError_t launch_norm_rows(const Shape& s, int B, const float* part, const void* r, float* h32,
                            void* h_out, const Norm& nm, float* u32, hipStream_t st);
// Router logit partials from h32 (three bf16 terms per fp32 value).
hipError_t launch_router_mfma(const Shape& s, const Device& d, int B, const float* h32,
                              const void* w_r, float* part, hipStream_t st);
// Grouped gate/up (routed experts and the shared expert) -> A, As.  Over 32 tokens the
// shared expert's gate/up is split over K; its partials use `scratch`
// (mfma_scratch_floats floats).
size_t mfma_scratch_floats(const Shape& s, int B);
// Whether batch B's gate/up also splits every group over K chunks (small intermediates), with
// a SwiGLU launch of its own after it (or, with mfma_swiglu_in_down, inside the down-projection).
bool mfma_gateup_split(const Shape& s, int B);
// `sel` picks the groups (both launches): every group, the active experts only, or the shared
// expert only (which reads no routing table), so that the shared expert can run on a stream of
// its own with the same kernels and the same bits.
constexpr int kGroupsEvery = 0, kGroupsRoutedOnly = 1, kGroupsSharedOnly = 2;
hipError_t launch_gateup_mfma(const Shape& s, const Device& d, int B, const float* h32,
                              const void* w13, const void* ws13, const Routing& rt, float* A,
                              float* As, float* scratch, hipStream_t st, int sel = 0);
// Whether the down-projection forms its activations itself, as the SwiGLU of the gate/up K-chunk
// partials (small intermediate up to 16 tokens): the gate/up launch then leaves A / As unwritten.
bool mfma_swiglu_in_down(const Shape& s, int B);
// Whether the grouped down-projection writes the rows of Y by slot t*k + j (up to 16 tokens;
// the combine then reads them without the inverse permutation) rather than by position.
bool mfma_y_by_slot(int B);
// Grouped down-projection -> Y (rows by slot or by position), ys (shared); its activations are A / As, or
// with mfma_swiglu_in_down the SwiGLU of the gate/up partials in gu_part (the gate/up's scratch).
hipError_t launch_down_mfma(const Shape& s, const Device& d, int B, const float* A,
                            const float* As, const void* w2, const void* ws2, const Routing& rt,
                            float* Y, float* ys, const float* gu_part, hipStream_t st,
                            int sel = 0);

}  // namespace kk

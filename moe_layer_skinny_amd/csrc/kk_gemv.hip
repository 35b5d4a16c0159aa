// GEMV path of the decode-layer step (batch 1-2): every weight row is streamed from HBM
// once with 128-bit non-temporal loads, each row's dot product finished with a wavefront
// shuffle reduction.  One stream, six launches per step:
//   1. o-proj + residual                     (activations held in registers)
//   2. router logits (split-K partials)         ||  shared expert gate/up, first half
//   3. top-k / gates / routing tables (block 0)  ||  shared expert gate/up, second half
//   4. routed gate/up over the active experts
//   5. routed + shared down-projection, one contiguous run of one expert's rows per unit
//   6. weighted combine into the residual
//
// "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly", section "Recovering
// time between operators": small-matrix projection kernels at batch 1-2; o-proj fused with
// the residual; the shared expert overlapping routing; fewer launches.  On this GPU a
// cross-stream fork/join and replayed graph nodes each cost more than a kernel boundary on
// one stream, and a device-scope fence per wave for an in-kernel cross-block handoff costs
// more still, so the shared expert overlaps the serial top-k inside launch 3 with no
// communication between its blocks.
#include "kk_common.cuh"
#include "kk_internal.h"
#include "kk_topk.cuh"

namespace kk {
namespace {

constexpr int kGemvThreads = 512;  // up to 8 waves; persistent blocks

// ------------------------------------------------------------------------------ o-proj
// h32[t][n] = r[t][n] + sum_k W_o[n][k] x[t][k]; optional h_out = RNE(h32).
// When they fit (NT * CPL <= 14 chunks) each lane keeps its own chunks of x in registers --
// the same chunk positions for every row, no LDS and no barrier before the first weight
// loads; otherwise x is staged in LDS as fp32 while the first rows are in flight.
template <typename T, int CPR, int NT, int R>
__global__ __launch_bounds__(kGemvThreads) void oproj_gemv_kernel(
    const T* __restrict__ x, const T* __restrict__ r, const T* __restrict__ w_o,
    float* __restrict__ h32, T* __restrict__ h_out, int H) {
  using G = Geo<T, CPR>;
  constexpr bool kRegs = NT * G::CPL <= 14;
  extern __shared__ float lds[];  // x as fp32 [NT][Ko] when not in registers
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wpb = blockDim.x >> 6;
  const int sub = lane % G::SEG, seg = lane / G::SEG;
  const int rows_per_unit = G::RPW * R;
  const int units = (H + rows_per_unit - 1) / rows_per_unit;
  const int stride = gridDim.x * wpb;
  int unit = blockIdx.x * wpb + wave;

  u32x4 w[R][G::CPL];
  auto issue = [&](int u) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int n = u * rows_per_unit + seg + G::RPW * q;
      if (n < H)
        load_row<T, CPR>(w_o + (size_t)n * G::K, sub, w[q]);
      else
#pragma unroll
        for (int i = 0; i < G::CPL; ++i) w[q][i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 xa[kRegs ? NT : 1][G::CPL];
  if constexpr (kRegs) {
    if (unit >= units) return;
    issue(unit);
#pragma unroll
    for (int t = 0; t < NT; ++t) load_act_chunks<T, CPR>(x + (size_t)t * G::K, sub, xa[t]);
  } else {
    if (unit < units) issue(unit);
    for (int i = threadIdx.x; i < NT * G::K; i += blockDim.x) lds[i] = Elem<T>::load(x, i);
    __syncthreads();
    if (unit >= units) return;
  }

  while (true) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int n = unit * rows_per_unit + seg + G::RPW * q;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float part;
        if constexpr (kRegs)
          part = dot_rr<T, CPR>(w[q], xa[t], sub);
        else
          part = dot_lane<T, CPR>(w[q], lds + t * G::K, sub);
        const float acc = seg_sum<G::SEG>(part);
        if (sub == 0 && n < H) {
          const size_t o = (size_t)t * H + n;
          const float hv = Elem<T>::load(r, o) + acc;
          h32[o] = hv;
          if (h_out) Elem<T>::store(h_out, o, hv);
        }
      }
    }
    unit += stride;
    if (unit >= units) break;
    __builtin_amdgcn_sched_barrier(0);
    issue(unit);
  }
}

// ------------------------------------------------------------------------------ gate / up
// One gate/up row pair of one expert for the positions [p0, p1) of that expert:
// A[p][i] = silu(W1[i] . u_t) * (W3[i] . u_t), u_t an fp32 row in LDS.
template <typename T, int CPR, int NT>
__device__ __forceinline__ void gateup_unit(const u32x4 (&wg)[Geo<T, CPR>::CPL],
                                            const u32x4 (&wu)[Geo<T, CPR>::CPL],
                                            const float* lds_u, int p0, int p1, int i, int I,
                                            int k, bool identity_tokens, const Routing& rt,
                                            float* __restrict__ A, int lane) {
  using G = Geo<T, CPR>;
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const int p = p0 + q;
    if (p < p1) {
      const int t = identity_tokens ? p : rt.perm[p] / k;
      float z1, z3;
      dot2_lane<T, CPR>(wg, wu, lds_u + t * G::K, lane, z1, z3);
      z1 = seg_sum<64>(z1);
      z3 = seg_sum<64>(z3);
      if (lane == 0) A[(size_t)p * I + i] = silu_f32(z1) * z3;
    }
  }
}

template <typename T, int CPR>
__device__ __forceinline__ void load_pair(const T* __restrict__ w13, int e, int i, int I,
                                          u32x4 (&wg)[Geo<T, CPR>::CPL],
                                          u32x4 (&wu)[Geo<T, CPR>::CPL], int lane) {
  using G = Geo<T, CPR>;
  const T* g_row = w13 + ((size_t)e * 2 * I + i) * G::K;
  load_row<T, CPR>(g_row, lane, wg);
  load_row<T, CPR>(g_row + (size_t)I * G::K, lane, wu);
}

__device__ __forceinline__ void stage_rows_f32(float* dst, const float* __restrict__ src, int n) {
  for (int i = threadIdx.x; i < n / 4; i += blockDim.x)
    reinterpret_cast<float4*>(dst)[i] = reinterpret_cast<const float4*>(src)[i];
}

// ------------------------------------------------------------------------------ router
// Shared expert gate/up rows [i0, i1) over all B tokens, spread over `nw` workers (waves),
// worker `gw`; wg/wu already hold the worker's first row pair when `primed`.  u rows are
// staged in LDS by the caller.
template <typename T, int CPRH, int NT>
__device__ __forceinline__ void shared_rows(const T* __restrict__ ws13, int Is, int i0, int i1,
                                            int gw, int nw, u32x4 (&wg)[Geo<T, CPRH>::CPL],
                                            u32x4 (&wu)[Geo<T, CPRH>::CPL], const float* lds_u,
                                            int k, int B, const Routing& rt, float* As, int lane) {
  int su = i0 + gw;
  if (su >= i1) return;
  while (true) {
    gateup_unit<T, CPRH, NT>(wg, wu, lds_u, 0, B, su, Is, k, true, rt, As, lane);
    su += nw;
    if (su >= i1) break;
    __builtin_amdgcn_sched_barrier(0);
    load_pair<T, CPRH>(ws13, 0, su, Is, wg, wu, lane);
  }
}

// Logit partials part[s][t][e] over `splits` K-slices (one (expert, slice) unit per wave,
// h32 read from L2); with ws13 != nullptr the launch also streams the shared expert's
// gate/up rows [0, i_split), each wave's first row pair requested before the logit work so
// HBM stays busy through this latency-bound phase.
template <typename T, int CPS, int CPRH, int NT>
__global__ __launch_bounds__(kGemvThreads) void router_logits_kernel(
    const float* __restrict__ h32, const T* __restrict__ w_r, int H, int E, int B, int splits,
    float* __restrict__ part, const T* __restrict__ ws13, int Is, int i_split, int k, Routing rt,
    float* __restrict__ As) {
  using G = Geo<T, CPS>;
  using GH = Geo<T, CPRH>;
  extern __shared__ float lds[];  // u [B][H] when the shared rows are streamed here
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wpb = blockDim.x >> 6;
  const int gw = blockIdx.x * wpb + wave, nw = gridDim.x * wpb;
  const bool shared = ws13 != nullptr;
  u32x4 wg[GH::CPL], wu[GH::CPL];
  if (shared && gw < i_split) load_pair<T, CPRH>(ws13, 0, gw, Is, wg, wu, lane);
  const int units = E * splits;
  for (int unit = gw; unit < units; unit += nw) {
    const int e = unit / splits, s = unit - e * splits;
    u32x4 w[G::CPL];
    load_row<T, CPS>(w_r + (size_t)e * H + (size_t)s * G::K, lane, w);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float acc =
          seg_sum<64>(dot_lane<T, CPS>(w, h32 + (size_t)t * H + (size_t)s * G::K, lane));
      if (lane == 0) part[((size_t)s * B + t) * E + e] = acc;
    }
  }
  if (!shared) return;
  stage_rows_f32(lds, h32, B * GH::K);
  __syncthreads();
  shared_rows<T, CPRH, NT>(ws13, Is, 0, i_split, gw, nw, wg, wu, lds, k, B, rt, As, lane);
}

// Block 0: top-k, gates and routing tables from the logit partials.  Blocks 1..: the shared
// expert's gate/up rows [i_split, Is) over all B tokens (ws13 != nullptr), so its weight
// stream overlaps the serial top-k without any cross-block communication.
template <typename T, int CPRH, int NT>
__global__ __launch_bounds__(kGemvThreads) void topk_shared_kernel(
    const float* __restrict__ part, int splits, const float* __restrict__ bias, int E, int k,
    int B, float routed_scale, Routing rt, const T* __restrict__ ws13, int Is, int i_split,
    const float* __restrict__ h32, float* __restrict__ As) {
  using GH = Geo<T, CPRH>;
  extern __shared__ float lds[];  // blocks >= 1: u [B][H]
  if (blockIdx.x == 0) {
    __shared__ TopkScratch sm;
    topk_tables(part, splits, bias, B, E, k, routed_scale, rt, sm);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wpb = blockDim.x >> 6;
  const int nw = (gridDim.x - 1) * wpb;
  const int gw = (blockIdx.x - 1) * wpb + wave;
  u32x4 wg[GH::CPL], wu[GH::CPL];
  if (i_split + gw < Is) load_pair<T, CPRH>(ws13, 0, i_split + gw, Is, wg, wu, lane);
  stage_rows_f32(lds, h32, B * GH::K);
  __syncthreads();
  shared_rows<T, CPRH, NT>(ws13, Is, i_split, Is, gw, nw, wg, wu, lds, k, B, rt, As, lane);
}

// ------------------------------------------------------------------------------ top-k, large batch
// One wave per token (grid = B): topk_idx / topk_gate rows.
__global__ __launch_bounds__(64) void topk_rows_kernel(const float* __restrict__ part, int splits,
                                                       const float* __restrict__ bias, int E,
                                                       int k, int B, float routed_scale,
                                                       Routing rt) {
  topk_row(part, splits, bias, B, E, k, routed_scale, blockIdx.x, rt, nullptr);
}

// One block: routing tables from the topk_idx rows of all B tokens.
__global__ __launch_bounds__(256) void tables_kernel(int E, int k, int B, Routing rt) {
  __shared__ TopkScratch sm;
  for (int i = threadIdx.x; i < B * k; i += blockDim.x) sm.sel[i] = rt.topk_idx[i];
  __syncthreads();
  build_tables(B, E, k, rt, sm);
}

// ------------------------------------------------------------------------------ gate / up
// Routed experts (act / n_act / offsets / perm) or the shared expert (positions = tokens).
template <typename T, int CPR, int NT>
__global__ __launch_bounds__(kGemvThreads) void gateup_gemv_kernel(
    const float* __restrict__ u, const T* __restrict__ w13, int I, int k, int B, int shared,
    Routing rt, float* __restrict__ A) {
  using G = Geo<T, CPR>;
  static_assert(G::SEG == 64, "gate/up rows must span the wave");
  extern __shared__ float lds[];  // u [B][H]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wpb = blockDim.x >> 6;
  const int n = shared ? 1 : *rt.n_act;
  const int units = n * I;
  const int stride = gridDim.x * wpb;
  int unit = blockIdx.x * wpb + wave;

  u32x4 wg[G::CPL], wu[G::CPL];
  auto expert_of = [&](int un) { return shared ? 0 : rt.act[un / I]; };
  if (unit < units) load_pair<T, CPR>(w13, expert_of(unit), unit % I, I, wg, wu, lane);
  stage_rows_f32(lds, u, B * G::K);
  __syncthreads();
  if (unit >= units) return;
  while (true) {
    const int i = unit % I;
    int p0 = 0, p1 = B;
    if (!shared) {
      const int e = rt.act[unit / I];
      p0 = rt.offsets[e];
      p1 = rt.offsets[e + 1];
    }
    gateup_unit<T, CPR, NT>(wg, wu, lds, p0, p1, i, I, k, shared != 0, rt, A, lane);
    unit += stride;
    if (unit >= units) break;
    __builtin_amdgcn_sched_barrier(0);
    load_pair<T, CPR>(w13, expert_of(unit), unit % I, I, wg, wu, lane);
  }
}

// ------------------------------------------------------------------------------ down (per expert)
// Y[p][n] = W2_e[n] . A[p] for every position p of active expert e, and ys[t][n] = Ws2[n] .
// As[t] for the shared expert (unit index n_act).  A unit is R consecutive row groups of
// one expert, so each wave streams a contiguous run of that expert's W2 and consecutive
// waves continue it; the weighted combine is a separate small launch.
template <typename T, int CPR, int NT, int R>
__global__ __launch_bounds__(kGemvThreads) void down_gemv_kernel(
    const float* __restrict__ A, const float* __restrict__ As, const T* __restrict__ w2,
    const T* __restrict__ ws2, int H, int k, int B, Routing rt, float* __restrict__ Y,
    float* __restrict__ ys) {
  using G = Geo<T, CPR>;
  extern __shared__ float lds[];  // A [B*k][I], As [B][I]
  float* sA = lds;
  float* sAs = lds + (size_t)B * k * G::K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wpb = blockDim.x >> 6;
  const int sub = lane % G::SEG, seg = lane / G::SEG;
  const int n_act = *rt.n_act;
  const int rows_per_unit = G::RPW * R;
  const int rb_per_expert = (H + rows_per_unit - 1) / rows_per_unit;
  const int units = (n_act + 1) * rb_per_expert;
  const int stride = gridDim.x * wpb;
  int unit = blockIdx.x * wpb + wave;

  u32x4 w[R][G::CPL];
  auto issue = [&](int u) {
    const int a = u / rb_per_expert, rb = u - a * rb_per_expert;
    const T* base = a < n_act ? w2 + (size_t)rt.act[a] * H * G::K : ws2;
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int n = rb * rows_per_unit + seg + G::RPW * q;
      if (n < H)
        load_row<T, CPR>(base + (size_t)n * G::K, sub, w[q]);
      else
#pragma unroll
        for (int i = 0; i < G::CPL; ++i) w[q][i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (unit < units) issue(unit);
  stage_rows_f32(sA, A, B * k * G::K);
  stage_rows_f32(sAs, As, B * G::K);
  __syncthreads();
  if (unit >= units) return;
  while (true) {
    const int a = unit / rb_per_expert, rb = unit - a * rb_per_expert;
    int p0 = 0, p1 = B;
    const bool routed = a < n_act;
    if (routed) {
      const int e = rt.act[a];
      p0 = rt.offsets[e];
      p1 = rt.offsets[e + 1];
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int n = rb * rows_per_unit + seg + G::RPW * q;
#pragma unroll
      for (int qq = 0; qq < NT; ++qq) {
        const int p = p0 + qq;
        if (p < p1) {
          const float* act = routed ? sA + (size_t)p * G::K : sAs + (size_t)p * G::K;
          const float v = seg_sum<G::SEG>(dot_lane<T, CPR>(w[q], act, sub));
          if (sub == 0 && n < H) (routed ? Y : ys)[(size_t)p * H + n] = v;
        }
      }
    }
    unit += stride;
    if (unit >= units) break;
    __builtin_amdgcn_sched_barrier(0);
    issue(unit);
  }
}

// out[t][n] = RNE(h32[t][n] + sum_j gate[t][j] * Y[inv_perm[t*k+j]][n] + ys[t][n]), j in
// ascending expert order.  KMAX >= k; every load is issued before the sum (clamped indices,
// zero gates past k) so the launch costs one memory latency.
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ h32,
                                                      const float* __restrict__ Y,
                                                      const float* __restrict__ ys, Routing rt,
                                                      int H, int k, int B, T* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H) return;
  const int t = i / H, n = i - t * H;
  float g[KMAX];
  int q[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int slot = t * k + min(j, k - 1);
    g[j] = j < k ? rt.topk_gate[slot] : 0.f;
    q[j] = rt.inv_perm[slot];
  }
  float y[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) y[j] = Y[(size_t)q[j] * H + n];
  float acc = h32[i];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) acc = fmaf(g[j], y[j], acc);
  Elem<T>::store(out, i, acc + ys[i]);
}

// ------------------------------------------------------------------------------ prep
// act / n_act / inv_perm from expert_offsets + perm supplied by the caller.  Tables that are
// not a valid routing of nslots slots (offsets not non-decreasing from 0 to nslots, perm not
// a permutation) set n_act = 0, so no kernel indexes through them.
__global__ __launch_bounds__(64) void moe_prep_kernel(int E, int nslots, Routing rt) {
  const int lane = threadIdx.x;
  const int per = (E + 63) / 64;
  bool ok = true;
  int lf = 0;
  for (int q = 0; q < per; ++q) {
    const int e = lane * per + q;
    if (e < E) {
      const int a = rt.offsets[e], b = rt.offsets[e + 1];
      ok = ok && a >= 0 && b >= a && b <= nslots;
      if (b > a) ++lf;
    }
  }
  if (lane == 0) ok = ok && rt.offsets[0] == 0 && rt.offsets[E] == nslots;
  for (int p = lane; p < nslots; p += 64) {
    const int v = rt.perm[p];
    ok = ok && v >= 0 && v < nslots;
  }
  const bool all_ok = __all(ok);
  int inc = lf;
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(inc, off, 64);
    if (lane >= off) inc += v;
  }
  int pos = inc - lf;
  if (all_ok) {
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      if (e < E && rt.offsets[e + 1] > rt.offsets[e]) rt.act[pos++] = e;
    }
    for (int p = lane; p < nslots; p += 64) rt.inv_perm[rt.perm[p]] = p;
  }
  if (lane == 63) *rt.n_act = all_ok ? inc : 0;
}

// ------------------------------------------------------------------------------ dispatch
// Lets a kernel take more than 64 KB of dynamic LDS (once per kernel instance).
template <typename K>
void allow_lds(K kernel, size_t bytes) {
  static thread_local const void* done[64];
  static thread_local int n_done = 0;
  if (bytes <= 64 * 1024) return;
  for (int i = 0; i < n_done; ++i)
    if (done[i] == (const void*)kernel) return;
  (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
  if (n_done < 64) done[n_done++] = (const void*)kernel;
}

// Persistent launch shape: blocks <= num_cu, 4..8 waves each, preferring a total wave count
// that divides the work evenly (no half-empty last round).
struct LaunchShape {
  int blocks, threads;
};
LaunchShape balanced(const Device& d, int units) {
  for (int wpb = 8; wpb >= 4; --wpb) {
    const int waves = d.num_cu * wpb;
    if (units % waves == 0) return {d.num_cu, wpb * 64};
  }
  const int waves = d.num_cu * 8;
  if (units < waves) return {(units + 7) / 8, 512};
  return {d.num_cu, 512};
}

template <typename T, int CPR, int R>
hipError_t oproj_t(const Shape& s, const Device& d, int B, const void* x, const void* r,
                   const void* w, float* h32, void* h_out, hipStream_t st) {
  // two tokens' activations share the register budget with half as many rows in flight
  constexpr int R2 = (R > 1 && Geo<T, CPR>::CPL > 4) ? R / 2 : R;
  const int rows_per_unit = Geo<T, CPR>::RPW * (B == 1 ? R : R2);
  const int units = (s.H + rows_per_unit - 1) / rows_per_unit;
  const LaunchShape ls = balanced(d, units);
  auto kern = B == 1 ? oproj_gemv_kernel<T, CPR, 1, R> : oproj_gemv_kernel<T, CPR, 2, R2>;
  const size_t lds = 2 * Geo<T, CPR>::CPL > 14 && B == 2 ? 2 * Geo<T, CPR>::K * sizeof(float) : 0;
  hipLaunchKernelGGL(kern, dim3(ls.blocks), dim3(ls.threads), lds, st, (const T*)x, (const T*)r,
                     (const T*)w, h32, (T*)h_out, s.H);
  return hipGetLastError();
}

// Shared expert rows streamed by the logits launch (the rest go with the top-k launch).
inline int shared_split(const Shape& s) { return s.Is / 2; }

template <typename T, int CPS, int CPRH>
hipError_t router_logits_t(const Shape& s, const Device& d, int B, const float* h32,
                           const void* w_r, float* part, const void* ws13, const Routing& rt,
                           float* As, hipStream_t st) {
  const int splits = s.H / Geo<T, CPS>::K;
  const int units = s.E * splits;
  const size_t lds = ws13 ? (size_t)B * Geo<T, CPRH>::K * sizeof(float) : 0;
  auto kern = B == 1 ? router_logits_kernel<T, CPS, CPRH, 1> : router_logits_kernel<T, CPS, CPRH, 2>;
  allow_lds(kern, lds);
  int blocks = (units + 7) / 8;
  if (ws13 && blocks < d.num_cu) blocks = d.num_cu;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kGemvThreads), lds, st, h32, (const T*)w_r, s.H, s.E,
                     B, splits, part, (const T*)ws13, s.Is, ws13 ? shared_split(s) : 0, s.k, rt, As);
  return hipGetLastError();
}

template <typename T, int CPS, int CPRH>
hipError_t topk_shared_t(const Shape& s, const Device& d, int B, const float* part,
                         const float* bias, const Routing& rt, const void* ws13,
                         const float* h32, float* As, hipStream_t st) {
  const int splits = s.H / Geo<T, CPS>::K;
  const size_t lds = ws13 ? (size_t)B * Geo<T, CPRH>::K * sizeof(float) : 0;
  auto kern = B == 1 ? topk_shared_kernel<T, CPRH, 1> : topk_shared_kernel<T, CPRH, 2>;
  allow_lds(kern, lds);
  const int blocks = ws13 ? 1 + d.num_cu : 1;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kGemvThreads), lds, st, part, splits, bias, s.E, s.k,
                     B, s.routed_scale, rt, (const T*)ws13, s.Is, ws13 ? shared_split(s) : s.Is,
                     h32, As);
  return hipGetLastError();
}

template <typename T, int CPR>
hipError_t gateup_t(const Shape& s, const Device& d, int B, const float* u, const void* w13,
                    bool shared, const Routing& rt, float* A, hipStream_t st) {
  const size_t lds = (size_t)B * Geo<T, CPR>::K * sizeof(float);
  auto kern = B == 1 ? gateup_gemv_kernel<T, CPR, 1> : gateup_gemv_kernel<T, CPR, 2>;
  allow_lds(kern, lds);
  const int inter = shared ? s.Is : s.I;
  hipLaunchKernelGGL(kern, dim3(d.num_cu), dim3(kGemvThreads), lds, st, u, (const T*)w13, inter,
                     s.k, B, shared ? 1 : 0, rt, A);
  return hipGetLastError();
}

template <typename T, int CPR>
hipError_t down_t(const Shape& s, const Device& d, int B, const float* A, const float* As,
                  const void* w2, const void* ws2, const Routing& rt, float* Y, float* ys,
                  hipStream_t st) {
  using G = Geo<T, CPR>;
  constexpr int R = G::CPL >= 4 ? 2 : 4;  // rows per unit: 8 KB runs at I = 2048
  const size_t lds = (size_t)(B * s.k + B) * G::K * sizeof(float);
  auto kern = B == 1 ? down_gemv_kernel<T, CPR, 1, R> : down_gemv_kernel<T, CPR, 2, R>;
  allow_lds(kern, lds);
  int bpc = (int)((size_t)d.max_lds / (lds ? lds : 1));
  bpc = bpc < 1 ? 1 : (bpc > 2 ? 2 : bpc);
  hipLaunchKernelGGL(kern, dim3(d.num_cu * bpc), dim3(kGemvThreads), lds, st, A, As, (const T*)w2,
                     (const T*)ws2, s.H, s.k, B, rt, Y, ys);
  return hipGetLastError();
}

template <typename T>
hipError_t combine_t(const Shape& s, int B, const float* h32, const float* Y, const float* ys,
                     const Routing& rt, void* out, hipStream_t st) {
  const int n = B * s.H;
  auto kern = s.k <= 8 ? combine_kernel<T, 8> : combine_kernel<T, 16>;
  hipLaunchKernelGGL(kern, dim3((n + 255) / 256), dim3(256), 0, st, h32, Y, ys, rt, s.H, s.k, B,
                     (T*)out);
  return hipGetLastError();
}

// Chunks (16 B) per row of K elements.
inline int cpr_of(int K, int dtype) { return K * (dtype == 1 ? 2 : 4) / 16; }

}  // namespace

bool gemv_supported(const Shape& s, int B) {
  if (B < 1 || B > 2) return false;
  if (s.I != s.Is) return false;
  if (s.dtype == 1)
    return s.H == 7168 && (s.Ko == 7168 || s.Ko == 448) && (s.I == 2048 || s.I == 128);
  return s.H == 256 && s.Ko == 256 && s.I == 128;
}

int router_gemv_splits(const Shape& s) { return s.dtype == 1 ? 7 : 1; }

hipError_t launch_oproj_gemv(const Shape& s, const Device& d, int B, const void* x, const void* r,
                             const void* w_o, float* h32, void* h_out, hipStream_t st) {
  const int c = cpr_of(s.Ko, s.dtype);
  if (s.dtype == 1) {
    if (c == 896) return oproj_t<uint16_t, 896, 2>(s, d, B, x, r, w_o, h32, h_out, st);
    if (c == 56) return oproj_t<uint16_t, 56, 4>(s, d, B, x, r, w_o, h32, h_out, st);
  } else if (c == 64) {
    return oproj_t<float, 64, 2>(s, d, B, x, r, w_o, h32, h_out, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_router_logits(const Shape& s, const Device& d, int B, const float* h32,
                                const void* w_r, float* part, const void* ws13, const Routing& rt,
                                float* As, hipStream_t st) {
  if (s.dtype == 1 && s.H == 7168)
    return router_logits_t<uint16_t, 128, 896>(s, d, B, h32, w_r, part, ws13, rt, As, st);
  if (s.dtype == 0 && s.H == 256)
    return router_logits_t<float, 64, 64>(s, d, B, h32, w_r, part, ws13, rt, As, st);
  return hipErrorInvalidValue;
}

hipError_t launch_topk_shared(const Shape& s, const Device& d, int B, const float* part,
                              const float* bias, const Routing& rt, const void* ws13,
                              const float* h32, float* As, hipStream_t st) {
  if (s.dtype == 1 && s.H == 7168)
    return topk_shared_t<uint16_t, 128, 896>(s, d, B, part, bias, rt, ws13, h32, As, st);
  if (s.dtype == 0 && s.H == 256)
    return topk_shared_t<float, 64, 64>(s, d, B, part, bias, rt, ws13, h32, As, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gateup_gemv(const Shape& s, const Device& d, int B, const float* u,
                              const void* w13, bool shared, const Routing& rt, float* A,
                              hipStream_t st) {
  const int c = cpr_of(s.H, s.dtype);
  if (s.dtype == 1 && c == 896) return gateup_t<uint16_t, 896>(s, d, B, u, w13, shared, rt, A, st);
  if (s.dtype == 0 && c == 64) return gateup_t<float, 64>(s, d, B, u, w13, shared, rt, A, st);
  return hipErrorInvalidValue;
}

hipError_t launch_down_gemv(const Shape& s, const Device& d, int B, const float* A,
                            const float* As, const void* w2, const void* ws2, const Routing& rt,
                            float* Y, float* ys, hipStream_t st) {
  const int c = cpr_of(s.I, s.dtype);
  if (s.dtype == 1) {
    if (c == 256) return down_t<uint16_t, 256>(s, d, B, A, As, w2, ws2, rt, Y, ys, st);
    if (c == 16) return down_t<uint16_t, 16>(s, d, B, A, As, w2, ws2, rt, Y, ys, st);
  } else if (c == 32) {
    return down_t<float, 32>(s, d, B, A, As, w2, ws2, rt, Y, ys, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const Shape& s, int B, const float* h32, const float* Y, const float* ys,
                          const Routing& rt, void* out, hipStream_t st) {
  if (s.dtype == 1) return combine_t<uint16_t>(s, B, h32, Y, ys, rt, out, st);
  return combine_t<float>(s, B, h32, Y, ys, rt, out, st);
}

hipError_t launch_topk_rows(const Shape& s, int B, const float* part, int splits,
                            const float* bias, const Routing& rt, hipStream_t st) {
  hipLaunchKernelGGL(topk_rows_kernel, dim3(B), dim3(64), 0, st, part, splits, bias, s.E, s.k, B,
                     s.routed_scale, rt);
  return hipGetLastError();
}

hipError_t launch_tables(const Shape& s, int B, const Routing& rt, hipStream_t st) {
  hipLaunchKernelGGL(tables_kernel, dim3(1), dim3(256), 0, st, s.E, s.k, B, rt);
  return hipGetLastError();
}

hipError_t launch_moe_prep(const Shape& s, int B, const Routing& rt, hipStream_t st) {
  hipLaunchKernelGGL(moe_prep_kernel, dim3(1), dim3(64), 0, st, s.E, B * s.k, rt);
  return hipGetLastError();
}

}  // namespace kk

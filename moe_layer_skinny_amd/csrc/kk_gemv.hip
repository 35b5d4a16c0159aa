// GEMV path of the decode-layer step (batch 1-2): every weight row is streamed from HBM
// once with 128-bit non-temporal loads, each row's dot product finished with a wavefront
// (DPP) reduction.  One stream, four launches per step:
//   1. o-proj + residual                     (activations held in registers)
//   2. router logits (K-slice partials)      ||  shared expert gate/up
//   3. top-k, gates and routing tables (every block, from the partials)  ||  shared expert
//      down-projection; then the routed gate/up over the active experts
//   4. routed down-projection with the weighted combine into the residual
// A layer without a norm can run three (a 448-wide o-proj slice at batch 1-2, a full-width one
// at batch 2): the router logits come from r and x through the router-o-proj product in the
// o-proj's launch, the top-k runs in the routed gate/up launch beside the shared expert's
// gate/up, and the shared down-projection joins the last launch.
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
template <typename T, int CPR, int NT, int R, int WPE = 2>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(WPE))) void oproj_gemv_kernel(
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

// Rows of T (16-byte chunks) -> fp32 in LDS, n elements (n a multiple of a chunk's elements).
template <typename T>
__device__ __forceinline__ void stage_to_f32(const T* __restrict__ src, int n, float* dst) {
  constexpr int EPC = Elem<T>::EPC;
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  for (int c = threadIdx.x; c < n / EPC; c += blockDim.x) {
    float f[EPC];
    Elem<T>::unpack(s[c], f);
    float4* d = reinterpret_cast<float4*>(dst + (size_t)c * EPC);
#pragma unroll
    for (int h = 0; h < EPC / 4; ++h) d[h] = make_float4(f[4 * h], f[4 * h + 1], f[4 * h + 2], f[4 * h + 3]);
  }
}

// ------------------------------------------------------------------------------ o-proj + router
// The o-proj and the router logits in one launch, the router not waiting for h: the logit
// W_r[e] . h_t = W_r[e] . r_t + (W_r W_o)[e] . x_t, with mr = W_r W_o computed once per layer
// (router_oproj_product_kernel) and kept as npl planes of T whose sum is its fp32 value,
// laid out [npl][E][Ko].  The unit space has H + npl E rows of Ko elements:
//  * rows 0..H-1 are W_o's: h32[t][n] = r[t][n] + W_o[n] . x_t (and h_out = RNE(h32));
//  * row H + p E + e is plane p of mr[e]: part[RS + p][t][e] = mr_p[e] . x_t.
// Besides its rows, the wave with global id g < E RS (ids across the blocks first) takes slice
// sl = g % RS of router row e = g / RS against r, staged in LDS as fp32:
// part[sl][t][e] = W_r[e][slice sl] . r_t.  The top-k sums the RS + npl partials of (t, e) in
// slot order.  x sits in registers as in oproj_gemv_kernel when it fits, else in LDS.
template <typename T, int CPR, int CPS, int NT, int R, int WPE = 2>
__global__ __launch_bounds__(kGemvThreads) __attribute__((amdgpu_waves_per_eu(WPE))) void oproj_router_gemv_kernel(
    const T* __restrict__ x, const T* __restrict__ r, const T* __restrict__ w_o,
    const T* __restrict__ w_r, const T* __restrict__ mr, int npl, float* __restrict__ h32,
    T* __restrict__ h_out, float* __restrict__ part, int H, int E, int RS) {
  using G = Geo<T, CPR>;
  using GS = Geo<T, CPS>;
  static_assert(GS::SEG == 64, "router slices span the wave");
  constexpr bool kRegs = NT * G::CPL <= 14;
  extern __shared__ float lds[];  // r as fp32 [NT][H], then x as fp32 [NT][Ko] if not in registers
  float* lr = lds;
  float* lx = lds + (size_t)NT * H;
  const int lane = threadIdx.x & 63, wpb = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % G::SEG, seg = lane / G::SEG;
  const int rows = H + npl * E;
  const int rows_per_unit = G::RPW * R;
  const int units = (rows + rows_per_unit - 1) / rows_per_unit;
  const int stride = gridDim.x * wpb;
  int unit = blockIdx.x * wpb + wave;

  // this thread's chunks of r, requested first: staging them then waits for them alone, not for
  // the weight loads queued behind (loads complete in order)
  constexpr int EPC = Elem<T>::EPC, RQ = 4;
  const int nrc = NT * H / EPC;
  const u32x4* rsrc = reinterpret_cast<const u32x4*>(r);
  u32x4 rc[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) rc[q] = rsrc[min((int)threadIdx.x + q * (int)blockDim.x, nrc - 1)];
  // this wave's router slice
  const int gs = wave * gridDim.x + blockIdx.x;
  const bool has_slice = gs < E * RS;
  const int se = has_slice ? gs / RS : 0, ssl = has_slice ? gs - se * RS : 0;
  u32x4 wr[GS::CPL];
  if (has_slice) load_row<T, CPS>(w_r + (size_t)se * H + (size_t)ssl * GS::K, lane, wr);

  u32x4 w[R][G::CPL];
  auto issue = [&](int u) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int n = u * rows_per_unit + seg + G::RPW * q;
      if (n < rows)
        load_row<T, CPR>(n < H ? w_o + (size_t)n * G::K : mr + (size_t)(n - H) * G::K, sub, w[q]);
      else
#pragma unroll
        for (int i = 0; i < G::CPL; ++i) w[q][i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  if (unit < units) issue(unit);
  u32x4 xa[kRegs ? NT : 1][G::CPL];
  if constexpr (kRegs) {
#pragma unroll
    for (int t = 0; t < NT; ++t) load_act_chunks<T, CPR>(x + (size_t)t * G::K, sub, xa[t]);
  }
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int c = threadIdx.x + q * blockDim.x;
    if (c < nrc) {
      float f[EPC];
      Elem<T>::unpack(rc[q], f);
      float4* d = reinterpret_cast<float4*>(lr + (size_t)c * EPC);
#pragma unroll
      for (int h = 0; h < EPC / 4; ++h) d[h] = make_float4(f[4 * h], f[4 * h + 1], f[4 * h + 2], f[4 * h + 3]);
    }
  }
  for (int c = threadIdx.x + RQ * blockDim.x; c < nrc; c += blockDim.x) {
    float f[EPC];
    Elem<T>::unpack(rsrc[c], f);
    float4* d = reinterpret_cast<float4*>(lr + (size_t)c * EPC);
#pragma unroll
    for (int h = 0; h < EPC / 4; ++h) d[h] = make_float4(f[4 * h], f[4 * h + 1], f[4 * h + 2], f[4 * h + 3]);
  }
  if constexpr (!kRegs) stage_to_f32<T>(x, NT * G::K, lx);
  __syncthreads();
  if (has_slice) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v = seg_sum_dpp<64>(dot_lane<T, CPS>(wr, lr + (size_t)t * H + (size_t)ssl * GS::K, lane));
      if (lane == 63) part[((size_t)ssl * NT + t) * E + se] = v;
    }
  }
  if (unit >= units) return;

  while (true) {
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int n = unit * rows_per_unit + seg + G::RPW * q;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float d;
        if constexpr (kRegs)
          d = dot_rr<T, CPR>(w[q], xa[t], sub);
        else
          d = dot_lane<T, CPR>(w[q], lx + t * G::K, sub);
        const float acc = seg_sum<G::SEG>(d);
        if (sub == 0 && n < rows) {
          if (n < H) {
            const size_t o = (size_t)t * H + n;
            const float hv = Elem<T>::load(r, o) + acc;
            h32[o] = hv;
            if (h_out) Elem<T>::store(h_out, o, hv);
          } else {
            const int pl = (n - H) / E, e = (n - H) - pl * E;
            part[((size_t)(RS + pl) * NT + t) * E + e] = acc;
          }
        }
      }
    }
    unit += stride;
    if (unit >= units) break;
    __builtin_amdgcn_sched_barrier(0);
    issue(unit);
  }
}

// The router-o-proj product of a layer, once: M[e][j] = sum_n W_r[e][n] W_o[n][j], accumulated
// in fp64, rounded to fp32 and stored as npl planes of T ([npl][E][Ko]): bf16 hi = RNE(m),
// lo = RNE(m - hi) (their sum reproduces m to 2^-17 relative); fp32 one plane, m itself.
// (A logit's error from the two planes: about 2^-17 of |M| |x| per term, ~1e-6 over 448
// terms and ~2e-5 over 7168 (|M| ~ 0.034 for weights of scale 0.02), far below the 1e-3 gap
// the selection keeps.)
// Block tile 32 experts x 64 columns, 32-wide steps along n staged in LDS; each thread owns
// 2 x 4 outputs.
template <typename T>
__global__ __launch_bounds__(256) void router_oproj_product_kernel(const T* __restrict__ w_r,
                                                                   const T* __restrict__ w_o, int E,
                                                                   int H, int Ko, T* __restrict__ mr,
                                                                   int npl) {
  __shared__ double sr[32][33];  // W_r tile [e][n]
  __shared__ double so[32][65];  // W_o tile [n][j]
  const int e0 = blockIdx.y * 32, j0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;  // columns j0 + 4 tx .., experts e0 + 2 ty ..
  double acc[2][4] = {};
  for (int n0 = 0; n0 < H; n0 += 32) {
    for (int i = threadIdx.x; i < 32 * 32; i += 256) {
      const int ee = i >> 5, nn = i & 31;
      sr[ee][nn] = e0 + ee < E && n0 + nn < H ? (double)Elem<T>::load(w_r, (size_t)(e0 + ee) * H + n0 + nn) : 0.0;
    }
    for (int i = threadIdx.x; i < 32 * 64; i += 256) {
      const int nn = i >> 6, jj = i & 63;
      so[nn][jj] = n0 + nn < H && j0 + jj < Ko ? (double)Elem<T>::load(w_o, (size_t)(n0 + nn) * Ko + j0 + jj) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int nn = 0; nn < 32; ++nn) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(sr[2 * ty + a][nn], so[nn][4 * tx + b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int e = e0 + 2 * ty + a, j = j0 + 4 * tx + b;
      if (e < E && j < Ko) {
        const float m = (float)acc[a][b];
        T* dst = mr + (size_t)e * Ko + j;
        if (npl == 1) {
          Elem<T>::store(dst, 0, m);
        } else {
          const uint16_t hi = f32_to_bf16(m);
          const float lo = m - __uint_as_float((uint32_t)hi << 16);
          Elem<T>::store(dst, 0, __uint_as_float((uint32_t)hi << 16));
          Elem<T>::store(dst, (size_t)E * Ko, lo);
        }
      }
    }
}

// ------------------------------------------------------------------------------ gate / up helpers
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
      // same per-lane order and lane combining as the routed gate/up kernel
      z1 = seg_sum_dpp<64>(z1);
      z3 = seg_sum_dpp<64>(z3);
      if (lane == 63) A[(size_t)p * I + i] = silu_f32(z1) * z3;
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

// Global -> LDS copy of n floats (n % 4 == 0, n > 0) in two halves: load() puts a thread's
// first Q float4s in registers, all in flight together (indices clamped instead of branched
// around), so it can be issued ahead of a weight stream; store() writes them to LDS after it,
// waiting only on these loads, and copies anything past Q * blockDim.x float4s by a loop.
template <int Q>
struct Stage {
  float4 v[Q];
  const float4* src;
  int n4;
  __device__ __forceinline__ void load(const float* __restrict__ s, int n) {
    src = reinterpret_cast<const float4*>(s);
    n4 = n / 4;
#pragma unroll
    for (int j = 0; j < Q; ++j) v[j] = src[min((int)(threadIdx.x + j * blockDim.x), n4 - 1)];
  }
  __device__ __forceinline__ void store(float* d) const {
    float4* dst = reinterpret_cast<float4*>(d);
    // past the end the last float4 is written again with its own value (no branch)
#pragma unroll
    for (int j = 0; j < Q; ++j) dst[min((int)(threadIdx.x + j * blockDim.x), n4 - 1)] = v[j];
    for (int i = threadIdx.x + Q * blockDim.x; i < n4; i += blockDim.x) dst[i] = src[i];
  }
  // Instead of h, stores u = h * gamma / sqrt(mean(h^2) + eps) for each token row of H floats
  // (H % 4 == 0; the Q float4s of the block cover all rows, NT of them at most).  Sums of
  // squares go per thread, per wave (DPP), then over the waves in wave order through
  // red[NT * waves], so every block of one launch shape writes the same bits.
  template <typename T, int NT>
  __device__ __forceinline__ void store_rmsnorm(float* d, const T* __restrict__ gamma, float eps,
                                                int H, float* red) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwv = blockDim.x >> 6;
    const int h4 = H / 4;
    float ss[NT];
    float4 g[Q];
#pragma unroll
    for (int t = 0; t < NT; ++t) ss[t] = 0.f;
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      const int i = threadIdx.x + j * blockDim.x;
      const int ic = min(i, n4 - 1);
      const int t = NT == 1 ? 0 : ic / h4;
      g[j] = Elem<T>::load4(gamma, (size_t)(ic - t * h4) * 4);
      const float4 x = v[j];
      const float sq = i < n4 ? x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w : 0.f;
#pragma unroll
      for (int q = 0; q < NT; ++q) ss[q] += q == t ? sq : 0.f;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      ss[t] = seg_sum_dpp<64>(ss[t]);
      if (lane == 63) red[wave * NT + t] = ss[t];
    }
    __syncthreads();
    float inv[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float sum = 0.f;
      for (int w = 0; w < nwv; ++w) sum += red[w * NT + t];
      inv[t] = 1.f / sqrtf(sum / (float)H + eps);
    }
    float4* dst = reinterpret_cast<float4*>(d);
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      // past the end the last float4 is written again with its own value
      const int ic = min((int)(threadIdx.x + j * blockDim.x), n4 - 1);
      const float r = inv[NT == 1 ? 0 : ic / h4];
      const float4 x = v[j];
      dst[ic] = make_float4(x.x * r * g[j].x, x.y * r * g[j].y, x.z * r * g[j].z,
                            x.w * r * g[j].w);
    }
  }
};

// float4s per thread that cover `rows` fp32 rows of K elements with kGemvThreads threads.
constexpr int stage_q(int rows, int K) { return (rows * K / 4 + kGemvThreads - 1) / kGemvThreads; }

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

// Router logit partials part[s][t][e] = h32[t][slice s] . W_r[e][slice s] (at most two
// (expert, slice) units per wave) and, with ws13 != nullptr, the shared expert's gate/up
// rows, As[t][i] = silu(Ws1[i] . u_t) * (Ws3[i] . u_t).  Every wave requests its share of the
// activation rows, then its router slices and its first shared row pair, at the start, so the
// launch streams both weight sets at full bandwidth; the top-k runs at the start of the routed
// gate/up launch.
template <typename T, int CPS, int CPRH, int NT>
__global__ __launch_bounds__(kGemvThreads) void router_logits_kernel(
    const float* __restrict__ h32, const T* __restrict__ w_r, int H, int E, int B, int splits,
    float* __restrict__ part, const T* __restrict__ ws13, int Is, int k, Routing rt,
    float* __restrict__ As, const T* __restrict__ gamma, float eps) {
  using G = Geo<T, CPS>;
  using GH = Geo<T, CPRH>;
  constexpr int MAXU = 2;  // (expert, slice) units per wave; the host checks E * splits
  extern __shared__ float lds[];  // u [B][H]
  __shared__ float nred[(kGemvThreads / 64) * NT];
  const int lane = threadIdx.x & 63, wpb = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // worker ids run across the blocks first, so a short list of units (the shared expert's
  // row pairs when its intermediate is small) is spread over the CUs
  const int gw = wave * gridDim.x + blockIdx.x, nw = gridDim.x * wpb;
  const bool shared = ws13 != nullptr;
  const int units = E * splits;
  // The activation rows are requested first: staging them then waits for them alone, not for
  // the weight loads queued behind (loads complete in order), so every wave can multiply as soon
  // as its own weights arrive instead of after the whole block's.
  Stage<stage_q(NT, GH::K)> st;
  st.load(h32, B * H);
  // router slices of this wave's units (a missing second unit re-reads the last one)
  u32x4 wr[MAXU][G::CPL];
#pragma unroll
  for (int j = 0; j < MAXU; ++j) {
    const int un = min(gw + j * nw, units - 1);
    const int e = un / splits, sl = un - e * splits;
    load_row<T, CPS>(w_r + (size_t)e * H + (size_t)sl * G::K, lane, wr[j]);
  }
  u32x4 wg[GH::CPL], wu[GH::CPL];
  if (shared && gw < Is) load_pair<T, CPRH>(ws13, 0, gw, Is, wg, wu, lane);
  if (gamma)
    st.template store_rmsnorm<T, NT>(lds, gamma, eps, H, nred);
  else
    st.store(lds);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < MAXU; ++j) {
    const int un = gw + j * nw;
    if (un < units) {
      const int e = un / splits, sl = un - e * splits;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float v = seg_sum_dpp<64>(dot_lane<T, CPS>(wr[j], lds + t * H + sl * G::K, lane));
        if (t < B && lane == 63) part[((size_t)sl * B + t) * E + e] = v;
      }
    }
  }
  if (shared) shared_rows<T, CPRH, NT>(ws13, Is, 0, Is, gw, nw, wg, wu, lds, k, B, rt, As, lane);
}

// ------------------------------------------------------------------------------ prefetch
// Reads n 16-byte chunks once with plain loads, which allocate in the caches on their way, and
// keeps nothing: a later launch that reads the same bytes is served from the memory-side cache.
__global__ __launch_bounds__(256) void prefetch_kernel(const u32x4* __restrict__ p, size_t n) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const u32x4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  asm volatile("" ::"v"(acc));  // the loads stay; nothing is stored
}

// ------------------------------------------------------------------------------ delay
// Waits `ticks` of the constant-rate device clock, sleeping between reads, then returns; the
// loop also stops after 2^22 sleeps (about a second), so the wave ends even if the clock
// stalls.  A test hook: placed first on one stream, it lets the other run ahead.
__global__ __launch_bounds__(64) void delay_kernel(long long ticks) {
  const long long t0 = wall_clock64();
  for (int i = 0; i < (1 << 22) && wall_clock64() - t0 < ticks; ++i) __builtin_amdgcn_s_sleep(8);
}

// ------------------------------------------------------------------------------ top-k, large batch
// One wave per token (grid = B): topk_idx / topk_gate rows.
__global__ __launch_bounds__(64) void topk_rows_kernel(const float* __restrict__ part, int splits,
                                                       const float* __restrict__ bias, int E,
                                                       int k, int B, float routed_scale,
                                                       Routing rt) {
  topk_row(part, splits, bias, B, E, k, routed_scale, blockIdx.x, rt, nullptr);
}

// Up to 16 tokens in one block: wave t writes token t's top-k row, then the block builds the
// routing tables (one launch instead of two).
__global__ __launch_bounds__(1024) void topk_tables_kernel(const float* __restrict__ part,
                                                          int splits,
                                                          const float* __restrict__ bias, int E,
                                                          int k, int B, float routed_scale,
                                                          Routing rt) {
  __shared__ TopkScratch sm;
  const int wave = threadIdx.x >> 6;
  if (wave < B) topk_row(part, splits, bias, B, E, k, routed_scale, wave, rt, sm.sel);
  __syncthreads();
  build_tables(B, E, k, rt, sm);
}

// One block: routing tables from the topk_idx rows of all B tokens.
__global__ __launch_bounds__(256) void tables_kernel(int E, int k, int B, Routing rt) {
  __shared__ TopkScratch sm;
  for (int i = threadIdx.x; i < B * k; i += blockDim.x) sm.sel[i] = rt.topk_idx[i];
  __syncthreads();
  build_tables(B, E, k, rt, sm);
}

// ------------------------------------------------------------------------------ gate / up
// Shared expert's down-projection rows for this launch's workers (waves 1.. of every block):
// ys[t][n] = Ws2[n] . As[t] over row groups g = worker, worker + nworkers, ...; each worker
// requests up to R row groups at once.
template <typename T, int CPRS, int NT, int R>
__device__ __forceinline__ void shared_down_rows(const T* __restrict__ ws2,
                                                 const float* __restrict__ As,
                                                 float* __restrict__ ys, int H, int B,
                                                 int worker, int nworkers, int lane) {
  using G = Geo<T, CPRS>;
  const int sub = lane % G::SEG, seg = lane / G::SEG;
  const int groups = (H + G::RPW - 1) / G::RPW;
  // the lane's activation values (As is fp32 [B][Is])
  float xa[NT][G::CPL][G::EPC];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int i = 0; i < G::CPL; ++i) {
      const int c = min(sub + G::SEG * i, CPRS - 1);
      const float4* p = reinterpret_cast<const float4*>(As + (size_t)min(t, B - 1) * G::K + c * G::EPC);
#pragma unroll
      for (int h = 0; h < G::EPC / 4; ++h) {
        const float4 v = p[h];
        xa[t][i][4 * h + 0] = v.x;
        xa[t][i][4 * h + 1] = v.y;
        xa[t][i][4 * h + 2] = v.z;
        xa[t][i][4 * h + 3] = v.w;
      }
    }
  for (int g0 = worker; g0 < groups; g0 += R * nworkers) {
    u32x4 w[R][G::CPL];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int n = min((g0 + q * nworkers) * G::RPW + seg, H - 1);
      load_row<T, CPRS>(ws2 + (size_t)n * G::K, sub, w[q]);
    }
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int g = g0 + q * nworkers;
      const int n = g * G::RPW + seg;
      float acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = 0.f;
#pragma unroll
      for (int i = 0; i < G::CPL; ++i) {
        if (G::EXACT || sub + G::SEG * i < CPRS) {
          float f[G::EPC];
          Elem<T>::unpack(w[q][i], f);
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int x = 0; x < G::EPC; ++x) acc[t] = fmaf(f[x], xa[t][i][x], acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("" : "+v"(acc[t]));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float v = seg_sum_dpp<G::SEG>(acc[t]);
        if (t < B && g < groups && n < H && sub == G::SEG - 1) ys[(size_t)t * H + n] = v;
      }
    }
  }
}

// Routing tables held in LDS by the routed gate/up launch when it runs the top-k itself.
struct LdsTables {
  int idx[kMaxSlots];
  float gate[kMaxSlots];
  int perm[kMaxSlots];
  int inv[kMaxSlots];
  int offsets[kMaxExperts + 1];
  int act[kMaxExperts];
  int n_act;
};

// Routed experts (act / n_act / offsets / perm) or the shared expert (positions = tokens).
// One wave per (expert, row i) unit: gate row i and up row i against the unit's tokens,
// A[position][i] = silu(W1[i] . u_t) * (W3[i] . u_t).  A unit's two rows are fetched in two
// K halves that alternate with their consumption, so a wave always has one half in flight
// while it works on the other (a unit past the end fetches from the activation buffer, so
// no load is branched around).  Tables come from the wave's own lanes: lane j holds act[j],
// the first position of that expert and its position count, lane p the token of position p.
//
// Before the routed rows, the launch can do work that only needs the previous launch:
//  * TOPK: every block runs the top-k from the logit partials (wave t: token t) and builds the
//    routing tables in its own LDS -- the same bits in every block; block 0 also writes
//    them out (topk_idx / topk_gate / offsets / perm / inv_perm / act / n_act);
//  * ws13 != nullptr: the other waves compute the shared expert's gate/up into As_out, so its
//    weight stream covers the top-k's latency; or
//  * ws2 != nullptr: waves 1.. compute the shared expert's down-projection into ys from As.
template <typename T, int CPR, int CPRS, int NT, bool TOPK, bool SGU>
__global__ __launch_bounds__(kGemvThreads) void gateup_gemv_kernel(
    const float* __restrict__ u, const T* __restrict__ w13, int I, int k, int B, int shared,
    Routing rt, float* __restrict__ A, const float* __restrict__ part, int splits,
    const float* __restrict__ bias, int E, float routed_scale, const T* __restrict__ ws2,
    const float* __restrict__ As, float* __restrict__ ys, int H, const T* __restrict__ gamma,
    float eps, const T* __restrict__ ws13, int Is, float* __restrict__ As_out) {
  using G = Geo<T, CPR>;
  static_assert(G::SEG == 64 && G::EXACT, "gate/up rows must span the wave exactly");
  constexpr int HA = (G::CPL + 1) / 2, HB = G::CPL - HA;
  extern __shared__ float lds[];  // u [B][K]
  __shared__ float nred[(kGemvThreads / 64) * NT];
  __shared__ TopkScratch sm;
  __shared__ LdsTables tb;
  __shared__ float lg[TOPK ? 2 * kMaxExperts : 1];
  __shared__ float lb[SGU ? kMaxExperts : 1];  // the bias, when the selection runs after the staging
  __shared__ int next_unit;  // two tokens, full-size rows: the block's next unit (unit loop)
  const int lane = threadIdx.x & 63, wpb = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nslot = B * k;
  if (NT > 1 && CPRS >= 256 && threadIdx.x == 0) next_unit = wpb;  // (read after the barriers below)
  // the logits first, by the whole block, before any weight stream competes with their loads;
  // the waves that run a token's selection (wave t: token t) request their bias values with
  // them.  With the shared gate/up (SGU), the waves past the selecting ones request their
  // first shared row pair before that (one token; with two, the pair waits for the staging, as
  // the registers would not hold it beside the staged rows).
  const int sw = (wave - B) * gridDim.x + blockIdx.x, nsw = gridDim.x * (wpb - B);
  u32x4 sg[SGU ? G::CPL : 1], su[SGU ? G::CPL : 1];
  if constexpr (SGU && NT == 1)
    if (wave >= B && sw < Is) load_pair<T, CPR>(ws13, 0, sw, Is, sg, su, lane);
  float bv[kMaxM];
  if (TOPK && !SGU && wave < B) load_bias(bias, E, bv);
  if constexpr (SGU)
    for (int i = threadIdx.x; i < E; i += blockDim.x) lb[i] = bias[i];
  Stage<stage_q(NT, G::K)> st;
  // (with the shared gate/up the activation rows are requested with the logits, so the two
  // round trips overlap; otherwise after them, so the logits are not queued behind)
  if constexpr (SGU) st.load(u, B * G::K);
  if (TOPK) {
    logits_to_lds(part, splits, B, E, lg);
    __syncthreads();
  }
  if constexpr (!SGU) st.load(u, B * G::K);
  if constexpr (SGU) {
    // the shared expert's gate/up rows read u, so it goes to LDS first; then the selecting
    // waves run the top-k while the others stream the shared rows into As_out
    if (gamma)
      st.template store_rmsnorm<T, NT>(lds, gamma, eps, G::K, nred);
    else
      st.store(lds);
    __syncthreads();
    if (TOPK && wave < B) {
      Routing rl{tb.idx, tb.gate, tb.offsets, tb.perm, tb.inv, tb.act, &tb.n_act};
#pragma unroll
      for (int m = 0; m < kMaxM; ++m) bv[m] = lb[min(lane + 64 * m, E - 1)];
      topk_row_lds(lg, bv, E, k, routed_scale, wave, rl, sm.sel);
    }
    if (wave >= B) {
      if constexpr (NT > 1)
        if (sw < Is) load_pair<T, CPR>(ws13, 0, sw, Is, sg, su, lane);
      __builtin_amdgcn_sched_barrier(0);
      shared_rows<T, CPR, NT>(ws13, Is, 0, Is, sw, nsw, sg, su, lds, k, B, rt, As_out, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    if (TOPK && wave < B) {
      Routing rl{tb.idx, tb.gate, tb.offsets, tb.perm, tb.inv, tb.act, &tb.n_act};
      topk_row_lds(lg, bv, E, k, routed_scale, wave, rl, sm.sel);
    }
    if (ws2 && wave > 0)
      shared_down_rows<T, CPRS, NT, 4>(ws2, As, ys, H, B, (wave - 1) * gridDim.x + blockIdx.x,
                                       gridDim.x * (wpb - 1), lane);
    if (gamma)
      st.template store_rmsnorm<T, NT>(lds, gamma, eps, G::K, nred);
    else
      st.store(lds);
  }
  __syncthreads();
  if (TOPK) {
    Routing rl{tb.idx, tb.gate, tb.offsets, tb.perm, tb.inv, tb.act, &tb.n_act};
    build_tables(B, E, k, rl, sm);
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int i = threadIdx.x; i < nslot; i += blockDim.x) {
        rt.topk_idx[i] = tb.idx[i];
        rt.topk_gate[i] = tb.gate[i];
        rt.perm[i] = tb.perm[i];
        rt.inv_perm[i] = tb.inv[i];
      }
      for (int i = threadIdx.x; i <= E; i += blockDim.x) rt.offsets[i] = tb.offsets[i];
      for (int i = threadIdx.x; i < tb.n_act; i += blockDim.x) rt.act[i] = tb.act[i];
      if (threadIdx.x == 0) *rt.n_act = tb.n_act;
    }
  }
  // (act has at least 64 entries; entries past n_act are not expert ids)
  const int* act = TOPK ? tb.act : rt.act;
  const int* offsets = TOPK ? tb.offsets : rt.offsets;
  const int* perm = TOPK ? tb.perm : rt.perm;
  const int t_a = act[lane];
  const int t_p = perm[min(lane, nslot - 1)];
  const int n = shared ? 1 : min(TOPK ? tb.n_act : *rt.n_act, 64);
  const int t_e = (!shared && lane < n) ? t_a : 0;
  const int t_lo = shared ? 0 : offsets[t_e];
  const int t_cnt = shared ? B : offsets[t_e + 1] - t_lo;
  const int t_tok = min(max(t_p / k, 0), B - 1);

  const int units = n * I;
  const int stride = gridDim.x * wpb;
  const T* dummy = reinterpret_cast<const T*>(u);
  u32x4 ga[HA], ua[HA], gb[HB > 0 ? HB : 1], ub[HB > 0 ? HB : 1];
  auto rows = [&](int un, const T*& g, const T*& up) {
    const int a = un / I, i = un - a * I;
    const int e = __builtin_amdgcn_readlane(t_e, min(a, 63));
    g = w13 + ((size_t)e * 2 * I + i) * G::K;
    up = g + (size_t)I * G::K;
    if (un >= units) g = up = dummy;
  };
  auto issue_a = [&](int un) {
    const T *g, *up;
    rows(un, g, up);
    const u32x4* pg = reinterpret_cast<const u32x4*>(g);
    const u32x4* pu = reinterpret_cast<const u32x4*>(up);
#pragma unroll
    for (int i = 0; i < HA; ++i) {
      ga[i] = __builtin_nontemporal_load(pg + lane + 64 * i);
      ua[i] = __builtin_nontemporal_load(pu + lane + 64 * i);
    }
  };
  auto issue_b = [&](int un) {
    const T *g, *up;
    rows(un, g, up);
    const u32x4* pg = reinterpret_cast<const u32x4*>(g);
    const u32x4* pu = reinterpret_cast<const u32x4*>(up);
#pragma unroll
    for (int i = 0; i < HB; ++i) {
      gb[i] = __builtin_nontemporal_load(pg + lane + 64 * (HA + i));
      ub[i] = __builtin_nontemporal_load(pu + lane + 64 * (HA + i));
    }
  };
  float z1[NT], z3[NT];
  // chunk j of both rows against the activation rows of the unit's tokens
  auto eat = [&](const u32x4& wg, const u32x4& wu, int j, const float* const (&xr)[NT]) {
    float fg[G::EPC], fu[G::EPC];
    Elem<T>::unpack(wg, fg);
    Elem<T>::unpack(wu, fu);
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const float4* x = reinterpret_cast<const float4*>(xr[q] + 64 * j * G::EPC);
#pragma unroll
      for (int h = 0; h < G::EPC / 4; ++h) {
        const float4 v = x[h];
        z1[q] = fmaf(fg[4 * h + 0], v.x, z1[q]);
        z3[q] = fmaf(fu[4 * h + 0], v.x, z3[q]);
        z1[q] = fmaf(fg[4 * h + 1], v.y, z1[q]);
        z3[q] = fmaf(fu[4 * h + 1], v.y, z3[q]);
        z1[q] = fmaf(fg[4 * h + 2], v.z, z1[q]);
        z3[q] = fmaf(fu[4 * h + 2], v.z, z3[q]);
        z1[q] = fmaf(fg[4 * h + 3], v.w, z1[q]);
        z3[q] = fmaf(fu[4 * h + 3], v.w, z3[q]);
      }
    }
  };

  // units run across the blocks first: with fewer units than waves every CU still streams.
  // Block b owns units b + j * gridDim.x and wave w starts on j = w.  For two tokens over
  // full-size rows (more than two units per wave), each next j comes from a block counter, so a
  // wave that gets fewer issue slots (the younger waves of a SIMD) takes fewer units and the
  // block's waves finish together (277.2 -> 274.1 us per step; one token, or the 128-wide
  // TP-share intermediate, measured no gain); otherwise j steps by the block's wave count.
  // Each unit writes its own outputs, so the assignment leaves every value as it is.
  constexpr bool kCounter = NT > 1 && CPRS >= 256;
  int cur = wave * gridDim.x + blockIdx.x;
  const bool dyn = kCounter && units > 2 * stride;
  auto grab = [&]() {
    if constexpr (kCounter) {
      if (dyn) {
        int j = 0;
        if (lane == 0) j = atomicAdd(&next_unit, 1);
        return (int)blockIdx.x + __builtin_amdgcn_readfirstlane(j) * (int)gridDim.x;
      }
    }
    return cur + stride;
  };
  issue_a(cur);
  issue_b(cur);
  for (int nxt; cur < units; cur = nxt) {
    nxt = grab();
    const int a = cur / I, i = cur - a * I;
    const int p0 = __builtin_amdgcn_readlane(t_lo, min(a, 63));
    const int cnt = __builtin_amdgcn_readlane(t_cnt, min(a, 63));
    const float* xr[NT];  // this lane's first activation value of each token's row
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int tq = __builtin_amdgcn_readlane(t_tok, min(p0 + min(q, cnt - 1), 63));
      xr[q] = lds + (shared ? min(q, B - 1) : tq) * G::K + lane * G::EPC;
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) z1[q] = z3[q] = 0.f;
    // (one chunk at a time: unpacked weights of several chunks would not fit beside the
    // buffers)
#pragma unroll
    for (int j = 0; j < HA; ++j) {
      eat(ga[j], ua[j], j, xr);
      if (NT > 1) __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_a(nxt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < HB; ++j) {
      eat(gb[j], ub[j], HA + j, xr);
      if (NT > 1) __builtin_amdgcn_sched_barrier(0);
    }
    // the sums are needed here for every token slot, used or not: keeps the compiler from
    // sinking a slot's whole dot product (and the weights it holds) into its store branch
#pragma unroll
    for (int q = 0; q < NT; ++q) asm volatile("" : "+v"(z1[q]), "+v"(z3[q]));
    __builtin_amdgcn_sched_barrier(0);
    issue_b(nxt);
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const float g = seg_sum_dpp<64>(z1[q]);
      const float v = seg_sum_dpp<64>(z3[q]);
      if (q < cnt && lane == 63) A[(size_t)(p0 + q) * I + i] = silu_f32(g) * v;
    }
  }
}

// ------------------------------------------------------------------------------ combine (MFMA path)
// out[t][n] = RNE(h32[t][n] + sum_j gate[t][j] * Y[row(t*k+j)][n] + ys[t][n]), j in ascending
// expert order, row(slot) = slot when the down-projection wrote Y by slot (by_slot), else
// inv_perm[slot].  KMAX >= k; every load is issued before the sum (clamped indices, zero gates
// past k), so with Y by slot the launch costs one memory latency.
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ h32,
                                                      const float* __restrict__ Y,
                                                      const float* __restrict__ ys, Routing rt,
                                                      int H, int k, int B, bool by_slot,
                                                      T* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H) return;
  const int t = i / H, n = i - t * H;
  float g[KMAX], y[KMAX];
  const bool routed = *rt.n_act > 0;  // 0: tables failed validation, routed terms left out
  int q[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int slot = t * k + min(j, k - 1);
    q[j] = by_slot ? slot : min(max(rt.inv_perm[slot], 0), B * k - 1);
    g[j] = rt.topk_gate[slot];
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) y[j] = Y[(size_t)q[j] * H + n];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    g[j] = (j < k && routed) ? g[j] : 0.f;
    y[j] = (j < k && routed) ? y[j] : 0.f;  // unwritten rows of Y are never used
  }
  float acc = h32[i];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) acc = fmaf(g[j], y[j], acc);
  Elem<T>::store(out, i, acc + ys[i]);
}

// ------------------------------------------------------------------------------ down + combine
// Row ownership: block b owns RG row groups (RPW consecutive rows each) of the output, groups
// b, b + nb, b + 2 nb, ... (interleaved, so the blocks that work in step read neighbouring
// rows and every HBM channel stays busy).  Its work items are (a, row group) for every active
// expert a and, with ws2, the shared expert as one more group after them (its positions are
// the B tokens, its activations the rows of As).  An item's dot products W2_a[n] . A[p] for
// each position p of expert a land in LDS, and once all items are done the block writes
// out[t][n] = RNE(h32[t][n] + sum_j g[t][j] * part[pos(t,j)][n] + y_s[t][n]) (j in ascending
// expert order, then the shared expert's output y_s: its group's dots, or ys when the shared
// expert's down-projection ran elsewhere), so no expert output leaves the chip.
// Items are split into contiguous runs over the waves.  A wave alternates two register
// buffers of U items (the loads of one in flight while the other is consumed), keeps the
// activation values of the group it is on in registers, and reads the group tables from its
// own lanes (lane i: expert act[i], its first position and its position count; lane n_act:
// the shared expert).
template <typename T, int CPR, int NT, int U, int WPB, int MINB>
__global__ __launch_bounds__(64 * WPB) __attribute__((amdgpu_waves_per_eu(MINB * WPB / 4))) void down_combine_kernel(
    const float* __restrict__ A, const float* __restrict__ ys, const T* __restrict__ w2,
    const float* __restrict__ h32, int H, int k, int B, int RG, Routing rt,
    T* __restrict__ out, const T* __restrict__ ws2, const float* __restrict__ As) {
  using G = Geo<T, CPR>;
  extern __shared__ float lds[];
  const bool sh = ws2 != nullptr;
  const int nslot = B * k, npos = nslot + (sh ? B : 0), RB = RG * G::RPW;
  float* sA = lds;                               // [npos][K]: A rows, then As rows
  float* part = sA + (size_t)npos * G::K;        // [npos][RB]
  float* sG = part + (size_t)npos * RB;          // [nslot] gates
  int* sQ = (int*)(sG + nslot);                  // [nslot] slot -> position
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane % G::SEG, seg = lane / G::SEG;
  const int t_a = rt.act[lane];                  // act has E >= 64 entries (read before n_act)
  const int n_act = min(*rt.n_act, 63);          // at most B * k <= 32 on this path
  const int ng = n_act + (sh ? 1 : 0);           // groups, the shared expert last
  const int nb = gridDim.x;
  auto row_of = [&](int rg, int sg) { return ((int)blockIdx.x + nb * rg) * G::RPW + sg; };
  const int items = ng * RG;
  const int i0 = wave * items / WPB, i1 = (wave + 1) * items / WPB;

  // activation rows (up to 8 slots per token in registers; more are copied by a loop)
  Stage<stage_q(8 * NT, G::K)> sta;
  sta.load(A, nslot * G::K);
  Stage<stage_q(NT, G::K)> stb;
  if (sh) stb.load(As, B * G::K);
  // the residual (and shared-expert) values of this thread's combine item, requested now
  // (every block has at most one item per thread at these shapes; otherwise the tail loads
  // them)
  const bool pre = B * RB <= (int)blockDim.x;
  float pre_h, pre_y = 0.f;
  {
    const int i = min((int)threadIdx.x, B * RB - 1);
    const int t = i / RB, nl = i - t * RB;
    const size_t o = (size_t)t * H + min(row_of(nl / G::RPW, nl % G::RPW), H - 1);
    pre_h = h32[o];
    if (!sh) pre_y = ys[o];
  }
  const int t_e = lane < n_act ? t_a : 0;  // entries past n_act are not expert ids
  const int t_lo = lane < n_act ? rt.offsets[t_e] : (lane == n_act ? nslot : 0);
  const int t_cnt = lane < n_act ? rt.offsets[t_e + 1] - t_lo : (lane == n_act ? B : 0);

  // Two register buffers of U items.  Loads are never branched around: an item past the
  // run's end reads the first row of A instead (L2-resident), so the waits stay exact.
  u32x4 w0[U][G::CPL], w1[U][G::CPL];
  const T* dummy = reinterpret_cast<const T*>(A);
  struct Cursor { int it, a, rg; };
  auto advance = [&](Cursor& c) {
    ++c.it;
    if (++c.rg == RG) { c.rg = 0; ++c.a; }
  };
  Cursor ci{i0, i0 / RG, i0 - (i0 / RG) * RG}, cc = ci;
  auto issue = [&](u32x4 (&w)[U][G::CPL]) {
#pragma unroll
    for (int q = 0; q < U; ++q) {
      const int e = __builtin_amdgcn_readlane(t_e, min(ci.a, 63));
      const int n = min(row_of(ci.rg, seg), H - 1);
      const T* row = (sh && ci.a == n_act) ? ws2 + (size_t)n * G::K : w2 + ((size_t)e * H + n) * G::K;
      load_row<T, CPR>(ci.it < i1 ? row : dummy, sub, w[q]);
      advance(ci);
    }
  };
  // The lane's activation values for the positions of the group being consumed, held in
  // registers while the run stays on that group (reloaded from LDS when it moves on).
  float xa[NT][G::CPL][G::EPC];
  int a_cur = -1;
  auto consume = [&](const u32x4 (&w)[U][G::CPL]) {
#pragma unroll
    for (int q = 0; q < U; ++q) {
      if (cc.it < i1) {
        const int a = cc.a;
        const int r0 = __builtin_amdgcn_readlane(t_lo, min(a, 63));
        const int cnt = __builtin_amdgcn_readlane(t_cnt, min(a, 63));
        if (a != a_cur) {
          a_cur = a;
#pragma unroll
          for (int qq = 0; qq < NT; ++qq) {
            const float* row = sA + (size_t)(r0 + min(qq, cnt - 1)) * G::K;
#pragma unroll
            for (int i = 0; i < G::CPL; ++i) {
              const int c = min(sub + G::SEG * i, CPR - 1);
#pragma unroll
              for (int h = 0; h < G::EPC / 4; ++h) {
                const float4 v = reinterpret_cast<const float4*>(row + c * G::EPC)[h];
                xa[qq][i][4 * h + 0] = v.x;
                xa[qq][i][4 * h + 1] = v.y;
                xa[qq][i][4 * h + 2] = v.z;
                xa[qq][i][4 * h + 3] = v.w;
              }
            }
          }
        }
        const int nl = cc.rg * G::RPW + seg;
        const bool live = row_of(cc.rg, seg) < H;
        float acc[NT];
#pragma unroll
        for (int qq = 0; qq < NT; ++qq) acc[qq] = 0.f;
#pragma unroll
        for (int i = 0; i < G::CPL; ++i) {
          if (G::EXACT || sub + G::SEG * i < CPR) {
            float f[G::EPC];
            Elem<T>::unpack(w[q][i], f);
#pragma unroll
            for (int qq = 0; qq < NT; ++qq)
#pragma unroll
              for (int x = 0; x < G::EPC; ++x) acc[qq] = fmaf(f[x], xa[qq][i][x], acc[qq]);
          }
        }
        // (needed for every slot, used or not: keeps a slot's dot product out of its branch)
#pragma unroll
        for (int qq = 0; qq < NT; ++qq) asm volatile("" : "+v"(acc[qq]));
#pragma unroll
        for (int qq = 0; qq < NT; ++qq) {
          const float v = seg_sum_dpp<G::SEG>(acc[qq]);
          if (qq < cnt && sub == G::SEG - 1 && live) part[(r0 + qq) * RB + nl] = v;
        }
      }
      advance(cc);
    }
  };
  issue(w0);
  issue(w1);
  sta.store(sA);
  if (sh) stb.store(sA + (size_t)nslot * G::K);
  // (n_act == 0 marks tables that failed validation: the routed terms are then left out, and
  // positions are clamped so that no index leaves the block's arrays)
  for (int i = threadIdx.x; i < nslot; i += blockDim.x) {
    sG[i] = n_act > 0 ? rt.topk_gate[i] : 0.f;
    sQ[i] = min(max(rt.inv_perm[i], 0), nslot - 1);
  }
  __syncthreads();
  for (int base = i0; base < i1; base += 2 * U) {
    consume(w0);
    __builtin_amdgcn_sched_barrier(0);
    issue(w0);
    __builtin_amdgcn_sched_barrier(0);
    consume(w1);
    __builtin_amdgcn_sched_barrier(0);
    issue(w1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B * RB; i += blockDim.x) {
    const int t = i / RB, nl = i - t * RB;
    const int n = row_of(nl / G::RPW, nl % G::RPW);
    if (n < H) {
      float acc = pre ? pre_h : h32[(size_t)t * H + n];
      if (n_act > 0)
        for (int j = 0; j < k; ++j) acc = fmaf(sG[t * k + j], part[sQ[t * k + j] * RB + nl], acc);
      const float y = sh ? part[(nslot + t) * RB + nl] : (pre ? pre_y : ys[(size_t)t * H + n]);
      Elem<T>::store(out, (size_t)t * H + n, acc + y);
    }
  }
}

// ------------------------------------------------------------------------------ prep
// act / n_act / inv_perm (and the pieces of at most 16 positions) from expert_offsets + perm
// supplied by the caller, after checking that they are a routing of nslots = B * k slots as
// kk_router_topk writes one: offsets non-decreasing from 0 to nslots with at most B positions
// per expert; perm a permutation of the slots; within each expert the slots in ascending
// token order (so no token twice); and topk_idx of every slot naming the expert whose range
// holds it.  Invalid tables set n_act = 0 and no pieces, so no kernel indexes through them,
// and write the reasons (kRouting* bits) to rt.status; valid ones write status 0.
// One wave (64 threads).
__global__ __launch_bounds__(64) void moe_prep_kernel(int E, int k, int nslots, int B, Routing rt) {
  __shared__ uint32_t seen[kMaxSlots / 32];
  const int lane = threadIdx.x;
  const int per = (E + 63) / 64;
  for (int i = lane; i < kMaxSlots / 32; i += 64) seen[i] = 0u;
  __syncthreads();
  int bad = 0;
  int lf = 0;
  for (int q = 0; q < per; ++q) {
    const int e = lane * per + q;
    if (e < E) {
      const int a = rt.offsets[e], b = rt.offsets[e + 1];
      if (!(a >= 0 && b >= a && b <= nslots && b - a <= B)) bad |= kRoutingOffsets;
      if (b > a) ++lf;
    }
  }
  if (lane == 0 && (rt.offsets[0] != 0 || rt.offsets[E] != nslots)) bad |= kRoutingOffsets;
  for (int p = lane; p < nslots; p += 64) {
    const int v = rt.perm[p];
    if (v < 0 || v >= nslots) {
      bad |= kRoutingPermRange;
    } else {
      const uint32_t bit = 1u << (v & 31);
      if (atomicOr(&seen[v >> 5], bit) & bit) bad |= kRoutingPermDup;
    }
  }
  // each expert's slots: ascending tokens, topk_idx naming that expert (only over ranges the
  // offsets check has passed, so every position read is in 0..nslots-1)
  if (!(bad & kRoutingOffsets)) {
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      if (e < E) {
        int prev = -1;
        for (int p = rt.offsets[e]; p < rt.offsets[e + 1]; ++p) {
          const int v = rt.perm[p];
          if (v < 0 || v >= nslots) continue;  // reported above
          const int t = v / k;
          if (t <= prev) bad |= kRoutingOrder;
          prev = t;
          if (rt.topk_idx[v] != e) bad |= kRoutingIdx;
        }
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) bad |= __shfl_xor(bad, off, 64);
  const bool all_ok = bad == 0;
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
  if (lane == 0 && rt.status) *rt.status = bad;
  if (rt.vg) {
    // pieces of at most 16 positions per active expert, in expert order (none if invalid)
    int vt = 0;
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      if (all_ok && e < E) vt += (rt.offsets[e + 1] - rt.offsets[e] + 15) >> 4;
    }
    int vinc = vt;
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(vinc, off, 64);
      if (lane >= off) vinc += v;
    }
    int vpos = vinc - vt, a = inc - lf;
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      if (all_ok && e < E) {
        const int c = rt.offsets[e + 1] - rt.offsets[e];
        for (int pc = 0; pc < (c + 15) >> 4; ++pc) rt.vg[vpos++] = (a << 2) | pc;
        if (c > 0) ++a;
      }
    }
    if (lane == 63) *rt.n_vg = vinc;
  }
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

template <typename T, int CPR, int CPS, int R>
hipError_t oproj_router_t(const Shape& s, const Device& d, int B, const void* x, const void* r,
                          const void* w_o, const void* w_r, const void* mr, float* h32,
                          void* h_out, float* part, hipStream_t st) {
  using G = Geo<T, CPR>;
  constexpr int R2 = (R > 1 && G::CPL > 4) ? R / 2 : R;
  const int npl = router_oproj_planes(s);
  const int RS = s.H / Geo<T, CPS>::K;
  if (RS * Geo<T, CPS>::K != s.H || RS + npl > kMaxTopkSplits) return hipErrorInvalidValue;
  const int rows_per_unit = G::RPW * (B == 1 ? R : R2);
  const int units = (s.H + npl * s.E + rows_per_unit - 1) / rows_per_unit;
  const LaunchShape ls = balanced(d, units);
  if ((long)ls.blocks * (ls.threads / 64) < (long)s.E * RS) return hipErrorInvalidValue;
  auto kern = B == 1 ? oproj_router_gemv_kernel<T, CPR, CPS, 1, R>
                     : oproj_router_gemv_kernel<T, CPR, CPS, 2, R2>;
  const bool regs = (B == 1 ? 1 : 2) * G::CPL <= 14;
  const size_t lds = ((size_t)B * s.H + (regs ? 0 : (size_t)B * G::K)) * sizeof(float);
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3(ls.blocks), dim3(ls.threads), lds, st, (const T*)x, (const T*)r,
                     (const T*)w_o, (const T*)w_r, (const T*)mr, npl, h32, (T*)h_out, part, s.H,
                     s.E, RS);
  return hipGetLastError();
}

template <typename T, int CPS, int CPRH>
hipError_t router_logits_t(const Shape& s, const Device& d, int B, const float* h32,
                           const void* w_r, float* part, const void* ws13, const Routing& rt,
                           float* As, const Norm& nm, hipStream_t st) {
  const int splits = s.H / Geo<T, CPS>::K;
  const int nw = d.num_cu * (kGemvThreads / 64);
  if (s.E * splits > 2 * nw) return hipErrorInvalidValue;
  const size_t lds = (size_t)B * s.H * sizeof(float);
  auto kern = B == 1 ? router_logits_kernel<T, CPS, CPRH, 1> : router_logits_kernel<T, CPS, CPRH, 2>;
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3(d.num_cu), dim3(kGemvThreads), lds, st, h32, (const T*)w_r, s.H,
                     s.E, B, splits, part, (const T*)ws13, s.Is, s.k, rt, As,
                     (const T*)nm.gamma, nm.eps);
  return hipGetLastError();
}

template <typename T, int CPR, int CPRS>
hipError_t gateup_t(const Shape& s, const Device& d, int B, const float* u, const void* w13,
                    bool shared, const Routing& rt, float* A, const GateupExtras& x,
                    hipStream_t st) {
  if (x.part && (x.splits > kMaxTopkSplits || shared)) return hipErrorInvalidValue;
  if (x.ws13 && (shared || x.ws2 || s.Is != s.I || !x.As_out)) return hipErrorInvalidValue;
  const size_t lds = (size_t)B * Geo<T, CPR>::K * sizeof(float);
  auto pick = [&](auto k1, auto k2) { return B == 1 ? k1 : k2; };
  if (x.ws13 && !x.part) return hipErrorInvalidValue;  // the shared gate/up covers a top-k
  // (the shared gate/up prologue serves the fused-router plan, bf16 layers only)
  constexpr bool kSgu = std::is_same<T, uint16_t>::value;
  if (x.ws13 && !kSgu) return hipErrorInvalidValue;
  auto kern = x.ws13 ? pick(gateup_gemv_kernel<T, CPR, CPRS, 1, true, kSgu>,
                            gateup_gemv_kernel<T, CPR, CPRS, 2, true, kSgu>)
              : x.part ? pick(gateup_gemv_kernel<T, CPR, CPRS, 1, true, false>,
                              gateup_gemv_kernel<T, CPR, CPRS, 2, true, false>)
                       : pick(gateup_gemv_kernel<T, CPR, CPRS, 1, false, false>,
                              gateup_gemv_kernel<T, CPR, CPRS, 2, false, false>);
  allow_lds(kern, lds);
  const int inter = shared ? s.Is : s.I;
  hipLaunchKernelGGL(kern, dim3(d.num_cu), dim3(kGemvThreads), lds, st, u, (const T*)w13, inter,
                     s.k, B, shared ? 1 : 0, rt, A, x.part, x.splits, x.bias, s.E, s.routed_scale,
                     (const T*)x.ws2, x.As, x.ys, s.H, (const T*)x.norm.gamma, x.norm.eps,
                     (const T*)x.ws13, s.Is, x.As_out);
  return hipGetLastError();
}

template <typename T, int CPR>
size_t down_combine_lds(const Shape& s, int B, int RG, bool sh) {
  using G = Geo<T, CPR>;
  const int nslot = B * s.k, npos = nslot + (sh ? B : 0);
  return ((size_t)npos * G::K + (size_t)npos * RG * G::RPW + 2 * (size_t)nslot) * 4;
}

// Row groups per block: two blocks of 8 waves per CU when their LDS fits and the kernel
// fits in 128 VGPRs (not so for two tokens' activations over 4 KB rows), else one.  Short rows
// (one chunk per lane: a 128-wide intermediate) also take one block per CU: their waves'
// longer runs measured faster (TP share down-projection, batch 1: 11.9 -> 11.1 us, batch 2:
// 16.0 -> 14.5; 4 KB rows at batch 1 the other way, 41.2 -> 43.2).
template <typename T, int CPR>
int down_groups_per_block(const Shape& s, const Device& d, int B, bool sh, int* per_cu) {
  const int groups = (s.H + Geo<T, CPR>::RPW - 1) / Geo<T, CPR>::RPW;
  const int rg2 = (groups + 2 * d.num_cu - 1) / (2 * d.num_cu);
  const bool two = 2 * down_combine_lds<T, CPR>(s, B, rg2, sh) <= (size_t)d.max_lds &&
                   !(B == 2 && Geo<T, CPR>::CPL >= 4) && !(B <= 2 && Geo<T, CPR>::CPL == 1);
  if (per_cu) *per_cu = two ? 2 : 1;
  return two ? rg2 : (groups + d.num_cu - 1) / d.num_cu;
}

template <typename T, int CPR, int U>
hipError_t down_combine_t(const Shape& s, const Device& d, int B, const float* A, const float* ys,
                          const void* w2, const float* h32, const Routing& rt, void* out,
                          const void* ws2, const float* As, hipStream_t st) {
  using G = Geo<T, CPR>;
  const bool sh = ws2 != nullptr;
  if (sh && (!As || s.Is != s.I)) return hipErrorInvalidValue;
  int per_cu = 1;
  const int RG = down_groups_per_block<T, CPR>(s, d, B, sh, &per_cu);
  const int groups = (s.H + G::RPW - 1) / G::RPW;
  const size_t lds = down_combine_lds<T, CPR>(s, B, RG, sh);
  constexpr int NT2_PER_CU = Geo<T, CPR>::CPL >= 4 ? 1 : 2;
  auto kern = per_cu == 2 ? (B == 1 ? down_combine_kernel<T, CPR, 1, U, 8, 2>
                                    : down_combine_kernel<T, CPR, 2, U, 8, NT2_PER_CU>)
                          : (B == 1 ? down_combine_kernel<T, CPR, 1, U, 8, 1>
                                    : down_combine_kernel<T, CPR, 2, U, 8, 1>);
  allow_lds(kern, lds);
  hipLaunchKernelGGL(kern, dim3((groups + RG - 1) / RG), dim3(kGemvThreads), lds, st, A, ys,
                     (const T*)w2, h32, s.H, s.k, B, RG, rt, (T*)out, (const T*)ws2, As);
  return hipGetLastError();
}

template <typename T>
hipError_t combine_t(const Shape& s, int B, const float* h32, const float* Y, const float* ys,
                     const Routing& rt, void* out, hipStream_t st) {
  const int n = B * s.H;
  auto kern = s.k <= 8 ? combine_kernel<T, 8> : combine_kernel<T, 16>;
  hipLaunchKernelGGL(kern, dim3((n + 255) / 256), dim3(256), 0, st, h32, Y, ys, rt, s.H, s.k, B,
                     mfma_y_by_slot(B), (T*)out);
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
    if (c == 896) return oproj_t<uint16_t, 896, 1>(s, d, B, x, r, w_o, h32, h_out, st);
    if (c == 56) return oproj_t<uint16_t, 56, 4>(s, d, B, x, r, w_o, h32, h_out, st);
  } else if (c == 64) {
    return oproj_t<float, 64, 2>(s, d, B, x, r, w_o, h32, h_out, st);
  }
  return hipErrorInvalidValue;
}

bool router_fused_applies(const Shape& s) {
  return s.dtype == 1 && s.H == 7168 && (s.Ko == 448 || s.Ko == 7168) && gemv_supported(s, 1);
}

int router_oproj_planes(const Shape& s) { return s.dtype == 1 ? 2 : 1; }

int router_fused_splits(const Shape& s) { return 2 + router_oproj_planes(s); }

size_t router_oproj_product_bytes(const Shape& s) {
  return (size_t)s.E * router_oproj_planes(s) * s.Ko * (s.dtype == 1 ? 2 : 4);
}

hipError_t launch_router_oproj_product(const Shape& s, const void* w_r, const void* w_o, void* mr,
                                       hipStream_t st) {
  if (!router_fused_applies(s)) return hipErrorInvalidValue;
  const dim3 grid((s.Ko + 63) / 64, (s.E + 31) / 32);
  hipLaunchKernelGGL(router_oproj_product_kernel<uint16_t>, grid, dim3(256), 0, st,
                     (const uint16_t*)w_r, (const uint16_t*)w_o, s.E, s.H, s.Ko, (uint16_t*)mr,
                     router_oproj_planes(s));
  return hipGetLastError();
}

hipError_t launch_oproj_router_gemv(const Shape& s, const Device& d, int B, const void* x,
                                    const void* r, const void* w_o, const void* w_r, const void* mr,
                                    float* h32, void* h_out, float* part, hipStream_t st) {
  const int c = cpr_of(s.Ko, s.dtype);
  if (!router_fused_applies(s)) return hipErrorInvalidValue;
  // router slices of 3584 against r; 448-wide input slice: 4 rows of W_o or M per wave, a full
  // 7168-wide input: one row per wave, x in registers (one token) or LDS (two)
  if (c == 56) return oproj_router_t<uint16_t, 56, 448, 4>(s, d, B, x, r, w_o, w_r, mr, h32, h_out, part, st);
  if (c == 896) return oproj_router_t<uint16_t, 896, 448, 1>(s, d, B, x, r, w_o, w_r, mr, h32, h_out, part, st);
  return hipErrorInvalidValue;
}

hipError_t launch_router_logits(const Shape& s, const Device& d, int B, const float* h32,
                                const void* w_r, float* part, const void* ws13, const Routing& rt,
                                float* As, const Norm& nm, hipStream_t st) {
  if (s.dtype == 1 && s.H == 7168)
    return router_logits_t<uint16_t, 128, 896>(s, d, B, h32, w_r, part, ws13, rt, As, nm, st);
  if (s.dtype == 0 && s.H == 256)
    return router_logits_t<float, 64, 64>(s, d, B, h32, w_r, part, ws13, rt, As, nm, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gateup_gemv(const Shape& s, const Device& d, int B, const float* u,
                              const void* w13, bool shared, const Routing& rt, float* A,
                              const GateupExtras& x, hipStream_t st) {
  const int c = cpr_of(s.H, s.dtype), cs = cpr_of(s.Is, s.dtype);
  if (s.dtype == 1 && c == 896 && cs == 256)
    return gateup_t<uint16_t, 896, 256>(s, d, B, u, w13, shared, rt, A, x, st);
  if (s.dtype == 1 && c == 896 && cs == 16)
    return gateup_t<uint16_t, 896, 16>(s, d, B, u, w13, shared, rt, A, x, st);
  if (s.dtype == 0 && c == 64 && cs == 32)
    return gateup_t<float, 64, 32>(s, d, B, u, w13, shared, rt, A, x, st);
  return hipErrorInvalidValue;
}

size_t down_combine_gemv_lds(const Shape& s, const Device& d, int B, bool shared_down) {
  const int c = cpr_of(s.I, s.dtype);
  const bool sh = shared_down;
  if (s.dtype == 1 && c == 256)
    return down_combine_lds<uint16_t, 256>(s, B, down_groups_per_block<uint16_t, 256>(s, d, B, sh, nullptr), sh);
  if (s.dtype == 1 && c == 16)
    return down_combine_lds<uint16_t, 16>(s, B, down_groups_per_block<uint16_t, 16>(s, d, B, sh, nullptr), sh);
  return down_combine_lds<float, 32>(s, B, down_groups_per_block<float, 32>(s, d, B, sh, nullptr), sh);
}

hipError_t launch_down_combine_gemv(const Shape& s, const Device& d, int B, const float* A,
                                    const float* ys, const void* w2, const float* h32,
                                    const Routing& rt, void* out, const void* ws2,
                                    const float* As, hipStream_t st) {
  const int c = cpr_of(s.I, s.dtype);
  if (s.dtype == 1) {
    if (c == 256) return down_combine_t<uint16_t, 256, 1>(s, d, B, A, ys, w2, h32, rt, out, ws2, As, st);
    // (128-wide rows: two 4-row items per buffer; with four the TP share's batch-1 and batch-2
    // steps took 1.2 and 0.9 us longer: each wave's first wait covered more loads)
    if (c == 16) return down_combine_t<uint16_t, 16, 2>(s, d, B, A, ys, w2, h32, rt, out, ws2, As, st);
  } else if (c == 32) {
    return down_combine_t<float, 32, 2>(s, d, B, A, ys, w2, h32, rt, out, ws2, As, st);
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

hipError_t launch_topk_tables(const Shape& s, int B, const float* part, int splits,
                              const float* bias, const Routing& rt, hipStream_t st) {
  if (B > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_tables_kernel, dim3(1), dim3(64 * B), 0, st, part, splits, bias, s.E,
                     s.k, B, s.routed_scale, rt);
  return hipGetLastError();
}

hipError_t launch_tables(const Shape& s, int B, const Routing& rt, hipStream_t st) {
  hipLaunchKernelGGL(tables_kernel, dim3(1), dim3(256), 0, st, s.E, s.k, B, rt);
  return hipGetLastError();
}

hipError_t launch_prefetch(const Device& d, const void* p, size_t bytes, hipStream_t st) {
  if (bytes % 16) return hipErrorInvalidValue;
  if (!bytes) return hipSuccess;
  hipLaunchKernelGGL(prefetch_kernel, dim3(d.num_cu), dim3(256), 0, st, (const u32x4*)p,
                     bytes / 16);
  return hipGetLastError();
}

hipError_t launch_delay(long long ticks, hipStream_t st) {
  if (ticks <= 0) return hipSuccess;
  hipLaunchKernelGGL(delay_kernel, dim3(1), dim3(64), 0, st, ticks);
  return hipGetLastError();
}

hipError_t launch_moe_prep(const Shape& s, int B, const Routing& rt, hipStream_t st) {
  if (B * s.k > kMaxSlots) return hipErrorInvalidValue;
  hipLaunchKernelGGL(moe_prep_kernel, dim3(1), dim3(64), 0, st, s.E, s.k, B * s.k, B, rt);
  return hipGetLastError();
}

}  // namespace kk

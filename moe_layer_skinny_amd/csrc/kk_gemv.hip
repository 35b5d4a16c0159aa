// GEMV path of the decode-layer step (batch 1-2): every weight row is streamed from HBM
// once with 128-bit non-temporal loads; activations sit in LDS as fp32; each row's dot
// product is finished with a wavefront shuffle reduction.
//
// "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly", section "Recovering
// time between operators": small-matrix projection kernels at batch 1-2, o-proj fused with
// the residual, router scores, selected experts, shared expert on another stream.
#include "kk_common.cuh"
#include "kk_internal.h"
#include "kk_topk.cuh"

namespace kk {
namespace {

constexpr int kGemvThreads = 512;  // 8 waves; one persistent block per CU
constexpr int kGemvWaves = kGemvThreads / kWave;

// Copy n floats (or bf16 -> fp32) from global to LDS with the whole block.
template <typename T>
__device__ __forceinline__ void stage_f32(float* dst, const T* __restrict__ src, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) dst[i] = Elem<T>::load(src, i);
}

// ------------------------------------------------------------------------------ o-proj
// h32[t][n] = r[t][n] + sum_k W_o[n][k] x[t][k]; optional h_out = RNE(h32).
template <typename T, int CPR, int NT, int R>
__global__ __launch_bounds__(kGemvThreads) void oproj_gemv_kernel(
    const T* __restrict__ x, const T* __restrict__ r, const T* __restrict__ w_o,
    float* __restrict__ h32, T* __restrict__ h_out, int H, int B) {
  using G = Geo<T, CPR>;
  extern __shared__ float lds[];  // x as fp32 [B][Ko]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % G::SEG, seg = lane / G::SEG;
  const int rows_per_unit = G::RPW * R;
  const int units = (H + rows_per_unit - 1) / rows_per_unit;
  const int stride = gridDim.x * kGemvWaves;
  int unit = blockIdx.x * kGemvWaves + wave;

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
  stage_f32<T>(lds, x, B * G::K);
  __syncthreads();

  for (; unit < units; unit += stride) {
    issue(unit);
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const int n = unit * rows_per_unit + seg + G::RPW * q;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t < B) {
          float acc = seg_sum<G::SEG>(dot_lane<T, CPR>(w[q], lds + t * G::K, sub));
          if (sub == 0 && n < H) {
            const size_t o = (size_t)t * H + n;
            const float hv = Elem<T>::load(r, o) + acc;
            h32[o] = hv;
            if (h_out) Elem<T>::store(h_out, o, hv);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------ router
// Logit partials over `splits` K-slices, then the last block to finish runs top-k, gates
// and the routing tables.  Each wave takes one (expert, slice) unit; h32 is read from L2.
template <typename T, int CPS, int NT>
__global__ __launch_bounds__(256) void router_gemv_kernel(
    const float* __restrict__ h32, const T* __restrict__ w_r, const float* __restrict__ bias,
    int H, int E, int k, int B, int splits, float routed_scale, float* __restrict__ part,
    unsigned* __restrict__ counter, Routing rt) {
  using G = Geo<T, CPS>;
  __shared__ TopkScratch sm;
  __shared__ int s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wpb = blockDim.x >> 6;
  const int units = E * splits;
  for (int unit = blockIdx.x * wpb + wave; unit < units; unit += gridDim.x * wpb) {
    const int e = unit / splits, s = unit - e * splits;
    u32x4 w[G::CPL];
    load_row<T, CPS>(w_r + (size_t)e * H + (size_t)s * G::K, lane, w);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < B) {
        const float acc =
            seg_sum<64>(dot_lane<T, CPS>(w, h32 + (size_t)t * H + (size_t)s * G::K, lane));
        if (lane == 0) part[((size_t)s * B + t) * E + e] = acc;
      }
    }
  }
  // Publish the partials, then elect the last block (device-scope release/acquire).
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1u) == gridDim.x - 1) ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  topk_tables(part, splits, bias, B, E, k, routed_scale, rt, sm);
  if (threadIdx.x == 0) atomicExch(counter, 0u);  // ready for the next launch
}

// ------------------------------------------------------------------------------ gate / up
// A[p][i] = silu(W1_e[i] . u_t) * (W3_e[i] . u_t) for every position p of expert e (token
// t = perm[p] / k), or for the shared expert (positions = tokens 0..B-1).
template <typename T, int CPR, int NT>
__global__ __launch_bounds__(kGemvThreads) void gateup_gemv_kernel(
    const float* __restrict__ u, const T* __restrict__ w13, int I, int k, int B, int shared,
    Routing rt, float* __restrict__ A) {
  using G = Geo<T, CPR>;
  static_assert(G::SEG == 64, "gate/up rows must span the wave");
  extern __shared__ float lds[];  // u [B][H]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = shared ? 1 : *rt.n_act;
  const int units = n * I;
  const int stride = gridDim.x * kGemvWaves;
  int unit = blockIdx.x * kGemvWaves + wave;

  u32x4 wg[G::CPL], wu[G::CPL];
  auto issue = [&](int un) {
    const int a = un / I, i = un - a * I;
    const int e = shared ? 0 : rt.act[a];
    const T* g_row = w13 + ((size_t)e * 2 * I + i) * G::K;
    load_row<T, CPR>(g_row, lane, wg);
    load_row<T, CPR>(g_row + (size_t)I * G::K, lane, wu);
  };
  for (int i = threadIdx.x; i < B * G::K / 4; i += blockDim.x)
    reinterpret_cast<float4*>(lds)[i] = reinterpret_cast<const float4*>(u)[i];
  __syncthreads();

  for (; unit < units; unit += stride) {
    issue(unit);
    const int a = unit / I, i = unit - a * I;
    int p0 = 0, p1 = B;
    if (!shared) {
      const int e = rt.act[a];
      p0 = rt.offsets[e];
      p1 = rt.offsets[e + 1];
    }
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int p = p0 + q;
      if (p < p1) {
        const int t = shared ? p : rt.perm[p] / k;
        const float* ut = lds + t * G::K;
        float z1, z3;
        dot2_lane<T, CPR>(wg, wu, ut, lane, z1, z3);
        z1 = seg_sum<64>(z1);
        z3 = seg_sum<64>(z3);
        if (lane == 0) A[(size_t)p * I + i] = silu_f32(z1) * z3;
      }
    }
  }
}

// ------------------------------------------------------------------------------ down + combine
// out[t][n] = RNE(h32[t][n] + sum_{e active} sum_{p of e, token t} g_p (W2_e[n] . A[p])
//                 + Ws2[n] . As[t]).  Each routed W2 row is read once for all its tokens.
// Lane partials are accumulated over experts (ascending) then the shared expert, and
// reduced across the row's lanes once per token.
template <typename T, int CPR, int NT, int EB>
__global__ __launch_bounds__(kGemvThreads) void down_combine_gemv_kernel(
    const float* __restrict__ A, const float* __restrict__ As, const T* __restrict__ w2,
    const T* __restrict__ ws2, int H, int k, int B, Routing rt, const float* __restrict__ h32,
    T* __restrict__ out) {
  using G = Geo<T, CPR>;
  extern __shared__ float lds[];  // A [B*k][I], As [B][I]
  float* sA = lds;
  float* sAs = lds + (size_t)B * k * G::K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % G::SEG, seg = lane / G::SEG;
  for (int i = threadIdx.x; i < B * k * G::K / 4; i += blockDim.x)
    reinterpret_cast<float4*>(sA)[i] = reinterpret_cast<const float4*>(A)[i];
  for (int i = threadIdx.x; i < B * G::K / 4; i += blockDim.x)
    reinterpret_cast<float4*>(sAs)[i] = reinterpret_cast<const float4*>(As)[i];
  __syncthreads();
  const int n_act = *rt.n_act;
  const int stride = gridDim.x * kGemvWaves * G::RPW;

  for (int base = (blockIdx.x * kGemvWaves + wave) * G::RPW; base < H; base += stride) {
    const int row = base + seg;
    const bool rv = row < H;
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;

    for (int a0 = 0; a0 < n_act; a0 += EB) {
      u32x4 w[EB][G::CPL];
      int eid[EB];
#pragma unroll
      for (int q = 0; q < EB; ++q) {
        const int a = a0 + q;
        eid[q] = a < n_act ? rt.act[a] : -1;
        if (eid[q] >= 0 && rv)
          load_row<T, CPR>(w2 + ((size_t)eid[q] * H + row) * G::K, sub, w[q]);
        else
#pragma unroll
          for (int i = 0; i < G::CPL; ++i) w[q][i] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < EB; ++q) {
        if (eid[q] < 0) continue;
        const int p0 = rt.offsets[eid[q]], p1 = rt.offsets[eid[q] + 1];
#pragma unroll
        for (int qq = 0; qq < NT; ++qq) {
          const int p = p0 + qq;
          if (p < p1) {
            const int slot = rt.perm[p];
            const int t = slot / k;
            const float g = rt.topk_gate[slot];
            const float d = dot_lane<T, CPR>(w[q], sA + (size_t)p * G::K, sub);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
              if (tt == t) acc[tt] = fmaf(g, d, acc[tt]);
          }
        }
      }
    }
    u32x4 ws[G::CPL];
    if (rv)
      load_row<T, CPR>(ws2 + (size_t)row * G::K, sub, ws);
    else
#pragma unroll
      for (int i = 0; i < G::CPL; ++i) ws[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < B) {
        const float v = seg_sum<G::SEG>(acc[t] + dot_lane<T, CPR>(ws, sAs + t * G::K, sub));
        if (sub == 0 && rv) {
          const size_t o = (size_t)t * H + row;
          Elem<T>::store(out, o, h32[o] + v);
        }
      }
    }
  }
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

template <typename T, int CPR, int R>
hipError_t oproj_t(const Shape& s, const Device& d, int B, const void* x, const void* r,
                   const void* w, float* h32, void* h_out, hipStream_t st) {
  const size_t lds = (size_t)B * Geo<T, CPR>::K * sizeof(float);
  auto kern = B == 1 ? oproj_gemv_kernel<T, CPR, 1, R> : oproj_gemv_kernel<T, CPR, 2, R>;
  allow_lds(kern, lds);
  const int rows_per_unit = Geo<T, CPR>::RPW * R;
  const int units = (s.H + rows_per_unit - 1) / rows_per_unit;
  int grid = d.num_cu;
  if (grid * kGemvWaves > units) grid = (units + kGemvWaves - 1) / kGemvWaves;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemvThreads), lds, st, (const T*)x, (const T*)r,
                     (const T*)w, h32, (T*)h_out, s.H, B);
  return hipGetLastError();
}

template <typename T, int CPS>
hipError_t router_t(const Shape& s, const Device& d, int B, const float* h32, const void* w_r,
                    const float* bias, float* part, unsigned* counter, const Routing& rt,
                    hipStream_t st) {
  const int splits = s.H / Geo<T, CPS>::K;
  const int units = s.E * splits;
  const int grid = (units + 3) / 4;
  auto kern = B == 1 ? router_gemv_kernel<T, CPS, 1> : router_gemv_kernel<T, CPS, 2>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, st, h32,
                     (const T*)w_r, bias, s.H, s.E, s.k, B, splits, s.routed_scale, part, counter,
                     rt);
  return hipGetLastError();
}

template <typename T, int CPR>
hipError_t gateup_t(const Shape& s, const Device& d, int B, const float* u, const void* w13,
                    bool shared, const Routing& rt, float* A, hipStream_t st) {
  const size_t lds = (size_t)B * Geo<T, CPR>::K * sizeof(float);
  auto kern = B == 1 ? gateup_gemv_kernel<T, CPR, 1> : gateup_gemv_kernel<T, CPR, 2>;
  allow_lds(kern, lds);
  const int inter = shared ? s.Is : s.I;
  const int max_act = shared ? 1 : (s.E < B * s.k ? s.E : B * s.k);
  const int units = max_act * inter;
  int grid = d.num_cu;
  if (grid * kGemvWaves > units) grid = (units + kGemvWaves - 1) / kGemvWaves;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemvThreads), lds, st, u, (const T*)w13, inter, s.k,
                     B, shared ? 1 : 0, rt, A);
  return hipGetLastError();
}

template <typename T, int CPR>
hipError_t down_t(const Shape& s, const Device& d, int B, const float* A, const float* As,
                  const void* w2, const void* ws2, const Routing& rt, const float* h32, void* out,
                  hipStream_t st) {
  using G = Geo<T, CPR>;
  const size_t lds = (size_t)(B * s.k + B) * G::K * sizeof(float);
  auto kern = B == 1 ? down_combine_gemv_kernel<T, CPR, 1, 4> : down_combine_gemv_kernel<T, CPR, 2, 4>;
  allow_lds(kern, lds);
  const int units = (s.H + G::RPW - 1) / G::RPW;
  int grid = d.num_cu;
  if (grid * kGemvWaves > units) grid = (units + kGemvWaves - 1) / kGemvWaves;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemvThreads), lds, st, A, As, (const T*)w2,
                     (const T*)ws2, s.H, s.k, B, rt, h32, (T*)out);
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

hipError_t launch_router_gemv(const Shape& s, const Device& d, int B, const float* h32,
                              const void* w_r, const float* bias, float* part, unsigned* counter,
                              const Routing& rt, hipStream_t st) {
  if (s.dtype == 1 && s.H == 7168)
    return router_t<uint16_t, 128>(s, d, B, h32, w_r, bias, part, counter, rt, st);
  if (s.dtype == 0 && s.H == 256)
    return router_t<float, 64>(s, d, B, h32, w_r, bias, part, counter, rt, st);
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

hipError_t launch_down_combine_gemv(const Shape& s, const Device& d, int B, const float* A,
                                    const float* As, const void* w2, const void* ws2,
                                    const Routing& rt, const float* h32, void* out,
                                    hipStream_t st) {
  const int c = cpr_of(s.I, s.dtype);
  if (s.dtype == 1) {
    if (c == 256) return down_t<uint16_t, 256>(s, d, B, A, As, w2, ws2, rt, h32, out, st);
    if (c == 16) return down_t<uint16_t, 16>(s, d, B, A, As, w2, ws2, rt, h32, out, st);
  } else if (c == 32) {
    return down_t<float, 32>(s, d, B, A, As, w2, ws2, rt, h32, out, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_moe_prep(const Shape& s, int B, const Routing& rt, hipStream_t st) {
  hipLaunchKernelGGL(moe_prep_kernel, dim3(1), dim3(64), 0, st, s.E, B * s.k, rt);
  return hipGetLastError();
}

}  // namespace kk

// Split-K MFMA path of the decode-layer step (batch 3-64), gfx950 v_mfma_f32_16x16x32_bf16.
//
// Every product is weights (A operand: 16 rows x 32 k) times activations (B operand: 32 k x
// 16 tokens) into fp32 accumulators (D: 16 rows x 16 tokens).  Lane l of a wave holds row
// (or token) l % 16 and k = 8 * (l / 16) + e of each operand.  Within a run of S MFMAs the
// four lane groups take contiguous k sub-ranges, so each lane reads 16*S contiguous bytes of
// its weight row per run (the same k mapping is used for both operands).
//
// fp32 activations (the residual stream h32 and the SwiGLU activations) enter the MFMA as
// NTERM bf16 terms hi + lo (+ lo2) whose sum reproduces them (to 2^-17 relative with two
// terms, exactly with three), so the products keep fp32-level accuracy; x is already bf16.
//
// Launches of one step:
//   1. o-proj partials over 7 K-slices (one 16-row tile x one slice per wave)
//   2. reduce: h32 = resid + sum of slices (fixed order), optional h_out
//   3. router logit partials (three-term h32), then the shared top-k launch
//   4. grouped gate/up over the active experts + the shared expert: the 8 waves of a block
//      split K of one (expert, 16 gate rows, 16 up rows) unit and reduce through LDS;
//      SwiGLU epilogue -> A (fp32, position-major)
//   5. grouped down-projection the same way -> Y (per position) and ys (shared)
//   6. the combine launch shared with the GEMV path
//
// "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly", section "Recovering time
// between operators": split-K at larger batches to expose parallel work; selected experts;
// shared expert; "vLLM Hyper-Optimizes Kimi K3 on NVIDIA GB300 for Blazing-FAST Inference",
// section "What's Optimized": different kernels per batch size.
#include "kk_common.cuh"
#include "kk_internal.h"

namespace kk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// 8 fp32 values -> NTERM bf16 vectors (RNE), each term the rounding of what the previous
// ones left over; the differences are exact in fp32.
template <int NTERM>
__device__ __forceinline__ void split_terms(const float (&x)[8], u32x4 (&out)[NTERM]) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
#pragma unroll
  for (int q = 0; q < NTERM; ++q) {
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b[e] = f32_to_bf16(r[e]);
      r[e] -= bf16_bits_to_f32(b[e]);
    }
    out[q] = u32x4{b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                   b[6] | (b[7] << 16)};
  }
}

// One lane's B operand for k = kk .. kk+7 of an activation row (bf16 source: one term;
// fp32 source: NTERM terms).  Invalid tokens read a valid row and are zeroed.
template <int NTERM, bool BF16SRC>
__device__ __forceinline__ void load_b(const void* row, int kk, bool valid, u32x4 (&out)[NTERM]) {
  if constexpr (BF16SRC) {
    const u32x4 v = *reinterpret_cast<const u32x4*>((const uint16_t*)row + kk);
    out[0] = valid ? v : u32x4{0u, 0u, 0u, 0u};
  } else {
    const float4* p = reinterpret_cast<const float4*>((const float*)row + kk);
    const float4 a = p[0], b = p[1];
    float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    if (!valid)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    split_terms<NTERM>(x, out);
  }
}

// acc[r][tt] += W[rows of tile r][k_begin, k_end) . X[tokens of tile tt][k_begin, k_end).
// wrow[r]: this lane's weight row of tile r; arow[tt]/aval[tt]: this lane's token row.
template <int NR, int TT, int NTERM, bool BF16SRC, int S>
__device__ __forceinline__ void mfma_span(const uint16_t* const (&wrow)[NR],
                                          const void* const (&arow)[TT], const bool (&aval)[TT],
                                          int ntt, int k_begin, int k_end, int g,
                                          f32x4 (&acc)[NR][TT]) {
  for (int k0 = k_begin; k0 < k_end; k0 += 32 * S) {
    const int kl = k0 + g * 8 * S;
    u32x4 wv[NR][S];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int s = 0; s < S; ++s)
        wv[r][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[r] + kl + 8 * s));
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        if (tt < ntt) {
          u32x4 bv[NTERM];
          load_b<NTERM, BF16SRC>(arow[tt], kl + 8 * s, aval[tt], bv);
#pragma unroll
          for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int q = 0; q < NTERM; ++q) acc[r][tt] = mfma(wv[r][s], bv[q], acc[r][tt]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------ split-K
// part[sp][t][n] = W[n][slice sp] . X[t][slice sp] for N rows (one 16-row tile per wave unit).
template <int TT, int NTERM, bool BF16SRC, int S>
__global__ __launch_bounds__(256) void mfma_splitk_kernel(const uint16_t* __restrict__ W, int N,
                                                          int K, const void* __restrict__ act,
                                                          int B, int splits,
                                                          float* __restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = blockIdx.x * (blockDim.x >> 6) + wave;
  const int tiles = N / 16;
  if (unit >= tiles * splits) return;
  const int tile = unit / splits, sp = unit - tile * splits;
  const int kspan = K / splits;
  const int g = lane >> 4, c = lane & 15;
  const uint16_t* wrow[1] = {W + (size_t)(tile * 16 + c) * K};
  const void* arow[TT];
  bool aval[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int j = tt * 16 + c;
    aval[tt] = j < B;
    const size_t off = (size_t)(aval[tt] ? j : 0) * K;
    arow[tt] = BF16SRC ? (const void*)((const uint16_t*)act + off) : (const void*)((const float*)act + off);
  }
  const int ntt = (B + 15) / 16;
  f32x4 acc[1][TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) acc[0][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  mfma_span<1, TT, NTERM, BF16SRC, S>(wrow, arow, aval, ntt, sp * kspan, (sp + 1) * kspan, g, acc);
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int j = tt * 16 + c;
    if (tt < ntt && j < B) {
      float4 v = {acc[0][tt][0], acc[0][tt][1], acc[0][tt][2], acc[0][tt][3]};
      *reinterpret_cast<float4*>(part + ((size_t)sp * B + j) * N + tile * 16 + 4 * g) = v;
    }
  }
}

// h32[t][n] = r[t][n] + sum_sp part[sp][t][n] (slice order); h_out = RNE(h32) if given.
template <typename T, int MAXS>
__global__ __launch_bounds__(256) void oproj_reduce_kernel(const float* __restrict__ part,
                                                           int splits, const T* __restrict__ r,
                                                           int B, int H, float* __restrict__ h32,
                                                           T* __restrict__ h_out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * H) return;
  float v[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) v[s] = part[(size_t)min(s, splits - 1) * B * H + i];
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) acc += s < splits ? v[s] : 0.f;
  const float hv = Elem<T>::load(r, i) + acc;
  h32[i] = hv;
  if (h_out) Elem<T>::store(h_out, i, hv);
}

// ------------------------------------------------------------------------------ grouped experts
// Group a < n_act: routed expert act[a] over its positions [offsets[e], offsets[e+1]);
// group n_act: the shared expert over tokens 0..B-1.  A unit is (group, row tile pair); the
// KW waves of a block each take K/KW of it and the partial tiles are summed through LDS in
// wave order.
//   MODE 0 (gate/up): rows i0+c of W1 and I+i0+c of W3 (K = H, activations h32 rows of the
//                     tokens); epilogue A[p][i] = silu(gate) * up (As[t][i] for shared).
//   MODE 1 (down):    rows n0+c and n0+16+c of W2 (K = I, activations A rows of the
//                     positions / As rows); epilogue Y[p][n] (ys[t][n] for shared).
struct ExpertArgs {
  const uint16_t* w_routed;  // w13 or w2
  const uint16_t* w_shared;  // ws13 or ws2
  const float* act_routed;   // MODE 0: h32 [B][H]; MODE 1: A [B*k][I]
  const float* act_shared;   // MODE 0: h32;        MODE 1: As [B][Is]
  float* out_routed;         // MODE 0: A [B*k][I]; MODE 1: Y [B*k][H]
  float* out_shared;         // MODE 0: As [B][Is]; MODE 1: ys [B][H]
  int H, I, k, B;
  Routing rt;
};

template <int MODE, int KW, int TT, int S>
__global__ __launch_bounds__(KW * 64) void mfma_expert_kernel(ExpertArgs x) {
  constexpr int NR = 2;
  extern __shared__ f32x4 red[];  // [KW][NR][TT][64] when KW > 1
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int n_act = *x.rt.n_act;
  const int K = MODE == 0 ? x.H : x.I;
  const int out_rows = MODE == 0 ? x.I : x.H;          // per group
  const int tiles = MODE == 0 ? x.I / 16 : x.H / 32;    // units per group
  const size_t wstride = MODE == 0 ? (size_t)2 * x.I * x.H : (size_t)x.H * x.I;
  const int units = (n_act + 1) * tiles;
  const int kspan = K / KW;

  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int a = unit / tiles, tile = unit - a * tiles;
    const bool shared = a == n_act;
    int p0 = 0, cnt = x.B;
    const uint16_t* wbase = x.w_shared;
    if (!shared) {
      const int e = x.rt.act[a];
      p0 = x.rt.offsets[e];
      cnt = x.rt.offsets[e + 1] - p0;
      wbase = x.w_routed + (size_t)e * wstride;
    }
    const int ntt = (cnt + 15) / 16;
    const uint16_t* wrow[NR];
    int row0;
    if (MODE == 0) {
      row0 = tile * 16;
      wrow[0] = wbase + (size_t)(row0 + c) * K;
      wrow[1] = wbase + (size_t)(x.I + row0 + c) * K;
    } else {
      row0 = tile * 32;
      wrow[0] = wbase + (size_t)(row0 + c) * K;
      wrow[1] = wbase + (size_t)(row0 + 16 + c) * K;
    }
    const void* arow[TT];
    bool aval[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int j = tt * 16 + c;
      aval[tt] = j < cnt;
      const int jj = aval[tt] ? j : 0;
      int src;  // activation row
      if (MODE == 0)
        src = shared ? jj : x.rt.perm[p0 + jj] / x.k;  // token rows of h32
      else
        src = shared ? jj : p0 + jj;                   // position rows of A / token rows of As
      const float* base = MODE == 0 ? x.act_routed : (shared ? x.act_shared : x.act_routed);
      arow[tt] = base + (size_t)src * K;
    }
    f32x4 acc[NR][TT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[r][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mfma_span<NR, TT, 2, false, S>(wrow, arow, aval, ntt, wave * kspan, (wave + 1) * kspan, g, acc);

    float* outp = shared ? x.out_shared : x.out_routed;
    const int pbase = shared ? 0 : p0;
    if constexpr (KW == 1) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int j = tt * 16 + c;
        if (tt < ntt && j < cnt) {
          float* o = outp + (size_t)(pbase + j) * out_rows + row0 + 4 * g;
          if (MODE == 0) {
            float4 v;
            v.x = silu_f32(acc[0][tt][0]) * acc[1][tt][0];
            v.y = silu_f32(acc[0][tt][1]) * acc[1][tt][1];
            v.z = silu_f32(acc[0][tt][2]) * acc[1][tt][2];
            v.w = silu_f32(acc[0][tt][3]) * acc[1][tt][3];
            *reinterpret_cast<float4*>(o) = v;
          } else {
            *reinterpret_cast<float4*>(o) = float4{acc[0][tt][0], acc[0][tt][1], acc[0][tt][2], acc[0][tt][3]};
            *reinterpret_cast<float4*>(o + 16) = float4{acc[1][tt][0], acc[1][tt][1], acc[1][tt][2], acc[1][tt][3]};
          }
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) red[((wave * NR + r) * TT + tt) * 64 + lane] = acc[r][tt];
      __syncthreads();
      // one thread per (tile slot tt, lane) sums the KW partial tiles in wave order
      for (int idx = threadIdx.x; idx < TT * 64; idx += blockDim.x) {
        const int tt = idx >> 6, ln = idx & 63;
        const int j = tt * 16 + (ln & 15), gg = ln >> 4;
        if (tt < ntt && j < cnt) {
          f32x4 s0 = red[((0 * NR + 0) * TT + tt) * 64 + ln];
          f32x4 s1 = red[((0 * NR + 1) * TT + tt) * 64 + ln];
          for (int w = 1; w < KW; ++w) {
            s0 += red[((w * NR + 0) * TT + tt) * 64 + ln];
            s1 += red[((w * NR + 1) * TT + tt) * 64 + ln];
          }
          float* o = outp + (size_t)(pbase + j) * out_rows + row0 + 4 * gg;
          if (MODE == 0) {
            float4 v;
            v.x = silu_f32(s0[0]) * s1[0];
            v.y = silu_f32(s0[1]) * s1[1];
            v.z = silu_f32(s0[2]) * s1[2];
            v.w = silu_f32(s0[3]) * s1[3];
            *reinterpret_cast<float4*>(o) = v;
          } else {
            *reinterpret_cast<float4*>(o) = float4{s0[0], s0[1], s0[2], s0[3]};
            *reinterpret_cast<float4*>(o + 16) = float4{s1[0], s1[1], s1[2], s1[3]};
          }
        }
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------------------ dispatch
template <typename K>
void allow_lds_mfma(K kernel) {
  static thread_local const void* done[64];
  static thread_local int n_done = 0;
  for (int i = 0; i < n_done; ++i)
    if (done[i] == (const void*)kernel) return;
  (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
  if (n_done < 64) done[n_done++] = (const void*)kernel;
}

inline int token_tiles(int B) { return B <= 16 ? 1 : (B <= 32 ? 2 : 4); }

template <int TT, int NTERM, bool BF16SRC, int S>
hipError_t splitk_t(const uint16_t* W, int N, int K, const void* act, int B, int splits,
                    float* part, hipStream_t st) {
  const int units = (N / 16) * splits;
  hipLaunchKernelGGL((mfma_splitk_kernel<TT, NTERM, BF16SRC, S>), dim3((units + 3) / 4), dim3(256),
                     0, st, W, N, K, act, B, splits, part);
  return hipGetLastError();
}

template <int NTERM, bool BF16SRC, int S>
hipError_t splitk_dispatch(const uint16_t* W, int N, int K, const void* act, int B, int splits,
                           float* part, hipStream_t st) {
  switch (token_tiles(B)) {
    case 1: return splitk_t<1, NTERM, BF16SRC, S>(W, N, K, act, B, splits, part, st);
    case 2: return splitk_t<2, NTERM, BF16SRC, S>(W, N, K, act, B, splits, part, st);
    default: return splitk_t<4, NTERM, BF16SRC, S>(W, N, K, act, B, splits, part, st);
  }
}

template <int MODE, int KW, int TT, int S>
hipError_t expert_t(const Device& d, const ExpertArgs& x, hipStream_t st) {
  auto kern = mfma_expert_kernel<MODE, KW, TT, S>;
  const size_t lds = KW > 1 ? (size_t)KW * 2 * TT * 64 * sizeof(f32x4) : 0;
  if (lds > 64 * 1024) allow_lds_mfma(kern);
  int bpc = KW >= 8 ? 2 : 16 / KW;
  if (lds && (size_t)bpc * lds > 160 * 1024) bpc = (int)((160 * 1024) / lds);
  if (bpc < 1) bpc = 1;
  hipLaunchKernelGGL(kern, dim3(d.num_cu * bpc), dim3(KW * 64), lds, st, x);
  return hipGetLastError();
}

template <int MODE, int KW, int S>
hipError_t expert_dispatch(const Device& d, const ExpertArgs& x, hipStream_t st) {
  switch (token_tiles(x.B)) {
    case 1: return expert_t<MODE, KW, 1, S>(d, x, st);
    case 2: return expert_t<MODE, KW, 2, S>(d, x, st);
    default: return expert_t<MODE, KW, 4, S>(d, x, st);
  }
}

}  // namespace

bool mfma_supported(const Shape& s, int B) {
  if (B < 1 || B > 64 || s.dtype != 1 || s.I != s.Is) return false;
  if (s.H != 7168 || s.E % 16 != 0) return false;
  if (!(s.Ko == 7168 || s.Ko == 448)) return false;
  return s.I == 2048 || s.I == 128;
}

int mfma_oproj_splits(const Shape& s) { return 7; }
int mfma_router_splits(const Shape& s) { return 7; }

hipError_t launch_oproj_mfma(const Shape& s, const Device& d, int B, const void* x,
                             float* part, const void* w_o, hipStream_t st) {
  const int splits = mfma_oproj_splits(s);
  if (s.Ko == 7168)
    return splitk_dispatch<1, true, 4>((const uint16_t*)w_o, s.H, s.Ko, x, B, splits, part, st);
  if (s.Ko == 448)
    return splitk_dispatch<1, true, 2>((const uint16_t*)w_o, s.H, s.Ko, x, B, splits, part, st);
  return hipErrorInvalidValue;
}

hipError_t launch_oproj_reduce(const Shape& s, int B, const float* part, const void* r,
                               float* h32, void* h_out, hipStream_t st) {
  const int n = B * s.H;
  hipLaunchKernelGGL((oproj_reduce_kernel<uint16_t, 8>), dim3((n + 255) / 256), dim3(256), 0, st,
                     part, mfma_oproj_splits(s), (const uint16_t*)r, B, s.H, h32, (uint16_t*)h_out);
  return hipGetLastError();
}

hipError_t launch_router_mfma(const Shape& s, const Device& d, int B, const float* h32,
                              const void* w_r, float* part, hipStream_t st) {
  return splitk_dispatch<3, false, 4>((const uint16_t*)w_r, s.E, s.H, h32, B,
                                      mfma_router_splits(s), part, st);
}

hipError_t launch_gateup_mfma(const Shape& s, const Device& d, int B, const float* h32,
                              const void* w13, const void* ws13, const Routing& rt, float* A,
                              float* As, hipStream_t st) {
  ExpertArgs x{(const uint16_t*)w13, (const uint16_t*)ws13, h32, h32, A, As, s.H, s.I, s.k, B, rt};
  return expert_dispatch<0, 8, 4>(d, x, st);  // K = H = 7168: 896 per wave
}

hipError_t launch_down_mfma(const Shape& s, const Device& d, int B, const float* A,
                            const float* As, const void* w2, const void* ws2, const Routing& rt,
                            float* Y, float* ys, hipStream_t st) {
  ExpertArgs x{(const uint16_t*)w2, (const uint16_t*)ws2, A, As, Y, ys, s.H, s.I, s.k, B, rt};
  if (s.I == 2048) return expert_dispatch<1, 8, 4>(d, x, st);  // 256 per wave
  if (s.I == 128) return expert_dispatch<1, 1, 4>(d, x, st);   // one 128-k run per unit
  return hipErrorInvalidValue;
}

}  // namespace kk

// Split-K MFMA path of the decode-layer step (batch 3-64), gfx950 v_mfma_f32_16x16x32_bf16.
//
// Every product is weights (A operand: 16 rows x 32 k) times activations (B operand: 32 k x
// 16 tokens) into fp32 accumulators (D: 16 rows x 16 tokens).  Lane l of a wave holds row
// (or token) l % 16 and k = 8 * (l / 16) + e of each operand.  Operands are staged through
// LDS: global loads stay row-contiguous (an operand read straight from HBM would touch 16
// rows per quarter-wave), and the MFMA reads its 16-row layout out of LDS.
//
// fp32 activations (the residual stream h32 and the SwiGLU activations) enter the MFMA as
// NTERM bf16 terms hi + lo (+ lo2) whose sum reproduces them (to 2^-17 relative with two
// terms, exactly with three), so the products keep fp32-level accuracy; x is already bf16.
//
// Launches of one step (5 to 10, by batch, intermediate size and o-proj width;
// kk_query_plan counts them):
//   1. o-proj partials over 7 K chunks (32 rows x one chunk per block unit; over 16 tokens
//      128-row units with all tokens)
//   2. reduce: h32 = resid + sum of chunks (fixed order), optional h_out (with an RMSNorm the
//      reduce also writes u32 = norm(h32))
//   3. router logit partials (three-term h32), then the top-k: one launch with the routing
//      tables up to 16 tokens, else a top-k launch and a tables launch
//      (a 448-wide o-proj slice without a norm: 1-3 are one launch, the o-proj with its
//      residual and the router from r and x through the router-o-proj product, then the top-k)
//   4. grouped gate/up over the active experts + the shared expert, one (expert, 16 gate
//      rows, 16 up rows) unit per block over the whole K; SwiGLU epilogue -> A (fp32).  Small
//      intermediates split every group over K chunks and add a SwiGLU launch that sums them
//      (up to 16 tokens the down-projection sums them instead); over 32 tokens the shared
//      expert's gate/up is a split-K launch of its own plus that SwiGLU launch
//   5. grouped down-projection the same way -> Y (by slot up to 16 tokens, else by position)
//      and ys (shared)
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

// K chunks of the shared expert's split-K gate/up over more than 32 tokens.
constexpr int kSharedSplits = 14;
// Gate/up K chunks for experts with a small intermediate: their groups have only I/16 row tiles
// (8 at I = 128), too few units to fill the chip, so each unit also takes one K chunk.
constexpr int kGateupSplits = 4;

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

// One token row per block: h = r + the o-proj K-split partials summed in slice order (as
// oproj_reduce_kernel), written to h32 / h_out, or h read from h32 when part is null; then
// u32 = h * gamma / sqrt(mean(h^2) + eps).  The sum of squares goes per thread, per wave (DPP),
// then over the waves in order.  Each thread holds columns threadIdx.x + j * blockDim.x.
template <typename T, int MAXS, int MAXJ>
__global__ __launch_bounds__(1024) void norm_rows_kernel(const float* __restrict__ part,
                                                        int splits, const T* __restrict__ r,
                                                        int B, int H, float* __restrict__ h32,
                                                        T* __restrict__ h_out,
                                                        const T* __restrict__ gamma, float eps,
                                                        float* __restrict__ u32) {
  __shared__ float red[16];
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwv = blockDim.x >> 6;
  const size_t row = (size_t)t * H;
  float hv[MAXJ], g[MAXJ];
  if (part) {
    float v[MAXJ][MAXS], rv[MAXJ];
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const int c = min((int)(threadIdx.x + j * blockDim.x), H - 1);
#pragma unroll
      for (int sp = 0; sp < MAXS; ++sp)
        v[j][sp] = part[(size_t)min(sp, splits - 1) * B * H + row + c];
      rv[j] = Elem<T>::load(r, row + c);
    }
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int sp = 0; sp < MAXS; ++sp) acc += sp < splits ? v[j][sp] : 0.f;
      hv[j] = rv[j] + acc;
    }
  } else {
#pragma unroll
    for (int j = 0; j < MAXJ; ++j)
      hv[j] = h32[row + min((int)(threadIdx.x + j * blockDim.x), H - 1)];
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int c = threadIdx.x + j * blockDim.x;
    g[j] = Elem<T>::load(gamma, min(c, H - 1));
    ss += c < H ? hv[j] * hv[j] : 0.f;
  }
  ss = seg_sum_dpp<64>(ss);
  if (lane == 63) red[wave] = ss;
  __syncthreads();
  float sum = 0.f;
  for (int w = 0; w < nwv; ++w) sum += red[w];
  const float inv = 1.f / sqrtf(sum / (float)H + eps);
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int c = threadIdx.x + j * blockDim.x;
    if (c < H) {
      if (part) {
        h32[row + c] = hv[j];
        if (h_out) Elem<T>::store(h_out, row + c, hv[j]);
      }
      u32[row + c] = hv[j] * inv * g[j];
    }
  }
}

// SwiGLU of K-chunk partials of gate/up rows: for each row r of a region,
// dst[r][i] = silu(sum_c P_c[r][i]) * sum_c P_c[r][I + i], chunks summed in order, with
// P_c = base + c * cstride and rows of 2I floats (gate values, then up values).  One launch
// covers two regions (the routed positions into A, the shared expert's tokens into As).
struct SwigluRegion {
  const float* base;
  size_t cstride;
  int rows, chunks;
  float* dst;
};
template <int MAXC>
__global__ __launch_bounds__(256) void swiglu_reduce_kernel(SwigluRegion r0, SwigluRegion r1,
                                                            int I) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  const bool second = i >= r0.rows * I;
  const SwigluRegion R = second ? r1 : r0;
  if (second) i -= r0.rows * I;
  if (i >= R.rows * I) return;
  const int t = i / I, n = i - t * I;
  float g[MAXC], u[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const size_t o = (size_t)min(c, R.chunks - 1) * R.cstride + (size_t)t * 2 * I + n;
    g[c] = R.base[o];
    u[c] = R.base[o + I];
  }
  float zg = 0.f, zu = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    zg += c < R.chunks ? g[c] : 0.f;
    zu += c < R.chunks ? u[c] : 0.f;
  }
  R.dst[i] = silu_f32(zg) * zu;
}

// Arguments of the grouped / split-K launches.
struct UnitArgs {
  const uint16_t* w_routed;  // MODE 0: w13; MODE 1: w2; MODE 2: the weight matrix [N][K]
  const uint16_t* w_shared;  // MODE 0: ws13; MODE 1: ws2
  const void* act_routed;    // MODE 0: h32 [B][H]; MODE 1: A [B*k][I]; MODE 2: X [B][K]
  const float* act_shared;   // MODE 0: h32; MODE 1: As [B][Is]
  float* out_routed;         // MODE 0: A; MODE 1: Y [B*k][H]; MODE 2: part [chunks][B][N]
  float* out_shared;         // MODE 0: As; MODE 1: ys [B][H]
  int H, I, k, B;
  int N, K, chunks;          // MODE 2 (and MODE 0 with gu_part)
  Routing rt;
  // MODE 0 split over `chunks` K chunks: the gate and up sums of chunk c, position p go to
  // gu_part[(c * gu_P + p) * 2I + i] and [.. + I + i] (the shared expert's tokens at
  // positions gu_P - B ..) instead of the SwiGLU into A / As
  float* gu_part;
  int gu_P;
  // MODE 2 with one K chunk and resid != nullptr: h32[t][n] = resid[t][n] + the product
  // (the o-proj with its residual add) instead of the partial
  const uint16_t* resid;
  float* h32;
  // MODE 1: rows of Y by slot t*k + j (up to 16 tokens) instead of by position
  bool y_by_slot;
  // MODE 0 / 1: the groups this launch covers: kGroupsEvery, kGroupsRoutedOnly (the active
  // experts) or kGroupsSharedOnly (the shared expert, which reads no routing table)
  int sel;
};

// ------------------------------------------------------------------------------ LDS-staged
// All MFMA launches share one kernel.  A unit is (group, pair of 16-row tiles, K chunk):
//   MODE 0 (gate/up): group a < n_act is routed expert act[a] over its positions, group
//     n_act the shared expert over tokens 0..B-1; tiles = W1 rows i0.. and W3 rows I+i0..;
//     K = H in one chunk; epilogue A[p][i] = silu(gate) * up (As[t][i] for shared).
//   MODE 1 (down): same groups; tiles = W2 rows n0.. and n0+16..; K = I in one chunk;
//     epilogue Y[p][n] (ys[t][n] for shared).
//   MODE 2 (split-K): one group, tokens 0..B-1; tiles = rows n0.. and n0+16.. of W [N][K];
//     chunk c of K -> part[c][t][n].
// The chunk is walked in stages of KS.  Each stage the 256 threads load the tile pair's 32
// rows x KS (every quarter-wave reading 256 contiguous bytes of one row) and the group's
// token rows x KS (bf16 as is, or fp32 split into NTERM bf16 terms on the way into LDS),
// then the four waves multiply (k-step, token tile) pairs out of LDS while the next stage's
// loads are in flight.  Each wave's partial tiles are summed through LDS in wave order at
// the end of the unit.
//   LDS weights: [32 rows][KS/8 + 1] 16-byte chunks (one chunk of padding per row)
//   LDS activations: [NTERM][16*TT tokens][KS/8 + 1] 16-byte chunks (token-major: a thread's
//   store lands next to its neighbours', and the padding spreads the 16 tokens one operand
//   read touches over all banks)
// One unit of the LDS-staged product: the tile pair `tile` of group (wbase, positions p0 ..
// p0 + cnt - 1, `shared`) over K chunk `chunk`.  The next stage's loads (DEPTH stages) are
// kept in flight in registers; with two, a stage past the end reads the activation buffer
// instead (small and cache-resident), so every loop pass issues the same loads.  Weights are
// read with non-temporal loads, or with plain (cached) loads when NTW is false, for units
// whose weights other blocks of the same XCD read again.
template <int MODE, int TT, int KS, int NTERM, bool BF16SRC, bool NTW = true, bool SLOT = false,
          int DEPTH = 1>
__device__ __forceinline__ void staged_unit(const UnitArgs& x, u32x4* lds, int tile, int chunk,
                                            int p0, int cnt, const uint16_t* wbase,
                                            bool shared) {
  constexpr int K8 = KS / 8;
  constexpr int WP = K8 + 1;
  constexpr int AP = K8 + 1;
  constexpr int NTOK = 16 * TT;
  constexpr int W_CH = 32 * WP;
  constexpr int WLD = (32 * K8 + 255) / 256;    // weight chunks per thread per stage
  constexpr int ALD = (NTOK * K8 + 255) / 256;  // activation chunks (8 values) per thread
  constexpr int KSTEPS = KS / 32;
  constexpr int AW = BF16SRC ? 1 : 2;           // 16-byte words per activation chunk
  u32x4* lw = lds;
  u32x4* la = lds + W_CH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int K = MODE == 0 ? x.H : (MODE == 1 ? x.I : x.K);
  const int out_rows = MODE == 0 ? x.I : (MODE == 1 ? x.H : x.N);
  const int chunks = (MODE == 2 || (MODE == 0 && x.gu_part)) ? x.chunks : 1;
  const int kchunk = K / chunks;
  const int nst = kchunk / KS;
  const int ntt = (cnt + 15) / 16;
  const int row0 = MODE == 0 ? tile * 16 : tile * 32;
  const int kbase = chunk * kchunk;
  // this thread's weight chunks: q = tid + 256 i -> (row q / K8, chunk q % K8)
  const uint16_t* wsrc[WLD];
#pragma unroll
  for (int i = 0; i < WLD; ++i) {
    const int q = min(tid + 256 * i, 32 * K8 - 1), rr = q / K8, ch = q - rr * K8;
    const int wr = MODE == 0 ? (rr < 16 ? row0 + rr : x.I + row0 + rr - 16) : row0 + rr;
    wsrc[i] = wbase + (size_t)wr * K + kbase + ch * 8;
  }
  // this thread's activation chunks: q = tid + 256 i -> (token slot q / K8, chunk q % K8)
  const void* asrc[ALD];
  bool aok[ALD];
#pragma unroll
  for (int i = 0; i < ALD; ++i) {
    const int q = min(tid + 256 * i, NTOK * K8 - 1), j = q / K8, ch = q - j * K8;
    aok[i] = j < cnt;
    const int jj = aok[i] ? j : 0;
    int src;
    if (MODE == 0)
      src = shared ? p0 + jj : x.rt.perm[p0 + jj] / x.k;
    else
      src = p0 + jj;
    const void* base = (MODE == 1 && shared) ? (const void*)x.act_shared : x.act_routed;
    const size_t off = (size_t)src * K + kbase + ch * 8;
    asrc[i] = BF16SRC ? (const void*)((const uint16_t*)base + off) : (const void*)((const float*)base + off);
  }
  // DEPTH register buffers of stage loads: DEPTH stages in flight while one is multiplied
  static_assert(DEPTH == 1 || DEPTH == 2, "one or two stages in flight");
  u32x4 wreg[DEPTH][WLD], areg[DEPTH][ALD][AW];
  const void* dummy = x.act_routed;
  auto load_stage = [&](int st, int b) {
    const bool live = st < nst;
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const u32x4* p = live ? reinterpret_cast<const u32x4*>(wsrc[i] + st * KS)
                            : reinterpret_cast<const u32x4*>(dummy);
      wreg[b][i] = NTW ? __builtin_nontemporal_load(p) : *p;
    }
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const u32x4* p = BF16SRC ? reinterpret_cast<const u32x4*>((const uint16_t*)asrc[i] + st * KS)
                               : reinterpret_cast<const u32x4*>((const float*)asrc[i] + st * KS);
      if (!live) p = reinterpret_cast<const u32x4*>(dummy);
#pragma unroll
      for (int w = 0; w < AW; ++w) areg[b][i][w] = aok[i] ? p[w] : u32x4{0u, 0u, 0u, 0u};
    }
  };
  f32x4 acc[2][TT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[r][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto store_stage = [&](int b) {
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int q = tid + 256 * i, rr = q / K8, ch = q - rr * K8;
      if (q < 32 * K8) lw[rr * WP + ch] = wreg[b][i];
    }
    // only the group's own token slots: the others were zeroed at the start of the unit
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int q = tid + 256 * i, j = q / K8, ch = q - j * K8;
      if (q < NTOK * K8 && aok[i]) {
        if constexpr (BF16SRC) {
          la[j * AP + ch] = areg[b][i][0];
        } else {
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = __uint_as_float(areg[b][i][0][e]);
            v[4 + e] = __uint_as_float(areg[b][i][1][e]);
          }
          u32x4 terms[NTERM];
          split_terms<NTERM>(v, terms);
#pragma unroll
          for (int q2 = 0; q2 < NTERM; ++q2) la[(q2 * NTOK + j) * AP + ch] = terms[q2];
        }
      }
    }
  };
  if (cnt < NTOK)
    for (int q = tid; q < NTERM * NTOK * AP; q += 256)
      if ((q / AP) % NTOK >= cnt) la[q] = u32x4{0u, 0u, 0u, 0u};
  // SLOT (one-tile down-projection units) with Y by slot, a routed group: the slot of the
  // epilogue's position (thread tid writes position tid % 16 of the unit), requested now so it
  // is there at the end
  int out_slot = 0;
  if constexpr (SLOT) {
    static_assert(MODE == 1 && TT == 1, "slots of one-tile down-projection units");
    if (!shared && x.y_by_slot && tid < 64) out_slot = x.rt.perm[p0 + min(tid & 15, cnt - 1)];
  }
  auto compute_stage = [&]() {
    for (int pr = wave; pr < KSTEPS * ntt; pr += 4) {
      const int ks = pr % KSTEPS, tt = pr / KSTEPS;
      const u32x4 a0 = lw[c * WP + ks * 4 + g];
      const u32x4 a1 = lw[(16 + c) * WP + ks * 4 + g];
      u32x4 bq[NTERM];
#pragma unroll
      for (int q2 = 0; q2 < NTERM; ++q2) bq[q2] = la[(q2 * NTOK + tt * 16 + c) * AP + ks * 4 + g];
#pragma unroll
      for (int t2 = 0; t2 < TT; ++t2) {
        if (t2 == tt) {
#pragma unroll
          for (int q2 = 0; q2 < NTERM; ++q2) {
            acc[0][t2] = mfma(a0, bq[q2], acc[0][t2]);
            acc[1][t2] = mfma(a1, bq[q2], acc[1][t2]);
          }
        }
      }
    }
  };

  if constexpr (DEPTH == 1) {
    load_stage(0, 0);
    for (int st = 0; st < nst; ++st) {
      store_stage(0);
      __syncthreads();
      if (st + 1 < nst) load_stage(st + 1, 0);
      compute_stage();
      __syncthreads();
    }
  } else {
    // (a stage past the end loads the activation buffer into the spare registers, never used)
    load_stage(0, 0);
    load_stage(1, 1);
    for (int st = 0; st < nst; st += 2) {
      store_stage(0);
      __syncthreads();
      load_stage(st + 2, 0);
      compute_stage();
      __syncthreads();
      if (st + 1 < nst) {
        store_stage(1);
        __syncthreads();
        load_stage(st + 3, 1);
        compute_stage();
        __syncthreads();
      }
    }
  }
  // sum the four waves' partial tiles in wave order, then the epilogue
  f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) red[((wave * 2 + r) * TT + tt) * 64 + lane] = acc[r][tt];
  __syncthreads();
  float* outp = shared ? x.out_shared : x.out_routed;
  for (int idx = tid; idx < TT * 64; idx += 256) {
    const int tt = idx >> 6, ln = idx & 63;
    const int j = tt * 16 + (ln & 15), gg = ln >> 4;
    if (tt < ntt && j < cnt) {
      f32x4 s0 = red[((0 * 2 + 0) * TT + tt) * 64 + ln];
      f32x4 s1 = red[((0 * 2 + 1) * TT + tt) * 64 + ln];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        s0 += red[((w * 2 + 0) * TT + tt) * 64 + ln];
        s1 += red[((w * 2 + 1) * TT + tt) * 64 + ln];
      }
      float* o;
      if (MODE == 2)
        o = outp + ((size_t)chunk * x.B + p0 + j) * out_rows + row0 + 4 * gg;
      else if (SLOT && !shared && x.y_by_slot)
        o = outp + (size_t)out_slot * out_rows + row0 + 4 * gg;
      else
        o = outp + (size_t)(p0 + j) * out_rows + row0 + 4 * gg;
      if (MODE == 2 && x.resid) {
        const size_t ho = (size_t)(p0 + j) * out_rows + row0 + 4 * gg;
        const float4 r0 = Elem<uint16_t>::load4(x.resid, ho);
        const float4 r1 = Elem<uint16_t>::load4(x.resid, ho + 16);
        *reinterpret_cast<float4*>(x.h32 + ho) = float4{r0.x + s0[0], r0.y + s0[1], r0.z + s0[2], r0.w + s0[3]};
        *reinterpret_cast<float4*>(x.h32 + ho + 16) = float4{r1.x + s1[0], r1.y + s1[1], r1.z + s1[2], r1.w + s1[3]};
      } else if (MODE == 0 && x.gu_part) {
        const int pos = shared ? x.gu_P - x.B + p0 + j : p0 + j;
        float* q = x.gu_part + ((size_t)chunk * x.gu_P + pos) * 2 * x.I + row0 + 4 * gg;
        *reinterpret_cast<float4*>(q) = float4{s0[0], s0[1], s0[2], s0[3]};
        *reinterpret_cast<float4*>(q + x.I) = float4{s1[0], s1[1], s1[2], s1[3]};
      } else if (MODE == 0) {
        *reinterpret_cast<float4*>(o) =
            float4{silu_f32(s0[0]) * s1[0], silu_f32(s0[1]) * s1[1], silu_f32(s0[2]) * s1[2],
                   silu_f32(s0[3]) * s1[3]};
      } else {
        *reinterpret_cast<float4*>(o) = float4{s0[0], s0[1], s0[2], s0[3]};
        *reinterpret_cast<float4*>(o + 16) = float4{s1[0], s1[1], s1[2], s1[3]};
      }
    }
  }
  __syncthreads();
}

// LDS bytes of one block of staged_unit<.., TT, KS, NTERM, ..>.
constexpr size_t staged_lds(int TT, int KS, int NTERM) {
  return (size_t)(32 * (KS / 8 + 1) + NTERM * (KS / 8 + 1) * 16 * TT) * 16 > (size_t)4 * 2 * TT * 64 * 16
             ? (size_t)(32 * (KS / 8 + 1) + NTERM * (KS / 8 + 1) * 16 * TT) * 16
             : (size_t)4 * 2 * TT * 64 * 16;
}

// Group a of a launch: its weights, positions and token count.
struct Group {
  const uint16_t* wbase;
  int p0, cnt;
  bool shared;
};
// A wave-uniform read of a routing table entry, through the scalar data cache when SCALAR.  The
// tables are written by an earlier launch (the cache starts each dispatch invalidated), so the
// read sees them; its wait then counts scalar loads only, not the vector loads (weights) in
// flight.  (Measured per kernel: it shortens the short-K down-projection, whose next unit's
// group is looked up behind the current unit's output-slot load, and costs the grouped
// launches a little.)
template <bool SCALAR>
__device__ __forceinline__ int table_entry(const int* p, int i) {
  if constexpr (SCALAR) return ((const __attribute__((address_space(4))) int*)p)[i];
  return p[i];
}

template <int MODE, bool SCALAR = false>
__device__ __forceinline__ Group group_of(const UnitArgs& x, int a, int n_groups) {
  Group gr{x.w_routed, 0, x.B, false};
  if (MODE == 2) return gr;
  const size_t wstride = MODE == 0 ? (size_t)2 * x.I * x.H : (size_t)x.H * x.I;
  gr.shared = a == n_groups - 1;
  if (gr.shared) {
    gr.wbase = x.w_shared;
  } else {
    const int e = table_entry<SCALAR>(x.rt.act, a);
    gr.p0 = table_entry<SCALAR>(x.rt.offsets, e);
    gr.cnt = table_entry<SCALAR>(x.rt.offsets, e + 1) - gr.p0;
    gr.wbase = x.w_routed + (size_t)e * wstride;
  }
  return gr;
}

// All MFMA launches of one token-tile width: units (group, tile pair, K chunk) over a
// persistent grid.  GSEL picks what a launch covers: 0 every group; 4 the routed experts cut
// into pieces of at most 16 positions (rt.vg), 5 those plus the shared expert's tokens in
// pieces of 16 (one-tile launches over any batch).
template <int MODE, int TT, int KS, int NTERM, bool BF16SRC, int GSEL>
__global__ __launch_bounds__(256) void mfma_staged_kernel(UnitArgs x) {
  extern __shared__ u32x4 lds[];  // weights then activations; reused for the final reduction
  // groups: the active experts 0 .. n_act - 1, then the shared expert; a launch covers all of
  // them, the routed ones (ng = n_act) or the shared one (n_act taken as 0: no table is read)
  const int n_act = (MODE == 2 || x.sel == kGroupsSharedOnly) ? 0 : *x.rt.n_act;
  const int n_groups = n_act + 1;
  const int ng = x.sel == kGroupsRoutedOnly ? n_act : n_groups;
  const int out_rows = MODE == 0 ? x.I : (MODE == 1 ? x.H : x.N);
  const int tiles = MODE == 0 ? x.I / 16 : out_rows / 32;
  const int chunks = (MODE == 2 || (MODE == 0 && x.gu_part)) ? x.chunks : 1;
  if constexpr (GSEL >= 4) {
    static_assert(TT == 1 && MODE != 2, "pieces are one token tile of a grouped launch");
    const int nv = x.sel == kGroupsSharedOnly ? 0 : *x.rt.n_vg;
    const int pieces = nv + (GSEL == 5 && x.sel != kGroupsRoutedOnly ? (x.B + 15) / 16 : 0);
    const int units = pieces * tiles * chunks;
    for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
      const int v = unit / (tiles * chunks);
      const int rem = unit - v * tiles * chunks;
      const int tile = rem / chunks, chunk = rem - tile * chunks;
      int p0, cnt;
      Group gr;
      if (v < nv) {
        const int ent = x.rt.vg[v], pc = ent & 3;
        gr = group_of<MODE>(x, ent >> 2, n_groups);
        p0 = gr.p0 + 16 * pc;
        cnt = min(16, gr.cnt - 16 * pc);
      } else {
        gr = group_of<MODE>(x, n_groups - 1, n_groups);
        p0 = 16 * (v - nv);
        cnt = min(16, x.B - p0);
      }
      // (the full-size routed pieces over 32 tokens: two stages in flight measured faster there;
      // the other launches keep four blocks per CU with one)
      staged_unit<MODE, 1, KS, NTERM, BF16SRC, true, false, GSEL == 4 ? 2 : 1>(
          x, lds, tile, chunk, p0, cnt, gr.wbase, gr.shared);
    }
    return;
  }
  const int units = (MODE == 2 ? 1 : ng) * tiles * chunks;
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int a = unit / (tiles * chunks);
    const int rem = unit - a * tiles * chunks;
    const int tile = rem / chunks, chunk = rem - tile * chunks;
    const Group gr = group_of<MODE>(x, a, n_groups);
    staged_unit<MODE, TT, KS, NTERM, BF16SRC, true, MODE == 1 && TT == 1>(
        x, lds, tile, chunk, gr.p0, gr.cnt, gr.wbase,
                                             gr.shared);
  }
}

// Down-projection of experts with a short K (K = I = 128): a unit is 128 output rows of one
// group, one 32-row tile pair per wave.  Its weights (32 KB) are staged once; each wave runs
// the whole K for its own tile pair, token tile by token tile, so a unit costs one weight round
// trip and needs no cross-wave reduction; the next unit's weights are requested as soon as
// this unit's are in LDS.  (The general unit splits K over the four waves, which for K = 128
// leaves one 32-wide step per wave and a reduction per 8 KB of weights.)  With x.gu_part the
// activations are formed as they are staged: the SwiGLU of the gate/up K-chunk partials, summed
// in chunk order (no SwiGLU launch between the gate/up and the down-projection).
template <int K>
__global__ __launch_bounds__(256) void mfma_down_shortk_kernel(UnitArgs x) {
  constexpr int K8 = K / 8, WP = K8 + 1, AP = K8 + 1, ROWS = 128, WLD = ROWS * K8 / 256;
  static_assert(16 * K8 == 256, "one activation chunk per thread and token tile");
  extern __shared__ u32x4 lds[];
  u32x4* lw = lds;              // [ROWS][WP]
  u32x4* la = lds + ROWS * WP;  // [2 terms][16 tokens][AP]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;
  const int n_act = x.sel == kGroupsSharedOnly ? 0 : *x.rt.n_act;
  const int n_groups = n_act + 1;  // the shared expert last
  const int tiles = x.H / ROWS;
  const int units = (x.sel == kGroupsRoutedOnly ? n_act : n_groups) * tiles;
  u32x4 wreg[WLD];
  auto load_w = [&](int un) {
    const int u = min(un, units - 1);  // past the end: a valid unit's rows, never used
    const int a = u / tiles, tile = u - a * tiles;
    const Group gr = group_of<1, true>(x, a, n_groups);
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int q = tid + 256 * i, rr = q / K8, ch = q - rr * K8;
      wreg[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(gr.wbase + (size_t)(tile * ROWS + rr) * K + ch * 8));
    }
  };
  // Up to 16 tokens (every group one token tile) each block takes a contiguous run of units,
  // so consecutive units mostly share a group, which stages its activations once per run.
  // Beyond, units are dealt out across the blocks, which spreads the multi-tile groups.
  const bool runs = x.B <= 16;
  const int per = (units + gridDim.x - 1) / gridDim.x;
  const int u0 = runs ? blockIdx.x * per : blockIdx.x;
  const int u1 = runs ? min(units, u0 + per) : units;
  const int step = runs ? 1 : gridDim.x;
  if (u0 >= u1) return;
  load_w(u0);
  int staged = -1;  // group whose (single) token tile la holds
  for (int unit = u0; unit < u1; unit += step) {
    const int a = unit / tiles, tile = unit - a * tiles;
    const Group gr = group_of<1, true>(x, a, n_groups);
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int q = tid + 256 * i, rr = q / K8, ch = q - rr * K8;
      lw[rr * WP + ch] = wreg[i];
    }
    const int ntt = (gr.cnt + 15) / 16;
    const float* asrc = gr.shared ? x.act_shared : reinterpret_cast<const float*>(x.act_routed);
    float* outp = gr.shared ? x.out_shared : x.out_routed;
    // With Y by slot (up to 16 tokens, one token tile): the slot of the lane's output position,
    // requested before the next unit's weights so that waiting for it does not wait for those.
    const int oslot = (gr.shared || !x.y_by_slot) ? 0 : x.rt.perm[gr.p0 + min(c, gr.cnt - 1)];
    if (unit + step < u1) load_w(unit + step);
    for (int tt = 0; tt < ntt; ++tt) {
      if (ntt > 1 || staged != a) {
        staged = ntt > 1 ? -1 : a;
        const int j = tid / K8, ch = tid - j * K8, jt = tt * 16 + j;
        const bool ok = jt < gr.cnt;
        float v[8];
        if (x.gu_part) {
          // the SwiGLU of the gate/up K-chunk partials of this position (the shared expert's
          // tokens after the routed positions), chunks summed in order
          const int pos = ok ? (gr.shared ? x.gu_P - x.B + jt : gr.p0 + jt) : 0;
          float4 pg[kGateupSplits][2], pu[kGateupSplits][2];
#pragma unroll
          for (int c2 = 0; c2 < kGateupSplits; ++c2) {
            const float* src = x.gu_part + ((size_t)c2 * x.gu_P + pos) * 2 * K + ch * 8;
            pg[c2][0] = reinterpret_cast<const float4*>(src)[0];
            pg[c2][1] = reinterpret_cast<const float4*>(src)[1];
            pu[c2][0] = reinterpret_cast<const float4*>(src + K)[0];
            pu[c2][1] = reinterpret_cast<const float4*>(src + K)[1];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float zg = 0.f, zu = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < kGateupSplits; ++c2) {
              const float4 g4 = pg[c2][e >> 2], u4 = pu[c2][e >> 2];
              zg += (e & 3) == 0 ? g4.x : (e & 3) == 1 ? g4.y : (e & 3) == 2 ? g4.z : g4.w;
              zu += (e & 3) == 0 ? u4.x : (e & 3) == 1 ? u4.y : (e & 3) == 2 ? u4.z : u4.w;
            }
            v[e] = silu_f32(zg) * zu;
          }
        } else {
          const int row = ok ? (gr.shared ? jt : gr.p0 + jt) : 0;
          const float4* src = reinterpret_cast<const float4*>(asrc + (size_t)row * K + ch * 8);
          const float4 v0 = src[0], v1 = src[1];
          v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
          v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
        }
        if (!ok)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = 0.f;
        u32x4 terms[2];
        split_terms<2>(v, terms);
        la[(0 * 16 + j) * AP + ch] = terms[0];
        la[(1 * 16 + j) * AP + ch] = terms[1];
      }
      __syncthreads();
      f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < K / 32; ++ks) {
        const u32x4 a0 = lw[(wave * 32 + c) * WP + ks * 4 + g];
        const u32x4 a1 = lw[(wave * 32 + 16 + c) * WP + ks * 4 + g];
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          const u32x4 b = la[(q2 * 16 + c) * AP + ks * 4 + g];
          acc0 = mfma(a0, b, acc0);
          acc1 = mfma(a1, b, acc1);
        }
      }
      const int j = tt * 16 + c;
      if (j < gr.cnt) {
        const int orow = gr.shared ? j : (x.y_by_slot ? oslot : gr.p0 + j);
        float* o = outp + (size_t)orow * x.H + tile * ROWS + wave * 32 + 4 * g;
        *reinterpret_cast<float4*>(o) = float4{acc0[0], acc0[1], acc0[2], acc0[3]};
        *reinterpret_cast<float4*>(o + 16) = float4{acc1[0], acc1[1], acc1[2], acc1[3]};
      }
      __syncthreads();  // la (next token tile) and lw (next unit) are rewritten after this
    }
  }
}

// Split-K product for many tokens with tall units: a unit is 128 weight rows x one K chunk for
// all the group's tokens (16 TT slots).  Each stage the block stages the 128 rows' KS columns of
// weights and the tokens' KS activations (NTERM bf16 terms) in LDS once, and wave w multiplies
// its own 32-row tile pair against every token tile over the stage's whole depth, so a stage's
// activations are staged once per 128 weight rows (not once per 32) and no cross-wave reduction
// is needed.  Out: part[chunk][t][n] for t < B (MODE 2 of UnitArgs).  The next stage's loads
// are in flight while the current one is multiplied; a stage past the end re-reads the
// activation buffer.
template <int TT, int KS, int NTERM, bool BF16SRC, int RTW = 2>
__global__ __launch_bounds__(256) void mfma_tall_kernel(UnitArgs x) {
  constexpr int ROWS = 64 * RTW, K8 = KS / 8, WP = K8 + 1, AP = K8 + 1, NTOK = 16 * TT;
  constexpr int WLD = ROWS * K8 / 256;          // weight chunks per thread per stage
  constexpr int ALD = (NTOK * K8 + 255) / 256;  // activation chunks (8 values) per thread
  constexpr int AW = BF16SRC ? 1 : 2;           // 16-byte words per activation chunk
  constexpr int KSTEPS = KS / 32;
  static_assert(ROWS * K8 % 256 == 0, "whole weight chunks per thread");
  extern __shared__ u32x4 lds[];
  u32x4* lw = lds;                  // [ROWS][WP]
  u32x4* la = lds + ROWS * WP;      // [NTERM][NTOK][AP]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c = lane & 15;
  const int K = x.K, N = x.N, B = x.B, chunks = x.chunks;
  const int kchunk = K / chunks, nst = kchunk / KS;
  const int units = (N / ROWS) * chunks;
  const int ntt = (B + 15) / 16;
  // slots past the batch stay zero in LDS for the whole launch
  for (int q = tid; q < NTERM * NTOK * AP; q += 256)
    if ((q / AP) % NTOK >= B) la[q] = u32x4{0u, 0u, 0u, 0u};
  const void* dummy = x.act_routed;
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int rb = unit / chunks, chunk = unit - rb * chunks;
    const int row0 = rb * ROWS, kbase = chunk * kchunk;
    const uint16_t* wsrc[WLD];
#pragma unroll
    for (int i = 0; i < WLD; ++i) {
      const int q = tid + 256 * i, rr = q / K8, ch = q - rr * K8;
      wsrc[i] = x.w_routed + (size_t)(row0 + rr) * K + kbase + ch * 8;
    }
    const void* asrc[ALD];
    bool aok[ALD];
#pragma unroll
    for (int i = 0; i < ALD; ++i) {
      const int q = min(tid + 256 * i, NTOK * K8 - 1), j = q / K8, ch = q - j * K8;
      aok[i] = tid + 256 * i < NTOK * K8 && j < B;
      const size_t off = (size_t)(aok[i] ? j : 0) * K + kbase + ch * 8;
      asrc[i] = BF16SRC ? (const void*)((const uint16_t*)x.act_routed + off)
                        : (const void*)((const float*)x.act_routed + off);
    }
    u32x4 wreg[WLD], areg[ALD][AW];
    auto load_stage = [&](int st) {
      const bool live = st < nst;
#pragma unroll
      for (int i = 0; i < WLD; ++i)
        wreg[i] = __builtin_nontemporal_load(live ? reinterpret_cast<const u32x4*>(wsrc[i] + st * KS)
                                                  : reinterpret_cast<const u32x4*>(dummy));
#pragma unroll
      for (int i = 0; i < ALD; ++i) {
        const u32x4* p = !live ? reinterpret_cast<const u32x4*>(dummy)
                         : BF16SRC ? reinterpret_cast<const u32x4*>((const uint16_t*)asrc[i] + st * KS)
                                   : reinterpret_cast<const u32x4*>((const float*)asrc[i] + st * KS);
#pragma unroll
        for (int w = 0; w < AW; ++w) areg[i][w] = aok[i] ? p[w] : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto store_stage = [&]() {
#pragma unroll
      for (int i = 0; i < WLD; ++i) {
        const int q = tid + 256 * i, rr = q / K8, ch = q - rr * K8;
        lw[rr * WP + ch] = wreg[i];
      }
#pragma unroll
      for (int i = 0; i < ALD; ++i) {
        const int q = tid + 256 * i, j = q / K8, ch = q - j * K8;
        if (q < NTOK * K8 && aok[i]) {
          if constexpr (BF16SRC) {
            la[j * AP + ch] = areg[i][0];
          } else {
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = __uint_as_float(areg[i][0][e]);
              v[4 + e] = __uint_as_float(areg[i][1][e]);
            }
            u32x4 terms[NTERM];
            split_terms<NTERM>(v, terms);
#pragma unroll
            for (int q2 = 0; q2 < NTERM; ++q2) la[(q2 * NTOK + j) * AP + ch] = terms[q2];
          }
        }
      }
    };
    f32x4 acc[RTW][TT];
#pragma unroll
    for (int r = 0; r < RTW; ++r)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[r][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    load_stage(0);
    for (int st = 0; st < nst; ++st) {
      store_stage();
      __syncthreads();
      if (st + 1 < nst) load_stage(st + 1);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        u32x4 a[RTW];
#pragma unroll
        for (int r = 0; r < RTW; ++r) a[r] = lw[(wave * 16 * RTW + 16 * r + c) * WP + ks * 4 + g];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if (tt < ntt) {
#pragma unroll
            for (int q2 = 0; q2 < NTERM; ++q2) {
              const u32x4 bq = la[(q2 * NTOK + tt * 16 + c) * AP + ks * 4 + g];
#pragma unroll
              for (int r = 0; r < RTW; ++r) acc[r][tt] = mfma(a[r], bq, acc[r][tt]);
            }
          }
        }
      }
      __syncthreads();
    }
    // lane (g, c) of each accumulator holds rows 4 g .. 4 g + 3 of its 16-row tile, token c
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int j = tt * 16 + c;
      if (tt < ntt && j < B) {
        float* o = x.out_routed + ((size_t)chunk * B + j) * N + row0 + wave * 16 * RTW + 4 * g;
#pragma unroll
        for (int r = 0; r < RTW; ++r)
          *reinterpret_cast<float4*>(o + 16 * r) =
              float4{acc[r][tt][0], acc[r][tt][1], acc[r][tt][2], acc[r][tt][3]};
      }
    }
  }
}

// LDS bytes of one block of mfma_tall_kernel<TT, KS, NTERM, .., RTW>.
constexpr size_t tall_lds(int TT, int KS, int NTERM, int RTW = 2) {
  return (size_t)(64 * RTW * (KS / 8 + 1) + NTERM * (KS / 8 + 1) * 16 * TT) * 16;
}

// Split-K product with the tokens split as well: units (row tile, K chunk, 16-token quarter),
// so that a launch over many tokens but few row tiles (the router: 12 row tiles x 7 chunks)
// still fills the chip.  Each quarter reads the unit's weights; the quarters of one (tile,
// chunk) run on one XCD, so all but the first are served by its L2.
template <int KS, int NTERM, bool BF16SRC>
__global__ __launch_bounds__(256) void mfma_token_split_kernel(UnitArgs x) {
  extern __shared__ u32x4 lds[];
  // Units run in groups of 8 (tile, chunk) pairs x nq quarters, the quarters of one pair 8
  // units apart: blocks b and b + 8 share an XCD, so the quarters read the pair's weights
  // through one L2 (plain loads, which allocate there) instead of once each from HBM.
  const int tiles = x.N / 32, nq = (x.B + 15) / 16;
  const int pairs = tiles * x.chunks;
  const int units = (pairs + 7) / 8 * 8 * nq;
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int grp = unit / (8 * nq), r = unit - grp * 8 * nq;
    const int q = r / 8, tc = grp * 8 + (r & 7);
    if (tc >= pairs) continue;
    const int tile = tc / x.chunks, chunk = tc - tile * x.chunks;
    const int p0 = 16 * q;
    staged_unit<2, 1, KS, NTERM, BF16SRC, false>(x, lds, tile, chunk, p0, min(16, x.B - p0),
                                                 x.w_routed, false);
  }
}

// The o-proj and the router in one launch, the router not waiting for h: logit = W_r . r +
// (W_r W_o) . x, with the router-o-proj product kept as two bf16 planes ([2][E][Ko]).  Four
// split-K products of bf16 activations: the router rows against r over eight K chunks of two
// stages (logit partial slots 0-7), the o-proj (one K chunk: h32 = r + W_o x in its epilogue),
// and the two product planes against x (slots 8 and 9).  Units are (product, row tile pair, K
// chunk), the router's first (the longest); over 16 tokens (QUARTERS) each unit also takes one
// 16-token quarter, the quarters of one (product, tile, chunk) 8 units apart so that they run on
// blocks of one XCD and read its weights through that XCD's L2 (plain loads).
struct MultiArgs {
  UnitArgs p[4];
  int units[4];
};
template <int KS, bool QUARTERS>
__global__ __launch_bounds__(256) void mfma_oproj_router_kernel(MultiArgs m) {
  extern __shared__ u32x4 lds[];
  const int c1 = m.units[0], c2 = c1 + m.units[1], c3 = c2 + m.units[2], pairs = c3 + m.units[3];
  const int B = m.p[0].B, nq = QUARTERS ? (B + 15) / 16 : 1;
  const int total = QUARTERS ? (pairs + 7) / 8 * 8 * nq : pairs;
  auto run = [&](const UnitArgs& x, int u, int q) {
    const int tile = u / x.chunks, chunk = u - tile * x.chunks;
    const int p0 = 16 * q;
    staged_unit<2, 1, KS, 1, true, !QUARTERS>(x, lds, tile, chunk, p0, min(16, B - p0), x.w_routed,
                                               false);
  };
  for (int unit = blockIdx.x; unit < total; unit += gridDim.x) {
    int tc = unit, q = 0;
    if (QUARTERS) {
      const int grp = unit / (8 * nq), r = unit - grp * 8 * nq;
      q = r / 8;
      tc = grp * 8 + (r & 7);
      if (tc >= pairs) continue;
    }
    if (tc < c1)
      run(m.p[0], tc, q);
    else if (tc < c2)
      run(m.p[1], tc - c1, q);
    else if (tc < c3)
      run(m.p[2], tc - c2, q);
    else
      run(m.p[3], tc - c3, q);
  }
}

// Grouped launch (gate/up or down) for batches over 16 tokens: groups of more than 16 tokens
// (the shared expert, and any routed expert that hot) use TTB-wide token tiles, the rest one
// tile, in the same launch; the groups are walked from the last (the shared expert) down, so
// its long units start first and overlap the routed ones.
template <int MODE, int TTB, int KSB, int KS1>
__global__ __launch_bounds__(256) void mfma_grouped_kernel(UnitArgs x) {
  extern __shared__ u32x4 lds[];
  const int n_act = x.sel == kGroupsSharedOnly ? 0 : *x.rt.n_act;
  const int n_groups = n_act + 1;
  // the launch's groups, from the top
  const int ng = x.sel == kGroupsRoutedOnly ? n_act : n_groups;
  const int tiles = MODE == 0 ? x.I / 16 : x.H / 32;
  const int units = ng * tiles;
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int a = ng - 1 - unit / tiles;
    const int tile = unit - (ng - 1 - a) * tiles;
    const Group gr = group_of<MODE>(x, a, n_groups);
    if (gr.cnt > 16)
      staged_unit<MODE, TTB, KSB, 2, false>(x, lds, tile, 0, gr.p0, gr.cnt, gr.wbase, gr.shared);
    else
      staged_unit<MODE, 1, KS1, 2, false>(x, lds, tile, 0, gr.p0, gr.cnt, gr.wbase, gr.shared);
  }
}

// ------------------------------------------------------------------------------ dispatch
template <typename Kern>
void allow_lds_mfma(Kern kernel) {
  static thread_local const void* done[64];
  static thread_local int n_done = 0;
  for (int i = 0; i < n_done; ++i)
    if (done[i] == (const void*)kernel) return;
  (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
  if (n_done < 64) done[n_done++] = (const void*)kernel;
}

inline int token_tiles(int B) { return B <= 16 ? 1 : (B <= 32 ? 2 : 4); }

// Persistent grid: as many blocks as are resident at once (registers and LDS permitting).
template <typename Kern>
int resident_grid(const Device& d, Kern kern, size_t lds, int max_units, int* cache) {
  if (*cache == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 256, lds) != hipSuccess || n < 1) n = 1;
    *cache = n;
  }
  const int grid = d.num_cu * *cache;
  return grid > max_units ? max_units : grid;
}

template <int MODE, int TT, int KS, int NTERM, bool BF16SRC, int GSEL = 0>
hipError_t staged_t(const Device& d, const UnitArgs& x, int max_units, hipStream_t st) {
  auto kern = mfma_staged_kernel<MODE, TT, KS, NTERM, BF16SRC, GSEL>;
  constexpr size_t lds = staged_lds(TT, KS, NTERM);
  if (lds > 64 * 1024) allow_lds_mfma(kern);
  static thread_local int bpc = 0;
  hipLaunchKernelGGL(kern, dim3(resident_grid(d, kern, lds, max_units, &bpc)), dim3(256), lds, st, x);
  return hipGetLastError();
}

template <int KS, int NTERM, bool BF16SRC>
hipError_t token_split_t(const Device& d, const UnitArgs& x, hipStream_t st) {
  auto kern = mfma_token_split_kernel<KS, NTERM, BF16SRC>;
  constexpr size_t lds = staged_lds(1, KS, NTERM);
  if (lds > 64 * 1024) allow_lds_mfma(kern);
  static thread_local int bpc = 0;
  const int units = ((x.N / 32) * x.chunks + 7) / 8 * 8 * ((x.B + 15) / 16);
  hipLaunchKernelGGL(kern, dim3(resident_grid(d, kern, lds, units, &bpc)), dim3(256), lds, st, x);
  return hipGetLastError();
}

template <int TT, int KS, int NTERM, bool BF16SRC, int RTW = 2>
hipError_t tall_t(const Device& d, const UnitArgs& x, hipStream_t st) {
  constexpr int ROWS = 64 * RTW;
  if (x.N % ROWS || x.K % x.chunks || (x.K / x.chunks) % KS || x.B > 16 * TT) return hipErrorInvalidValue;
  auto kern = mfma_tall_kernel<TT, KS, NTERM, BF16SRC, RTW>;
  constexpr size_t lds = tall_lds(TT, KS, NTERM, RTW);
  if (lds > 64 * 1024) allow_lds_mfma(kern);
  static thread_local int bpc = 0;
  hipLaunchKernelGGL(kern, dim3(resident_grid(d, kern, lds, (x.N / ROWS) * x.chunks, &bpc)), dim3(256),
                     lds, st, x);
  return hipGetLastError();
}

template <int MODE, int TTB, int KSB, int KS1>
hipError_t grouped_t(const Device& d, const UnitArgs& x, int max_units, hipStream_t st) {
  auto kern = mfma_grouped_kernel<MODE, TTB, KSB, KS1>;
  constexpr size_t lds = staged_lds(TTB, KSB, 2) > staged_lds(1, KS1, 2) ? staged_lds(TTB, KSB, 2)
                                                                          : staged_lds(1, KS1, 2);
  if (lds > 64 * 1024) allow_lds_mfma(kern);
  static thread_local int bpc = 0;
  hipLaunchKernelGGL(kern, dim3(resident_grid(d, kern, lds, max_units, &bpc)), dim3(256), lds, st, x);
  return hipGetLastError();
}

// Split-K launches (one token group): stage depth 256 k for up to 32 tokens, 128 k for 64;
// KMAX caps it (K = 448).
template <int MODE, int NTERM, bool BF16SRC, int KMAX = 256>
hipError_t staged_dispatch(const Device& d, const UnitArgs& x, int max_units, hipStream_t st) {
  constexpr int K1 = KMAX < 256 ? KMAX : 256, K4 = KMAX < 128 ? KMAX : 128;
  switch (token_tiles(x.B)) {
    case 1: return staged_t<MODE, 1, K1, NTERM, BF16SRC>(d, x, max_units, st);
    case 2: return staged_t<MODE, 2, K1, NTERM, BF16SRC>(d, x, max_units, st);
    default: return staged_t<MODE, 4, K4, NTERM, BF16SRC>(d, x, max_units, st);
  }
}

// Grouped launches: up to 16 tokens, every group goes through the one-tile kernel with
// 256-k stages.  Beyond, one launch mixes one-tile units with wider ones for the groups of
// more than 16 tokens (the shared expert and any routed expert that hot).
template <int MODE, int KMAX = 256>
hipError_t grouped_dispatch(const Device& d, const UnitArgs& x, int max_units, hipStream_t st) {
  constexpr int K1 = KMAX < 256 ? KMAX : 256, K4 = KMAX < 128 ? KMAX : 128;
  if (x.B <= 16) return staged_t<MODE, 1, K1, 2, false, 0>(d, x, max_units, st);
  if (x.B <= 32) return grouped_t<MODE, 2, K1, K1>(d, x, max_units, st);
  return grouped_t<MODE, 4, K4, K1>(d, x, max_units, st);
}

}  // namespace

bool mfma_supported(const Shape& s, int B) {
  if (B < 1 || B > 64 || s.dtype != 1 || s.I != s.Is) return false;
  if (s.H != 7168 || s.E % 32 != 0) return false;
  if (!(s.Ko == 7168 || s.Ko == 448)) return false;
  return s.I == 2048 || s.I == 128;
}

// K chunks of the split-K launches (the partials the reduce / top-k launches sum).
int mfma_oproj_splits(const Shape& s) { return s.Ko == 7168 ? 7 : 1; }
bool mfma_gateup_split(const Shape& s, int B) {
  return s.I <= 256 && (B <= 16 || B > 32) && s.H % (kGateupSplits * 256) == 0;
}

bool mfma_y_by_slot(int B) { return B <= 16; }

bool mfma_swiglu_in_down(const Shape& s, int B) {
  return mfma_gateup_split(s, B) && B <= 16 && s.I == 128 && s.H % 128 == 0;
}

// Gate/up K-chunk partials of the split launches (routed and shared), or the shared expert's
// split-K partials over 32 tokens when the gate/up is not split.
size_t mfma_scratch_floats(const Shape& s, int B) {
  const size_t chunked = s.I <= 256 ? (size_t)kGateupSplits * (B * s.k + B) * 2 * s.I : 0;
  const size_t shared = (size_t)kSharedSplits * B * 2 * s.Is;
  return chunked > shared ? chunked : shared;
}
int mfma_router_splits(const Shape& s) { return 7; }

hipError_t launch_oproj_mfma(const Shape& s, const Device& d, int B, const void* x,
                             float* part, const void* w_o, hipStream_t st) {
  UnitArgs a{};
  a.w_routed = (const uint16_t*)w_o;
  a.act_routed = x;
  a.out_routed = part;
  a.B = B;
  a.N = s.H;
  a.K = s.Ko;
  a.chunks = mfma_oproj_splits(s);
  const int units = (s.H / 32) * a.chunks;
  if (s.Ko == 7168) {  // 7 x 1024 k
    // 128-row units, so that the tokens' activations are staged once per 128 weight rows and
    // each wave runs the whole K chunk for its rows (no cross-wave reduction): up to 16 tokens
    // too, where they measured 0.4-1.8 us shorter than 32-row units with K split over the waves
    (void)units;
    if (B > 32) return tall_t<4, 128, 1, true>(d, a, st);
    if (B > 16) return tall_t<2, 128, 1, true>(d, a, st);
    return tall_t<1, 128, 1, true>(d, a, st);
  }
  if (s.Ko == 448) {  // up to 32 tokens the whole 448 k in one stage (one weight round trip)
    if (B <= 16) return staged_t<2, 1, 448, 1, true>(d, a, units, st);
    if (B <= 32) return staged_t<2, 2, 448, 1, true>(d, a, units, st);
    return staged_t<2, 4, 64, 1, true>(d, a, units, st);  // 448 = 7 x 64
  }
  return hipErrorInvalidValue;
}

constexpr int kFusedRouterChunks = 8;
int mfma_fused_splits(const Shape& s) { return kFusedRouterChunks + 2; }

hipError_t launch_oproj_router_mfma(const Shape& s, const Device& d, int B, const void* x,
                                    const void* r, const void* w_o, const void* w_r,
                                    const void* mr, float* h32, float* oproj_part,
                                    float* logit_part, hipStream_t st) {
  constexpr int KS = 448;  // the 448-wide input slice in one stage; router chunks of 4 stages
  if (B > 64 || s.dtype != 1 || s.Ko != KS || s.H % (kFusedRouterChunks * KS) || s.E % 32)
    return hipErrorInvalidValue;
  MultiArgs m{};
  auto product = [&](int q, const void* w, const void* act, float* out, int N, int K, int chunks) {
    UnitArgs& a = m.p[q];
    a.w_routed = (const uint16_t*)w;
    a.act_routed = act;
    a.out_routed = out;
    a.B = B;
    a.N = N;
    a.K = K;
    a.chunks = chunks;
    m.units[q] = (N / 32) * chunks;
  };
  const size_t slot = (size_t)B * s.E;
  const int rc = kFusedRouterChunks;
  product(0, w_r, r, logit_part, s.E, s.H, rc);
  product(1, w_o, x, oproj_part, s.H, s.Ko, 1);
  m.p[1].resid = (const uint16_t*)r;
  m.p[1].h32 = h32;
  product(2, mr, x, logit_part + rc * slot, s.E, s.Ko, 1);
  product(3, (const uint16_t*)mr + (size_t)s.E * s.Ko, x, logit_part + (rc + 1) * slot, s.E, s.Ko, 1);
  const int pairs = m.units[0] + m.units[1] + m.units[2] + m.units[3];
  constexpr size_t lds = staged_lds(1, KS, 1);
  if (B <= 16) {
    auto kern = mfma_oproj_router_kernel<KS, false>;
    if (lds > 64 * 1024) allow_lds_mfma(kern);
    static thread_local int bpc = 0;
    hipLaunchKernelGGL(kern, dim3(resident_grid(d, kern, lds, pairs, &bpc)), dim3(256), lds, st, m);
  } else {
    auto kern = mfma_oproj_router_kernel<KS, true>;
    if (lds > 64 * 1024) allow_lds_mfma(kern);
    static thread_local int bpc = 0;
    const int units = (pairs + 7) / 8 * 8 * ((B + 15) / 16);
    hipLaunchKernelGGL(kern, dim3(resident_grid(d, kern, lds, units, &bpc)), dim3(256), lds, st, m);
  }
  return hipGetLastError();
}

hipError_t launch_oproj_reduce(const Shape& s, int B, const float* part, const void* r,
                               float* h32, void* h_out, hipStream_t st) {
  const int n = B * s.H;
  hipLaunchKernelGGL((oproj_reduce_kernel<uint16_t, 8>), dim3((n + 255) / 256), dim3(256), 0, st,
                     part, mfma_oproj_splits(s), (const uint16_t*)r, B, s.H, h32, (uint16_t*)h_out);
  return hipGetLastError();
}

hipError_t launch_norm_rows(const Shape& s, int B, const float* part, const void* r, float* h32,
                            void* h_out, const Norm& nm, float* u32, hipStream_t st) {
  constexpr int MAXS = 8, MAXJ = 8;
  const int threads = s.H >= 1024 ? 1024 : (s.H + 63) / 64 * 64;
  if (!nm.gamma || s.H % 4 || s.H > MAXJ * threads || (part && mfma_oproj_splits(s) > MAXS))
    return hipErrorInvalidValue;
  const int splits = part ? mfma_oproj_splits(s) : 1;
  if (s.dtype == 1)
    hipLaunchKernelGGL((norm_rows_kernel<uint16_t, MAXS, MAXJ>), dim3(B), dim3(threads), 0, st,
                       part, splits, (const uint16_t*)r, B, s.H, h32, (uint16_t*)h_out,
                       (const uint16_t*)nm.gamma, nm.eps, u32);
  else
    hipLaunchKernelGGL((norm_rows_kernel<float, MAXS, MAXJ>), dim3(B), dim3(threads), 0, st,
                       part, splits, (const float*)r, B, s.H, h32, (float*)h_out,
                       (const float*)nm.gamma, nm.eps, u32);
  return hipGetLastError();
}

hipError_t launch_router_mfma(const Shape& s, const Device& d, int B, const float* h32,
                              const void* w_r, float* part, hipStream_t st) {
  UnitArgs a{};
  a.w_routed = (const uint16_t*)w_r;
  a.act_routed = h32;
  a.out_routed = part;
  a.B = B;
  a.N = s.E;
  a.K = s.H;
  a.chunks = mfma_router_splits(s);  // 7 x 1024 k
  // over 16 tokens the 12 x 7 (row tile, chunk) units alone would leave most of the chip idle
  if (B > 16) return token_split_t<256, 3, false>(d, a, st);
  return staged_dispatch<2, 3, false>(d, a, (s.E / 32) * a.chunks, st);
}

hipError_t launch_gateup_mfma(const Shape& s, const Device& d, int B, const float* h32,
                              const void* w13, const void* ws13, const Routing& rt, float* A,
                              float* As, float* scratch, hipStream_t st, int sel) {
  const bool routed = sel != kGroupsSharedOnly, shared = sel != kGroupsRoutedOnly;
  UnitArgs a{};
  a.sel = sel;
  a.w_routed = (const uint16_t*)w13;
  a.w_shared = (const uint16_t*)ws13;
  a.act_routed = h32;
  a.act_shared = h32;
  a.out_routed = A;
  a.out_shared = As;
  a.H = s.H;
  a.I = s.I;
  a.k = s.k;
  a.B = B;
  a.rt = rt;
  const int max_units = ((s.E < B * s.k ? s.E : B * s.k) + 1) * (s.I / 16);
  const bool split = mfma_gateup_split(s, B);
  const int nslot = B * s.k;
  auto reduce = [&](const SwigluRegion& r0, const SwigluRegion& r1) {
    const int n = (r0.rows + r1.rows) * s.I;
    if (n == 0) return hipSuccess;
    if (r0.chunks > 8 || r1.chunks > 8)
      hipLaunchKernelGGL((swiglu_reduce_kernel<16>), dim3((n + 255) / 256), dim3(256), 0, st, r0,
                         r1, s.I);
    else
      hipLaunchKernelGGL((swiglu_reduce_kernel<8>), dim3((n + 255) / 256), dim3(256), 0, st, r0,
                         r1, s.I);
    return hipGetLastError();
  };
  if (split) {
    // every group over K chunks (the shared expert's tokens at positions nslot ..), then the
    // SwiGLU of the summed chunks: up to 16 tokens one unit per (group, tile, chunk); over 32
    // the routed experts cut into pieces of at most 16 positions and the shared expert's
    // tokens in pieces of 16
    a.gu_part = scratch;
    a.gu_P = nslot + B;
    a.chunks = kGateupSplits;
    const int piece_units = (s.E + nslot / 16 + (B + 15) / 16) * (s.I / 16) * kGateupSplits;
    hipError_t e = B <= 16 ? staged_t<0, 1, 256, 2, false, 0>(d, a, max_units * kGateupSplits, st)
                           : staged_t<0, 1, 256, 2, false, 5>(d, a, piece_units, st);
    if (e != hipSuccess) return e;
    if (mfma_swiglu_in_down(s, B)) return hipSuccess;  // the down-projection sums the chunks
    const size_t cs = (size_t)a.gu_P * 2 * s.I;
    return reduce(SwigluRegion{scratch, cs, routed ? nslot : 0, kGateupSplits, A},
                  SwigluRegion{scratch + (size_t)nslot * 2 * s.I, cs, shared ? B : 0,
                               kGateupSplits, As});
  }
  if (B > 16 && B <= 32) {
    // every routed expert and the shared one cut into pieces of 16 positions, one-tile units
    const int units = (s.E + B * s.k / 16 + (B + 15) / 16) * (s.I / 16);
    return staged_t<0, 1, 256, 2, false, 5>(d, a, units, st);
  }
  if (B <= 16) return grouped_dispatch<0>(d, a, max_units, st);
  // over 32 tokens (not split) the shared expert's gate/up is a split-K product of its own
  // (its group alone has too few row tiles to fill the chip) with 128-row units; then every
  // routed expert, hot ones cut into pieces of 16 positions, in one one-tile launch, and one
  // launch applies the SwiGLU to the shared partials
  UnitArgs sh{};
  sh.w_routed = (const uint16_t*)ws13;
  sh.act_routed = h32;
  sh.out_routed = scratch;
  sh.B = B;
  sh.N = 2 * s.Is;
  sh.K = s.H;
  sh.chunks = kSharedSplits;
  hipError_t e = shared ? tall_t<4, 128, 2, false>(d, sh, st) : hipSuccess;
  if (e != hipSuccess) return e;
  const int units = (s.E + nslot / 16 + 1) * (s.I / 16);
  e = routed ? staged_t<0, 1, 256, 2, false, 4>(d, a, units, st) : hipSuccess;
  if (e != hipSuccess) return e;
  return reduce(SwigluRegion{scratch, 0, 0, 1, A},
                SwigluRegion{scratch, (size_t)B * 2 * s.Is, shared ? B : 0, kSharedSplits, As});
}

hipError_t launch_down_mfma(const Shape& s, const Device& d, int B, const float* A,
                            const float* As, const void* w2, const void* ws2, const Routing& rt,
                            float* Y, float* ys, const float* gu_part, hipStream_t st, int sel) {
  UnitArgs a{};
  a.sel = sel;
  if (mfma_swiglu_in_down(s, B)) {
    a.gu_part = const_cast<float*>(gu_part);
    a.gu_P = B * s.k + B;
  }
  a.y_by_slot = mfma_y_by_slot(B);
  a.w_routed = (const uint16_t*)w2;
  a.w_shared = (const uint16_t*)ws2;
  a.act_routed = A;
  a.act_shared = As;
  a.out_routed = Y;
  a.out_shared = ys;
  a.H = s.H;
  a.I = s.I;
  a.k = s.k;
  a.B = B;
  a.rt = rt;
  const int max_units = ((s.E < B * s.k ? s.E : B * s.k) + 1) * (s.H / 32);
  if (s.I == 2048) return grouped_dispatch<1>(d, a, max_units, st);
  if (s.I == 128 && s.H % 128 == 0) {
    auto kern = mfma_down_shortk_kernel<128>;
    constexpr size_t lds = (size_t)(128 * (128 / 8 + 1) + 2 * 16 * (128 / 8 + 1)) * 16;
    static thread_local int bpc = 0;
    const int units = ((s.E < B * s.k ? s.E : B * s.k) + 1) * (s.H / 128);
    hipLaunchKernelGGL(kern, dim3(resident_grid(d, kern, lds, units, &bpc)), dim3(256), lds, st, a);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace kk

// Router tail shared by both paths: logits (sum of K-slice partials) -> sigmoid scores ->
// fp64 selection keys -> top-k by wavefront arg-max rounds (DPP) -> renormalised gates ->
// token->expert permutation and expert offsets by prefix sum.
//
// "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly", section "Recovering time
// between operators" (router scores in MoE preparation).  Reading of the unstated math:
// sigmoid scores, selection on score + per-expert bias (lower index first on equal keys;
// a key is formed in fp64 as (1 + bias) - sigmoid(-logit), the sigmoid taken in fp32, and
// ranked on its value truncated to 43 mantissa bits),
// gates = selected unbiased scores / their sum * routed_scale, experts of a token listed in
// ascending index; perm orders slots (t*k + j) by (expert, token).
#pragma once

#include "kk_common.cuh"
#include "kk_internal.h"

namespace kk {

constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 16;
constexpr int kMaxSlots = 64 * kMaxTopK;  // max batch * max top-k

struct TopkScratch {
  int sel[kMaxSlots];                      // selected expert of each slot
  unsigned long long mask[kMaxExperts];    // bit t set: token t routed to expert e
  int start[kMaxExperts];                  // exclusive prefix sum of counts
};

// Order-preserving 64-bit image of a double (larger key -> larger integer), with the low 9
// bits replaced by (511 - e) so that one integer maximum picks the largest key and, among
// keys equal to 43 mantissa bits, the lowest expert index.
__device__ __forceinline__ uint64_t rank_key(double key, int e) {
  uint64_t u = (uint64_t)__double_as_longlong(key);
  u = (u >> 63) ? ~u : (u | (1ull << 63));
  return (u & ~0x1FFull) | (uint64_t)(511 - e);
}

// One token's selection on one wave from its logits and the bias (lane l holds expert
// l + 64 m in l_[m] and bv[m]): sigmoid scores, fp64 keys, then k rounds of wave arg-max,
// renormalised gates; topk_idx / topk_gate rows written in ascending expert order, and the
// selected experts returned through sel (nullable).  Each lane sorts its packed keys once
// (descending), so a round reduces only the lanes' heads and the winner pops its own.
constexpr int kMaxM = kMaxExperts / 64;
__device__ inline void topk_select(const float (&l_)[kMaxM], const float (&bv)[kMaxM], int E, int k,
                                   float routed_scale, int t, const Routing& rt, int* sel) {
  const int lane = threadIdx.x & 63;
  double sc[kMaxM];
  uint64_t rk[kMaxM];
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) {
    sc[m] = 0.0;
    rk[m] = 0ull;
    if (64 * m < E) {  // uniform: slots past the last expert cost nothing
      const int e = lane + 64 * m;
      // t = 1 - s = sigmoid(-l) in fp32 keeps its relative precision where s saturates
      // towards 1; the score and the key are then formed in fp64
      const float t = 1.0f / (1.0f + expf(l_[m]));
      sc[m] = 1.0 - (double)t;
      rk[m] = e < E ? rank_key((1.0 + (double)bv[m]) - (double)t, e) : 0ull;
    }
  }
  // per-lane sort, descending (19-comparator odd-even merge network over 8 keys)
  uint64_t sk[kMaxM];
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) sk[m] = rk[m];
  static_assert(kMaxM == 8, "the sorting network is written for 8 keys per lane");
  auto ce = [&](int i, int j) {
    const uint64_t a = sk[i], b = sk[j];
    const bool sw = b > a;
    sk[i] = sw ? b : a;
    sk[j] = sw ? a : b;
  };
  ce(0, 1); ce(2, 3); ce(4, 5); ce(6, 7);
  ce(0, 2); ce(1, 3); ce(4, 6); ce(5, 7);
  ce(1, 2); ce(5, 6);
  ce(0, 4); ce(1, 5); ce(2, 6); ce(3, 7);
  ce(2, 4); ce(3, 5);
  ce(1, 2); ce(3, 4); ce(5, 6);
  // k rounds: the wave maximum of the heads wins; its lane drops it.  The high words decide
  // unless several heads share the maximal one; only then are their low words compared.
  uint32_t selmask = 0;
  for (int r = 0; r < k; ++r) {
    const uint32_t hi = (uint32_t)(sk[0] >> 32), lo = (uint32_t)sk[0];
    const uint32_t mh = wave_max_u32(hi);
    const uint64_t tied = __ballot(hi == mh);
    const uint32_t ml = __popcll(tied) == 1
                            ? (uint32_t)__builtin_amdgcn_readlane((int)lo, __builtin_ctzll(tied))
                            : wave_max_u32(hi == mh ? lo : 0u);
    const int win = 511 - (int)(ml & 0x1FFu);
    const bool mine = (win & 63) == lane;
    if (mine) selmask |= 1u << (win >> 6);
#pragma unroll
    for (int m = 0; m < kMaxM - 1; ++m) sk[m] = mine ? sk[m + 1] : sk[m];
    sk[kMaxM - 1] = mine ? 0ull : sk[kMaxM - 1];
  }
  double ssum = 0.0;
#pragma unroll
  for (int m = 0; m < kMaxM; ++m)
    if ((selmask >> m) & 1u) ssum += sc[m];
  ssum = wave_sum_f64_dpp(ssum);
  const double gscale = (double)routed_scale / ssum;
  int base = 0;
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) {
    const bool on = (selmask >> m) & 1u;
    const unsigned long long bal = __ballot(on);
    if (on) {
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      const int e = lane + 64 * m;
      rt.topk_idx[t * k + pos] = e;
      rt.topk_gate[t * k + pos] = (float)(sc[m] * gscale);
      if (sel) sel[t * k + pos] = e;
    }
    base += __popcll(bal);
  }
}

// The bias of this lane's experts (lane l: expert l + 64 m), clamped loads.
__device__ __forceinline__ void load_bias(const float* __restrict__ bias, int E, float (&bv)[kMaxM]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) bv[m] = bias[min(lane + 64 * m, E - 1)];
}

// One token's top-k on one wave from logit partials part[splits][B][E] (splits <=
// kMaxTopkSplits), summed in slice order.  All global loads (partials and bias) are issued
// before any is used (addresses clamped instead of branched around, so nothing waits on a
// join).
constexpr int kMaxTopkSplits = 10;
__device__ __forceinline__ void topk_row(const float* part, int splits, const float* __restrict__ bias,
                                int B, int E, int k, float routed_scale, int t, const Routing& rt,
                                int* sel) {
  constexpr int MAXS = kMaxTopkSplits;
  const int lane = threadIdx.x & 63;
  float pv[kMaxM][MAXS], bv[kMaxM];
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) {
    const int ec = min(lane + 64 * m, E - 1);
#pragma unroll
    for (int s = 0; s < MAXS; ++s) pv[m][s] = part[((size_t)min(s, splits - 1) * B + t) * E + ec];
  }
  load_bias(bias, E, bv);
  float l_[kMaxM];
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) {
    float l = 0.f;
#pragma unroll
    for (int s = 0; s < MAXS; ++s) l += s < splits ? pv[m][s] : 0.f;
    l_[m] = l;
  }
  topk_select(l_, bv, E, k, routed_scale, t, rt, sel);
}

// Block-wide: logits lg[t * E + e] of all B tokens summed from part[splits][B][E] in slice
// order (B * E <= 2 * blockDim.x), each thread's loads all in flight together.
__device__ inline void logits_to_lds(const float* part, int splits, int B, int E, float* lg) {
  constexpr int MAXS = kMaxTopkSplits;
  const int n = B * E;
  float pv[2][MAXS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = min((int)(threadIdx.x + j * blockDim.x), n - 1);
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      pv[j][s] = part[(size_t)min(s, splits - 1) * n + i];
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    float l = 0.f;
#pragma unroll
    for (int s = 0; s < MAXS; ++s) l += s < splits ? pv[j][s] : 0.f;
    if (i < n) lg[i] = l;
  }
}

// One token's top-k on one wave from its logits in LDS; bv holds the lane's bias values.
__device__ inline void topk_row_lds(const float* lg, const float (&bv)[kMaxM], int E, int k,
                                    float routed_scale, int t, const Routing& rt, int* sel) {
  const int lane = threadIdx.x & 63;
  float l_[kMaxM];
#pragma unroll
  for (int m = 0; m < kMaxM; ++m) l_[m] = lg[t * E + min(lane + 64 * m, E - 1)];
  topk_select(l_, bv, E, k, routed_scale, t, rt, sel);
}

// Routing tables from the selected experts of all B tokens (sm.sel filled, block-wide):
// per-expert token masks, counts, exclusive prefix sum -> offsets, active list, n_act, perm
// (slots by (expert, token)) and its inverse.
__device__ inline void build_tables(int B, int E, int k, const Routing& rt, TopkScratch& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (B == 1) {
    // one token: its k experts (ascending, one slot each) are the active list in order, and
    // positions are slots
    int sv[kMaxTopK];  // the selected experts in registers (k <= kMaxTopK)
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) sv[j] = j < k ? sm.sel[j] : 0x7fffffff;
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
      int c = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) c += sv[j] < e ? 1 : 0;
      rt.offsets[e] = c;
    }
    for (int j = threadIdx.x; j < k; j += blockDim.x) {
      rt.act[j] = sm.sel[j];
      rt.perm[j] = j;
      rt.inv_perm[j] = j;
      if (rt.vg) rt.vg[j] = j << 2;
    }
    if (threadIdx.x == 0) {
      *rt.n_act = k;
      if (rt.n_vg) *rt.n_vg = k;
    }
    return;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) sm.mask[e] = 0ull;
  __syncthreads();
  for (int i = threadIdx.x; i < B * k; i += blockDim.x)
    atomicOr(&sm.mask[sm.sel[i]], 1ull << (i / k));
  __syncthreads();
  if (wave == 0) {
    // lane l owns experts l*per .. l*per+per-1 (per <= kMaxM); their counts (<= 64) are read
    // from the masks once.  Counts and active flags are scanned together as
    // (count | flag << 16), and the pieces of at most 16 positions in a second scan.
    const int per = (E + 63) / 64;
    uint32_t cnt[kMaxM];
    uint32_t loc = 0, vt = 0;
#pragma unroll
    for (int q = 0; q < kMaxM; ++q) {
      const int e = lane * per + q;
      cnt[q] = q < per && e < E ? (uint32_t)__popcll(sm.mask[e]) : 0u;
      loc += cnt[q] | ((cnt[q] > 0 ? 1u : 0u) << 16);
      vt += (cnt[q] + 15u) >> 4;
    }
    const uint32_t inc = wave_incl_scan_u32(loc);
    const uint32_t vinc = rt.vg ? wave_incl_scan_u32(vt) : 0u;
    uint32_t ec = (inc - loc) & 0xFFFFu, ef = (inc - loc) >> 16, vpos = vinc - vt;
#pragma unroll
    for (int q = 0; q < kMaxM; ++q) {
      const int e = lane * per + q;
      if (q < per && e < E) {
        sm.start[e] = (int)ec;
        rt.offsets[e] = (int)ec;
        ec += cnt[q];
        if (cnt[q] > 0) {
          if (rt.vg) {
#pragma unroll
            for (uint32_t pc = 0; pc < 4; ++pc)
              if (16u * pc < cnt[q]) rt.vg[vpos++] = (int)((ef << 2) | pc);
          }
          rt.act[ef++] = e;
        }
      }
    }
    if (lane == 63) {
      rt.offsets[E] = (int)(inc & 0xFFFFu);
      *rt.n_act = (int)(inc >> 16);
      if (rt.n_vg) *rt.n_vg = (int)vinc;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B * k; i += blockDim.x) {
    const int t = i / k, e = sm.sel[i];
    const int p = sm.start[e] + __popcll(sm.mask[e] & ((1ull << t) - 1ull));
    rt.perm[p] = i;
    rt.inv_perm[i] = p;
  }
}

}  // namespace kk

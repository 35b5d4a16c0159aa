// Router tail shared by both paths: logits (sum of K-slice partials) -> sigmoid scores ->
// fp64 selection keys -> top-k by wavefront arg-max rounds -> renormalised gates ->
// token->expert permutation and expert offsets by prefix sum.  Runs in one block.
//
// "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly", section "Recovering time
// between operators" (router scores in MoE preparation).  Reading of the unstated math:
// sigmoid scores, selection on score + per-expert bias (lower index first on equal keys),
// gates = selected unbiased scores / their sum * routed_scale, experts of a token listed in
// ascending index; perm orders slots (t*k + j) by (expert, token).
#pragma once

#include "kk_common.cuh"
#include "kk_internal.h"

namespace kk {

constexpr int kMaxExperts = 512;
constexpr int kMaxSlots = 64 * 16;  // max batch * max top-k

struct TopkScratch {
  int sel[kMaxSlots];                      // selected expert of each slot
  unsigned long long mask[kMaxExperts];    // bit t set: token t routed to expert e
  int start[kMaxExperts];                  // exclusive prefix sum of counts
};

// part: [splits][B][E] fp32 logit partials, summed in slice order.  blockDim.x >= 64.
__device__ inline void topk_tables(const float* part, int splits, const float* __restrict__ bias,
                                   int B, int E, int k, float routed_scale, const Routing& rt,
                                   TopkScratch& sm) {
  constexpr int MAXM = kMaxExperts / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const double kNegInf = -__builtin_huge_val();
  for (int e = threadIdx.x; e < E; e += blockDim.x) sm.mask[e] = 0ull;

  for (int t = wave; t < B; t += nw) {
    double key[MAXM], sc[MAXM];
    bool sel[MAXM];
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      const int e = lane + 64 * m;
      sel[m] = false;
      key[m] = kNegInf;
      sc[m] = 0.0;
      if (e < E) {
        float l = 0.f;
        for (int s = 0; s < splits; ++s) l += part[((size_t)s * B + t) * E + e];
        const double sv = 1.0 / (1.0 + exp(-(double)l));
        sc[m] = sv;
        key[m] = sv + (double)bias[e];
      }
    }
    for (int r = 0; r < k; ++r) {
      double bk = kNegInf;
      int bi = 0x7fffffff;
#pragma unroll
      for (int m = 0; m < MAXM; ++m) {  // ascending index: strict > keeps the lower one
        const int e = lane + 64 * m;
        if (e < E && !sel[m] && key[m] > bk) {
          bk = key[m];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double ok = __shfl_xor(bk, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (ok > bk || (ok == bk && oi < bi)) {
          bk = ok;
          bi = oi;
        }
      }
#pragma unroll
      for (int m = 0; m < MAXM; ++m)
        if (lane + 64 * m == bi) sel[m] = true;
    }
    double ssum = 0.0;
#pragma unroll
    for (int m = 0; m < MAXM; ++m)
      if (sel[m]) ssum += sc[m];
    ssum = wave_sum_f64(ssum);
    int base = 0;
#pragma unroll
    for (int m = 0; m < MAXM; ++m) {
      const unsigned long long bal = __ballot(sel[m]);
      if (sel[m]) {
        const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
        const int e = lane + 64 * m;
        rt.topk_idx[t * k + pos] = e;
        rt.topk_gate[t * k + pos] = (float)((double)routed_scale * sc[m] / ssum);
        sm.sel[t * k + pos] = e;
      }
      base += __popcll(bal);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B * k; i += blockDim.x)
    atomicOr(&sm.mask[sm.sel[i]], 1ull << (i / k));
  __syncthreads();
  if (wave == 0) {
    const int per = (E + 63) / 64;
    int lc = 0, lf = 0;
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      if (e < E) {
        const int c = __popcll(sm.mask[e]);
        lc += c;
        lf += c > 0;
      }
    }
    int ic = lc, jf = lf;
    for (int off = 1; off < 64; off <<= 1) {
      const int vc = __shfl_up(ic, off, 64);
      const int vf = __shfl_up(jf, off, 64);
      if (lane >= off) {
        ic += vc;
        jf += vf;
      }
    }
    int ec = ic - lc, ef = jf - lf;
    for (int q = 0; q < per; ++q) {
      const int e = lane * per + q;
      if (e < E) {
        const int c = __popcll(sm.mask[e]);
        sm.start[e] = ec;
        rt.offsets[e] = ec;
        if (c > 0) rt.act[ef++] = e;
        ec += c;
      }
    }
    if (lane == 63) {
      rt.offsets[E] = ic;
      *rt.n_act = jf;
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

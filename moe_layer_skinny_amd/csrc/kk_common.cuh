// Device helpers shared by the kernels of the decode-layer step (gfx950, wave64).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kk {

constexpr int kWave = 64;

// One 16-byte chunk of a weight row (a native vector, so it loads as one dwordx4).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Element traits of the weight / activation storage type.  A "chunk" is 16 bytes.
template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 bit patterns
  static constexpr int EPC = 8;
  __device__ static __forceinline__ void unpack(const u32x4& w, float (&f)[8]) {
    f[0] = bf_lo(w.x);
    f[1] = bf_hi(w.x);
    f[2] = bf_lo(w.y);
    f[3] = bf_hi(w.y);
    f[4] = bf_lo(w.z);
    f[5] = bf_hi(w.z);
    f[6] = bf_lo(w.w);
    f[7] = bf_hi(w.w);
  }
  __device__ static __forceinline__ float load(const uint16_t* p, size_t i) {
    return __uint_as_float((uint32_t)p[i] << 16);
  }
  __device__ static __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
  // elements i..i+3 (i % 4 == 0)
  __device__ static __forceinline__ float4 load4(const uint16_t* p, size_t i) {
    const uint2 w = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y));
  }
};

template <>
struct Elem<float> {
  static constexpr int EPC = 4;
  __device__ static __forceinline__ void unpack(const u32x4& w, float (&f)[4]) {
    f[0] = __uint_as_float(w.x);
    f[1] = __uint_as_float(w.y);
    f[2] = __uint_as_float(w.z);
    f[3] = __uint_as_float(w.w);
  }
  __device__ static __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
  __device__ static __forceinline__ float4 load4(const float* p, size_t i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
};

// Sum over the SEG lanes of each aligned lane segment (SEG a power of two <= 64).
template <int SEG>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int off = SEG / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, SEG);
  return v;
}

// Weight-row geometry of a GEMV over rows of CPR 16-byte chunks.  A wave covers RPW rows
// at once, SEG lanes per row (SEG = 64 for rows of >= 33 chunks); lane `sub` of a segment
// holds chunks sub, sub + SEG, ... (CPL of them), so every wave-wide load instruction
// reads whole rows' contiguous 16-byte pieces.
template <typename T, int CPR>
struct Geo {
  static constexpr int EPC = Elem<T>::EPC;
  static constexpr int SEG = CPR > 32 ? 64 : (CPR > 16 ? 32 : 16);
  static constexpr int RPW = kWave / SEG;
  static constexpr int CPL = (CPR + SEG - 1) / SEG;
  static constexpr int K = CPR * EPC;  // elements per row
  static constexpr bool EXACT = (CPR % SEG) == 0;
};

template <typename T, int CPR>
__device__ __forceinline__ void load_row(const T* __restrict__ row, int sub,
                                         u32x4 (&w)[Geo<T, CPR>::CPL]) {
  using G = Geo<T, CPR>;
  const u32x4* p = reinterpret_cast<const u32x4*>(row);
#pragma unroll
  for (int i = 0; i < G::CPL; ++i) {
    const int c = sub + G::SEG * i;
    if (G::EXACT || c < CPR)
      w[i] = __builtin_nontemporal_load(p + c);
    else
      w[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Lane-partial dot of the loaded row chunks with an fp32 activation row held in LDS.
template <typename T, int CPR>
__device__ __forceinline__ float dot_lane(const u32x4 (&w)[Geo<T, CPR>::CPL], const float* act,
                                          int sub) {
  using G = Geo<T, CPR>;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < G::CPL; ++i) {
    const int c = sub + G::SEG * i;
    if (G::EXACT || c < CPR) {
      float f[G::EPC];
      Elem<T>::unpack(w[i], f);
      const float4* a = reinterpret_cast<const float4*>(act + c * G::EPC);
#pragma unroll
      for (int q = 0; q < G::EPC / 4; ++q) {
        const float4 av = a[q];
        acc = fmaf(f[4 * q + 0], av.x, acc);
        acc = fmaf(f[4 * q + 1], av.y, acc);
        acc = fmaf(f[4 * q + 2], av.z, acc);
        acc = fmaf(f[4 * q + 3], av.w, acc);
      }
    }
  }
  return acc;
}

// Lane-partial dot of loaded row chunks with an activation row held in registers as raw
// chunks of the same element type (the lane's own chunk positions).
template <typename T, int CPR>
__device__ __forceinline__ float dot_rr(const u32x4 (&w)[Geo<T, CPR>::CPL],
                                        const u32x4 (&x)[Geo<T, CPR>::CPL], int sub) {
  using G = Geo<T, CPR>;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < G::CPL; ++i) {
    const int c = sub + G::SEG * i;
    if (G::EXACT || c < CPR) {
      float f[G::EPC], a[G::EPC];
      Elem<T>::unpack(w[i], f);
      Elem<T>::unpack(x[i], a);
#pragma unroll
      for (int q = 0; q < G::EPC; ++q) acc = fmaf(f[q], a[q], acc);
    }
  }
  return acc;
}

// The lane's chunks of one activation row (plain loads: activations are read many times).
template <typename T, int CPR>
__device__ __forceinline__ void load_act_chunks(const T* __restrict__ row, int sub,
                                                u32x4 (&x)[Geo<T, CPR>::CPL]) {
  using G = Geo<T, CPR>;
  const u32x4* p = reinterpret_cast<const u32x4*>(row);
#pragma unroll
  for (int i = 0; i < G::CPL; ++i) {
    const int c = sub + G::SEG * i;
    x[i] = (G::EXACT || c < CPR) ? p[c] : u32x4{0u, 0u, 0u, 0u};
  }
}

// ---- wavefront reductions with DPP lane moves (VALU latency instead of the LDS crossbar).
// DPP controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror =
// 0x141, row_mirror = 0x140, row_bcast15 = 0x142 (rows 1, 3), row_bcast31 = 0x143 (rows
// 2, 3), row_shr:n = 0x110 + n.  After the six combining steps lane 63 holds the result.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Maximum of v over the 64 lanes, returned to every lane: each step is one DPP-fed max
// (lanes outside a step's rows combine with 0, the identity); lane 63 ends with the total.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum of v over the 64 lanes in a fixed combining order, returned to every lane.
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  auto step = [](double x, uint64_t moved) { return x + __longlong_as_double((long long)moved); };
  v = step(v, dpp_u64<0xB1>((uint64_t)__double_as_longlong(v)));
  v = step(v, dpp_u64<0x4E>((uint64_t)__double_as_longlong(v)));
  v = step(v, dpp_u64<0x141>((uint64_t)__double_as_longlong(v)));
  v = step(v, dpp_u64<0x140>((uint64_t)__double_as_longlong(v)));
  // rows 1 and 3 add their left neighbour row's total; rows 0 and 2 add nothing
  {
    const uint64_t bits = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)bits, 0x142, 0xA, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(bits >> 32), 0x142, 0xA, 0xF, false);
    v += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  }
  {
    const uint64_t bits = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)bits, 0x143, 0xC, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(bits >> 32), 0x143, 0xC, 0xF, false);
    v += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  }
  return __longlong_as_double((long long)readlane_u64((uint64_t)__double_as_longlong(v), 63));
}

// Sum of v over each segment of SEG lanes (16, 32 or 64) in a fixed combining order, valid in
// the segment's last lane (lane % SEG == SEG - 1).  Four steps give every lane of a row of 16
// its row total; rows 1 and 3 then add the total of the row before them, and row 3 the total
// of rows 0-1.
template <int SEG>
__device__ __forceinline__ float seg_sum_dpp(float v) {
  static_assert(SEG == 16 || SEG == 32 || SEG == 64, "segments of 16, 32 or 64 lanes");
  auto mv = [](float x, auto ctrl_tag) {
    constexpr int C = decltype(ctrl_tag)::value;
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), C, 0xF, 0xF, false));
  };
  v += mv(v, std::integral_constant<int, 0xB1>{});
  v += mv(v, std::integral_constant<int, 0x4E>{});
  v += mv(v, std::integral_constant<int, 0x141>{});
  v += mv(v, std::integral_constant<int, 0x140>{});
  if (SEG >= 32) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
  if (SEG >= 64) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
  return v;
}

// Inclusive prefix sum of v over lanes 0..63 (Hillis-Steele within rows of 16, then the
// row totals carried across rows).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
  return v;
}

// Gate and up rows against the same activation row: each activation chunk is read from
// LDS once and feeds both sums.
template <typename T, int CPR>
__device__ __forceinline__ void dot2_lane(const u32x4 (&wa)[Geo<T, CPR>::CPL],
                                          const u32x4 (&wb)[Geo<T, CPR>::CPL], const float* act,
                                          int sub, float& sa, float& sb) {
  using G = Geo<T, CPR>;
  float a0 = 0.f, b0 = 0.f;
#pragma unroll
  for (int i = 0; i < G::CPL; ++i) {
    const int c = sub + G::SEG * i;
    if (G::EXACT || c < CPR) {
      float fa[G::EPC], fb[G::EPC];
      Elem<T>::unpack(wa[i], fa);
      Elem<T>::unpack(wb[i], fb);
      const float4* a = reinterpret_cast<const float4*>(act + c * G::EPC);
#pragma unroll
      for (int q = 0; q < G::EPC / 4; ++q) {
        const float4 av = a[q];
        a0 = fmaf(fa[4 * q + 0], av.x, a0);
        b0 = fmaf(fb[4 * q + 0], av.x, b0);
        a0 = fmaf(fa[4 * q + 1], av.y, a0);
        b0 = fmaf(fb[4 * q + 1], av.y, b0);
        a0 = fmaf(fa[4 * q + 2], av.z, a0);
        b0 = fmaf(fb[4 * q + 2], av.z, b0);
        a0 = fmaf(fa[4 * q + 3], av.w, a0);
        b0 = fmaf(fb[4 * q + 3], av.w, b0);
      }
      // keep the LDS reads chunk by chunk: hoisting them all would double the live registers
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  sa = a0;
  sb = b0;
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// ---- MFMA operands (v_mfma_f32_16x16x32_bf16) ----------------------------------------
// A: 16 rows x 32 k, B: 32 k x 16 columns, D: 16 x 16 fp32.  Lane l holds row (column)
// l % 16 and k = 8 * (l / 16) + e of each operand; of D it holds rows 4 * (l / 16) + i,
// column l % 16.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}


typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 (a in the low half), round to nearest even: gfx950's
// v_cvt_pk_bf16_f32, the same bits as f32_to_bf16 for every non-NaN input.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// 8 fp32 values -> NTERM bf16 vectors (RNE), each term the rounding of what the previous
// ones left over; the differences are exact in fp32.
template <int NTERM>
__device__ __forceinline__ void split_terms(const float (&x)[8], u32x4 (&out)[NTERM]) {
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e];
#pragma unroll
  for (int q = 0; q < NTERM; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = pack_bf16x2(r[2 * e], r[2 * e + 1]);
      if (q + 1 < NTERM) {
        r[2 * e] -= __uint_as_float(w[e] << 16);
        r[2 * e + 1] -= __uint_as_float(w[e] & 0xffff0000u);
      }
    }
    out[q] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

}  // namespace kk

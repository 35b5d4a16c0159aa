// Seeded synthetic inputs, device side: fills a device buffer with the same
// Philox4x32-10 stream as philox_host.c (Salmon et al., SC'11, section 3.2),
// element n from counter (n_lo, n_hi, 0, 0) under key (key0, key1), turned into
// one standard normal draw by the Box-Muller transform (Box and Muller, 1958),
// scaled by sigma in double, rounded to fp32 (RNE) and, for bf16, to bf16 (RNE).
// The logarithm, square root and cosine are the same +, -, *, / sequences as on
// the host (IEEE double operations, each rounded on its own: this file is built
// with -ffp-contract=off and the pragma below, so none is fused), hence the same
// bits.  Used to place the ~34 GB of routed-expert weights in HBM without a host
// round trip.  Holds no arithmetic of the decode layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u;
constexpr uint32_t kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u;
constexpr uint32_t kW1 = 0xBB67AE85u;

__device__ __forceinline__ void philox10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                         uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kW0;
      k1 += kW1;
    }
    uint32_t hi0 = __umulhi(kM0, c0), lo0 = kM0 * c0;
    uint32_t hi1 = __umulhi(kM1, c2), lo1 = kM1 * c2;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
}

#pragma clang fp contract(off)

// ln m = 2 s sum_j s^2j / (2j + 1), s = (m - 1) / (m + 1); sin / cos Taylor series.
__constant__ const double kAtanh[12] = {
    0x1.0000000000000p+0, 0x1.5555555555555p-2, 0x1.999999999999ap-3, 0x1.2492492492492p-3,
    0x1.c71c71c71c71cp-4, 0x1.745d1745d1746p-4, 0x1.3b13b13b13b14p-4, 0x1.1111111111111p-4,
    0x1.e1e1e1e1e1e1ep-5, 0x1.af286bca1af28p-5, 0x1.8618618618618p-5, 0x1.642c8590b2164p-5};
__constant__ const double kSin[11] = {
    0x1.0000000000000p+0, -0x1.5555555555555p-3, 0x1.1111111111111p-7, -0x1.a01a01a01a01ap-13,
    0x1.71de3a556c734p-19, -0x1.ae64567f544e4p-26, 0x1.6124613a86d09p-33, -0x1.ae7f3e733b81fp-41,
    0x1.952c77030ad4ap-49, -0x1.2f49b46814157p-57, 0x1.71b8ef6dcf572p-66};
__constant__ const double kCos[12] = {
    0x1.0000000000000p+0, -0x1.0000000000000p-1, 0x1.5555555555555p-5, -0x1.6c16c16c16c17p-10,
    0x1.a01a01a01a01ap-16, -0x1.27e4fb7789f5cp-22, 0x1.1eed8eff8d898p-29, -0x1.93974a8c07c9dp-37,
    0x1.ae7f3e733b81fp-45, -0x1.6827863b97d97p-53, 0x1.e542ba4020225p-62, -0x1.0ce396db7f853p-70};
constexpr double kLn2 = 0x1.62e42fefa39efp-1;
constexpr double kSqrt2 = 0x1.6a09e667f3bcdp+0;
constexpr double kHalfPi = 0x1.921fb54442d18p+0;

__device__ __forceinline__ double bits_to_f64(uint64_t b) { return __longlong_as_double((long long)b); }
__device__ __forceinline__ uint64_t f64_to_bits(double d) { return (uint64_t)__double_as_longlong(d); }

// ln u, u in [2^-53, 1]
__device__ __forceinline__ double ln_unit(double u) {
  const uint64_t b = f64_to_bits(u);
  int e = (int)((b >> 52) & 0x7FF) - 1023;
  double m = bits_to_f64((b & 0xFFFFFFFFFFFFFull) | (1023ull << 52));
  if (m > kSqrt2) {
    m = __dmul_rn(m, 0.5);
    e += 1;
  }
  const double s = __ddiv_rn(__dsub_rn(m, 1.0), __dadd_rn(m, 1.0));
  const double s2 = __dmul_rn(s, s);
  double p = kAtanh[11];
#pragma unroll
  for (int j = 10; j >= 0; --j) p = __dadd_rn(__dmul_rn(p, s2), kAtanh[j]);
  return __dadd_rn(__dmul_rn((double)e, kLn2), __dmul_rn(__dmul_rn(2.0, s), p));
}

// sqrt a, a >= 0: halved-exponent first guess, four Newton steps
__device__ __forceinline__ double sqrt_newton(double a) {
  if (a == 0.0) return 0.0;
  double y = bits_to_f64((f64_to_bits(a) >> 1) + 0x1FF8000000000000ull);
#pragma unroll
  for (int i = 0; i < 4; ++i) y = __dmul_rn(0.5, __dadd_rn(y, __ddiv_rn(a, y)));
  return y;
}

// cos(2 pi w / 2^32)
__device__ __forceinline__ double cos_turn(uint32_t w) {
  const uint32_t q = w >> 30;
  const double x = __dmul_rn(__dmul_rn((double)(w & 0x3FFFFFFFu), 0x1p-30), kHalfPi);
  const double x2 = __dmul_rn(x, x);
  double v;
  if (q & 1u) {
    double p = kSin[10];
#pragma unroll
    for (int j = 9; j >= 0; --j) p = __dadd_rn(__dmul_rn(p, x2), kSin[j]);
    v = __dmul_rn(x, p);
  } else {
    double p = kCos[11];
#pragma unroll
    for (int j = 10; j >= 0; --j) p = __dadd_rn(__dmul_rn(p, x2), kCos[j]);
    v = p;
  }
  return (q == 1 || q == 2) ? -v : v;
}

__device__ __forceinline__ float element_f32(uint64_t n, uint32_t k0, uint32_t k1, double sigma) {
  uint32_t c0 = (uint32_t)n, c1 = (uint32_t)(n >> 32), c2 = 0u, c3 = 0u;
  philox10(c0, c1, c2, c3, k0, k1);
  const uint64_t m53 = (((uint64_t)c0 << 32) | c1) >> 11;
  const double u1 = __dmul_rn((double)(m53 + 1ull), 0x1p-53);
  const double r = sqrt_newton(-__dmul_rn(2.0, ln_unit(u1)));
  const double v = __dmul_rn(__dmul_rn(r, cos_turn(c2)), sigma);
  return __double2float_rn(v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void fill_bf16(uint16_t* __restrict__ out, uint64_t first, uint64_t count, uint32_t k0,
                          uint32_t k1, double sigma) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    out[i] = f32_to_bf16_rne(element_f32(first + i, k0, k1, sigma));
}

__global__ void fill_f32(float* __restrict__ out, uint64_t first, uint64_t count, uint32_t k0,
                         uint32_t k1, double sigma) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    out[i] = element_f32(first + i, k0, k1, sigma);
}

}  // namespace

// dtype 0: fp32, 1: bf16.  Returns a hipError_t value (0 on success).
extern "C" int synth_dev_fill(void* dst, int dtype, uint64_t first, uint64_t count, uint32_t key0,
                              uint32_t key1, double sigma, void* stream) {
  if (count == 0) return 0;
  if (!dst || (dtype != 0 && dtype != 1)) return (int)hipErrorInvalidValue;
  const int threads = 256;
  uint64_t want = (count + threads - 1) / threads;
  int blocks = (int)(want < 65536 ? want : 65536);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == 0)
    hipLaunchKernelGGL(fill_f32, dim3(blocks), dim3(threads), 0, s, (float*)dst, first, count, key0,
                       key1, sigma);
  else
    hipLaunchKernelGGL(fill_bf16, dim3(blocks), dim3(threads), 0, s, (uint16_t*)dst, first, count,
                       key0, key1, sigma);
  return (int)hipGetLastError();
}

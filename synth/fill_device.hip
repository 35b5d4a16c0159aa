// Seeded synthetic inputs, device side: fills a device buffer with the same
// Philox4x32-10 stream as philox_host.c (Salmon et al., SC'11, section 3.2),
// element n from counter (n_lo, n_hi, 0, 0) under key (key0, key1), summed over
// the four output words, centred, scaled in double, rounded to fp32 (RNE) and,
// for bf16, to bf16 (RNE).  Used to place the ~34 GB of routed-expert weights
// in HBM without a host round trip.  Holds no arithmetic of the decode layer.
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

__device__ __forceinline__ float element_f32(uint64_t n, uint32_t k0, uint32_t k1, double scale) {
  uint32_t c0 = (uint32_t)n, c1 = (uint32_t)(n >> 32), c2 = 0u, c3 = 0u;
  philox10(c0, c1, c2, c3, k0, k1);
  uint64_t s = (uint64_t)c0 + c1 + c2 + c3;
  int64_t centred = (int64_t)s - (int64_t)((1ull << 33) - 2ull);
  double v = __dmul_rn((double)centred, scale);
  return __double2float_rn(v);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void fill_bf16(uint16_t* __restrict__ out, uint64_t first, uint64_t count, uint32_t k0,
                          uint32_t k1, double scale) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    out[i] = f32_to_bf16_rne(element_f32(first + i, k0, k1, scale));
}

__global__ void fill_f32(float* __restrict__ out, uint64_t first, uint64_t count, uint32_t k0,
                         uint32_t k1, double scale) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    out[i] = element_f32(first + i, k0, k1, scale);
}

}  // namespace

// dtype 0: fp32, 1: bf16.  Returns a hipError_t value (0 on success).
extern "C" int synth_dev_fill(void* dst, int dtype, uint64_t first, uint64_t count, uint32_t key0,
                              uint32_t key1, double scale, void* stream) {
  if (count == 0) return 0;
  if (!dst || (dtype != 0 && dtype != 1)) return (int)hipErrorInvalidValue;
  const int threads = 256;
  uint64_t want = (count + threads - 1) / threads;
  int blocks = (int)(want < 65536 ? want : 65536);
  hipStream_t s = (hipStream_t)stream;
  if (dtype == 0)
    hipLaunchKernelGGL(fill_f32, dim3(blocks), dim3(threads), 0, s, (float*)dst, first, count, key0,
                       key1, scale);
  else
    hipLaunchKernelGGL(fill_bf16, dim3(blocks), dim3(threads), 0, s, (uint16_t*)dst, first, count,
                       key0, key1, scale);
  return (int)hipGetLastError();
}

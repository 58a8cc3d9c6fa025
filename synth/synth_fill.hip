// Device twin of synth/gen.py: fills a [B][H][N_alloc][D] tensor slice with the
// counter-based N(0, 1) values defined there (splitmix64 words, sum of twelve
// 16-bit uniforms), bit-identical to the host generator.  Inputs only: this file
// holds no attention arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t sum16(uint64_t w) {
  return (uint32_t)(w & 0xFFFF) + (uint32_t)((w >> 16) & 0xFFFF) +
         (uint32_t)((w >> 32) & 0xFFFF) + (uint32_t)(w >> 48);
}

__device__ __forceinline__ float normal_at(uint64_t key, uint64_t e) {
  uint64_t base = key + (3ull * e + 1ull) * kGolden;
  int32_t s = (int32_t)(sum16(mix64(base)) + sum16(mix64(base + kGolden)) +
                        sum16(mix64(base + 2ull * kGolden)));
  return (float)(s - 393210) * (1.0f / 65536.0f);  // exact: |num| < 2^19, power-of-two scale
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool kBf16>
__global__ void fill_kernel(void* __restrict__ dst, int B, int H, long long n_alloc, int D,
                            long long row0, long long rows, long long n0, uint64_t key) {
  const long long total = (long long)B * H * rows * D;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += stride) {
    const int c = (int)(idx % D);
    long long t = idx / D;
    const long long r = t % rows;
    t /= rows;
    const int h = (int)(t % H);
    const int b = (int)(t / H);
    const uint64_t e =
        (((((uint64_t)b << 12) + (uint64_t)h) << 24) + (uint64_t)(n0 + r)) * 1024ull + (uint64_t)c;
    const float x = normal_at(key, e);
    const long long off = (((long long)b * H + h) * n_alloc + row0 + r) * D + c;
    if (kBf16)
      static_cast<uint16_t*>(dst)[off] = bf16_rne(x);
    else
      static_cast<float*>(dst)[off] = x;
  }
}

}  // namespace

extern "C" int synth_fill_normal(int dtype, void* dst, int B, int H, long long n_alloc, int D,
                                 long long row0, long long rows, long long n0,
                                 unsigned long long key, void* stream) {
  if (dst == nullptr || B <= 0 || H <= 0 || D <= 0 || D > 1024 || rows <= 0 || row0 < 0 ||
      row0 + rows > n_alloc || n0 < 0 || n0 + rows > (1ll << 24) || B > (1 << 18) ||
      H > (1 << 12))
    return (int)hipErrorInvalidValue;
  const long long total = (long long)B * H * rows * D;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536ll * 8) blocks = 65536ll * 8;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == 1)
    hipLaunchKernelGGL(fill_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, dst, B, H,
                       n_alloc, D, row0, rows, n0, (uint64_t)key);
  else if (dtype == 0)
    hipLaunchKernelGGL(fill_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, dst, B, H,
                       n_alloc, D, row0, rows, n0, (uint64_t)key);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

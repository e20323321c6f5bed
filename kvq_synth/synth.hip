// Device side of the seeded input generator (the host side is kvq_synth/__init__.py,
// which defines the same values).  Holds no quantization or attention arithmetic.
//
// SplitMix64 (Steele, Lea, Flood 2014; constants as published by Vigna): the n-th
// output of a stream with state s is mix64(s + (n + 1) * GAMMA).  An element with
// counter idx draws outputs n = 3*idx + j, j = 0..2, splits each into four 16-bit
// uniforms and returns (sum - 6*65536) * 2^-16 (Irwin-Hall of order 12), times its
// gain, rounded to fp16.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float ih12(uint64_t key, uint64_t idx) {
  int32_t total = 0;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const uint64_t h = mix64(key + (idx * 3 + (uint64_t)(j + 1)) * kGamma);
    total += (int32_t)(h & 0xFFFF) + (int32_t)((h >> 16) & 0xFFFF) +
             (int32_t)((h >> 32) & 0xFFFF) + (int32_t)(h >> 48);
  }
  return (float)(total - 6 * 65536) * 0x1p-16f;
}

// out[((b*H + h)*T + t)*D + d] for coordinates (b0 + b, h, t0 + t, d).
__global__ void fill_kernel(uint16_t* out, uint64_t key, int32_t B, int32_t H, int64_t T,
                            int32_t D, int64_t t0, int32_t b0, const float* gains) {
  const int64_t n = (int64_t)B * H * T * D;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int32_t d = (int32_t)(i % D);
    const int64_t r = i / D;
    const int64_t t = r % T;
    const int64_t bh = r / T;
    const int32_t h = (int32_t)(bh % H);
    const int32_t b = (int32_t)(bh / H);
    const uint64_t idx = ((uint64_t)(b0 + b) << 48) | ((uint64_t)h << 36) |
                         ((uint64_t)(t0 + t) << 8) | (uint64_t)d;
    float x = ih12(key, idx);
    if (gains) x = x * gains[h * D + d];
    out[i] = __builtin_bit_cast(uint16_t, (_Float16)x);
  }
}

}  // namespace

extern "C" int kvq_synth_fill(uint16_t* out, uint64_t key, int32_t B, int32_t H, int64_t T,
                              int32_t D, int64_t t0, int32_t b0, const float* gains,
                              void* stream) {
  if (out == nullptr || B < 0 || H < 0 || T < 0 || D <= 0 || D > 256) return 1;
  const int64_t n = (int64_t)B * H * T * D;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  fill_kernel<<<dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream>>>(
      out, key, B, H, T, D, t0, b0, gains);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Device side of the seeded input generator (libsynth.so).  Not part of the
// layer: it only fills input tensors, with the same counter-based definition as
// synth/__init__.py (SplitMix64 output function per element, an Irwin-Hall sum
// of eight 16-bit fields or a 24-bit uniform, one exact int->float conversion
// and one float multiply, then bf16 round-to-nearest-even), so host and device
// produce identical bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr unsigned long long kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ unsigned long long mix64(unsigned long long z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__device__ __forceinline__ float value(unsigned long long key, unsigned long long i, int dist,
                                       float coef) {
  const unsigned long long base = key + (2ull * i + 1ull) * kGolden;
  const unsigned long long w0 = mix64(base);
  if (dist == 0) {
    const unsigned long long w1 = mix64(base + kGolden);
    long long s = 0;
#pragma unroll
    for (int sh = 0; sh < 64; sh += 16) s += (long long)((w0 >> sh) & 0xFFFFull);
#pragma unroll
    for (int sh = 0; sh < 64; sh += 16) s += (long long)((w1 >> sh) & 0xFFFFull);
    const float z = (float)(2 * s - 8 * 65535);
    return z * coef;
  }
  const long long u = (long long)(w0 >> 40);
  const float z = (float)(2 * u + 1 - (1ll << 24));
  return z * coef;
}

__global__ void fill_kernel(void* out, long long rows, long long cols, long long row0,
                            unsigned long long key, int dist, const float* coef, int is_bf16) {
  const long long n = rows * cols;
  for (long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (long long)gridDim.x * blockDim.x) {
    const long long c = e % cols;
    const unsigned long long i = (unsigned long long)(row0 * cols + e);
    const float v = value(key, i, dist, coef[c]);
    if (is_bf16) {
      uint32_t u = __float_as_uint(v);
      u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
      static_cast<uint16_t*>(out)[e] = (uint16_t)u;
    } else {
      static_cast<float*>(out)[e] = v;
    }
  }
}

}  // namespace

extern "C" int synth_fill(void* out, long long rows, long long cols, long long row0,
                          unsigned long long key, int dist, const float* coef, int is_bf16,
                          hipStream_t stream) {
  if (rows < 0 || cols <= 0 || !out || !coef || (dist != 0 && dist != 1)) return 1;
  if (rows == 0) return 0;
  const long long n = rows * cols;
  long long blocks = (n + 255) / 256;
  if (blocks > 1 << 20) blocks = 1 << 20;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, rows, cols,
                     row0, key, dist, coef, is_bf16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

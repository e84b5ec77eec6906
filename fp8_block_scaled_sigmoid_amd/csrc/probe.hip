// Attainable FP8 MFMA rate of the device: a kernel that does nothing but
// back-to-back v_mfma_f32_16x16x128_f8f6f4 (the instruction every grouped GEMM
// here is built on), so a GEMM's throughput can be reported against what the
// matrix cores reach in practice as well as against the published peak.
//
// Each wave keeps 16 independent accumulators (a dependent MFMA follows 15
// others, far beyond the instruction's latency) and two fragments per operand
// with small finite E4M3 codes; the accumulators are summed into `sink` at the
// end so no MFMA is dead code.
#include "common.h"

namespace {

using namespace moe;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;   // 4 waves

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters,
                                                                   float* __restrict__ sink) {
  const int tid = (int)threadIdx.x;
  // codes 0x30..0x37 (0.5 .. 0.9375) and 0x38..0x3F (1 .. 1.875): finite, no NaN
  const int ca = 0x30303030 | (tid & 7) * 0x01010101;
  const int cb = 0x38383838 | ((tid >> 3) & 7) * 0x01010101;
  i32x8 a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] = i32x8{ca, ca, ca, ca, ca, ca, ca, ca + i};
    b[i] = i32x8{cb, cb, cb, cb, cb, cb, cb, cb + i};
  }
  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i & 1], b[(i >> 1) & 1], acc[i],
                                                                 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  sink[(long long)blockIdx.x * kProbeThreads + tid] = s;
}

}  // namespace

extern "C" moe_status_t moe_probe_fp8_mfma(int blocks, int iters, float* sink, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || blocks > (1 << 20)) return MOE_ERR_SHAPE;
  if (!sink) return MOE_ERR_NULL;
  if (moe_status_t s = check_device()) return s;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                     iters, sink);
  return launch_status();
}

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

// Attainable HBM rates, to state each bandwidth-bound step against what the
// memory system delivers in practice for its own mix of reads and writes.
// Each mode streams `bytes` once, a workgroup taking contiguous 32 KiB chunks
// in grid-stride order, with 16-byte accesses:
//   mode 0  reads, eight non-temporal loads in flight per lane;
//   mode 1  writes, eight non-temporal stores per lane per chunk;
//   mode 2  reads, four ordinary loads in flight per lane;
//   mode 3  writes, ordinary stores.
// Loaded data is XOR-folded into `sink` so no load is dead.  The benchmark
// takes the faster read mode and the faster write mode as the attainable
// rates.
namespace {

typedef int i32x4p __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kChunkVec = kStreamThreads * 8;          // 16-byte vectors per 32 KiB chunk

template <bool NT, int DEPTH>
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const i32x4p* __restrict__ p,
                                                                     long long n,
                                                                     unsigned* __restrict__ sink) {
  i32x4p acc = {0, 0, 0, 0};
  const long long chunks = n / kChunkVec;
  for (long long c = blockIdx.x; c < chunks; c += gridDim.x) {
    const i32x4p* q = p + c * kChunkVec + threadIdx.x;
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += DEPTH) {
      i32x4p v[DEPTH];
#pragma unroll
      for (int j = 0; j < DEPTH; ++j)
        v[j] = NT ? __builtin_nontemporal_load(q + (j0 + j) * kStreamThreads) : q[(j0 + j) * kStreamThreads];
#pragma unroll
      for (int j = 0; j < DEPTH; ++j) acc ^= v[j];
    }
  }
  // the tail past the last whole chunk
  for (long long i = chunks * kChunkVec + (long long)blockIdx.x * kStreamThreads + threadIdx.x; i < n;
       i += (long long)gridDim.x * kStreamThreads)
    acc ^= p[i];
  unsigned v = (unsigned)(acc.x ^ acc.y ^ acc.z ^ acc.w);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v ^= (unsigned)__shfl_xor((int)v, o, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, v);
}

template <bool NT>
__global__ __launch_bounds__(kStreamThreads) void stream_write_kernel(i32x4p* __restrict__ p,
                                                                      long long n) {
  const i32x4p v = {(int)threadIdx.x, (int)blockIdx.x, 0x5A5A5A5A, 0x3C3C3C3C};
  const long long chunks = n / kChunkVec;
  for (long long c = blockIdx.x; c < chunks; c += gridDim.x) {
    i32x4p* q = p + c * kChunkVec + threadIdx.x;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (NT) __builtin_nontemporal_store(v, q + j * kStreamThreads);
      else q[j * kStreamThreads] = v;
    }
  }
  for (long long i = chunks * kChunkVec + (long long)blockIdx.x * kStreamThreads + threadIdx.x; i < n;
       i += (long long)gridDim.x * kStreamThreads)
    p[i] = v;
}

}  // namespace

extern "C" moe_status_t moe_probe_hbm(int mode, void* buf, size_t bytes, unsigned* sink,
                                      hipStream_t stream) {
  if (mode < 0 || mode > 3 || bytes % 16 != 0) return MOE_ERR_SHAPE;
  const bool read = mode == 0 || mode == 2;
  if (!buf || (read && !sink)) return MOE_ERR_NULL;
  if (!aligned16(buf)) return MOE_ERR_ALIGN;
  if (bytes == 0) return MOE_OK;
  if (moe_status_t s = check_device()) return s;
  const int cus = cu_count();
  if (cus <= 0) return MOE_ERR_HIP;
  const unsigned grid = (unsigned)cus * 8;            // 32 waves per compute unit
  const long long n = (long long)(bytes / 16);
  switch (mode) {
    case 0:
      hipLaunchKernelGGL((stream_read_kernel<true, 8>), dim3(grid), dim3(kStreamThreads), 0, stream,
                         static_cast<const i32x4p*>(buf), n, sink);
      break;
    case 2:
      hipLaunchKernelGGL((stream_read_kernel<false, 4>), dim3(grid), dim3(kStreamThreads), 0, stream,
                         static_cast<const i32x4p*>(buf), n, sink);
      break;
    case 1:
      hipLaunchKernelGGL(stream_write_kernel<true>, dim3(grid), dim3(kStreamThreads), 0, stream,
                         static_cast<i32x4p*>(buf), n);
      break;
    default:
      hipLaunchKernelGGL(stream_write_kernel<false>, dim3(grid), dim3(kStreamThreads), 0, stream,
                         static_cast<i32x4p*>(buf), n);
      break;
  }
  return launch_status();
}

// Fine-grained FP8 quantisers: one scale per 1x128 activation tile and per
// 128x128 weight block, recomputed from the data on every call ("DeepSeek-V3:
// Auxiliary-Loss-Free MoE Load Balancing, Multi-Token Prediction, and FP8
// Training at 671B Scale", section V, FP8 detail 1 and Figure 6; "DeepSeek-V3
// Technical Report" (deepforge), part 1 "Per-tile FP8 scaling").
//
// Both are HBM streams: 16 lanes own one 128-element tile row (8 elements, one
// 16-byte bf16 load each), the tile maximum is a 16-lane xor-shuffle reduction,
// and each lane stores its 8 codes as one 8-byte store.
#include "common.h"

namespace {

using namespace moe;

constexpr int kQuantBlock = 256;  // 16 tiles of 128 per block

template <typename InT>
__device__ __forceinline__ void load8(const InT* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// codes of v * m, or all zero when m == 0 (the zero-tile rule: no -0 codes)
__device__ __forceinline__ uint2 encode8(const float (&v)[8], float m) {
  uint2 o;
  o.x = e4m3_pack4(v[0] * m, v[1] * m, v[2] * m, v[3] * m);
  o.y = e4m3_pack4(v[4] * m, v[5] * m, v[6] * m, v[7] * m);
  if (m == 0.0f) o = make_uint2(0u, 0u);
  return o;
}

// x [rows, ld] -> q [rows, cols], d [rows, cols/128].  Each 16-lane group
// takes two tiles per pass (both loads issued before either is used).
template <typename InT>
__global__ __launch_bounds__(kQuantBlock) void quant_1x128_kernel(
    const InT* __restrict__ x, int rows, int cols, int ld, uint8_t* __restrict__ q,
    float* __restrict__ d) {
  const int tiles_per_row = cols >> 7;
  const long long n_tiles = (long long)rows * tiles_per_row;
  const int sub = threadIdx.x & 15;
  const long long groups = (long long)gridDim.x * (kQuantBlock / 16);
  for (long long tile = (long long)blockIdx.x * (kQuantBlock / 16) + (threadIdx.x >> 4);
       tile - (threadIdx.x >> 4) < n_tiles; tile += 2 * groups) {
    float v[2][8];
    float amax[2] = {0.0f, 0.0f};
    long long r[2];
    int j[2];
    bool live[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const long long t = tile + u * groups;
      live[u] = t < n_tiles;
      r[u] = live[u] ? t / tiles_per_row : 0;
      j[u] = live[u] ? (int)(t - r[u] * tiles_per_row) : 0;
      if (live[u]) load8<InT>(x + r[u] * (long long)ld + j[u] * 128 + sub * 8, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (live[u]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) amax[u] = fmaxf(amax[u], fabsf(v[u][i]));
      }
      amax[u] = group_max<16>(amax[u]);
      if (live[u]) {
        float m, dd;
        tile_scale(amax[u], m, dd);
        *reinterpret_cast<uint2*>(q + r[u] * (long long)cols + j[u] * 128 + sub * 8) =
            encode8(v[u], m);
        if (sub == 0) d[r[u] * tiles_per_row + j[u]] = dd;
      }
    }
  }
}

// One block per 128x128 block: w [batch, rows, cols] bf16 -> q, d.
__global__ __launch_bounds__(256) void quant_128x128_kernel(
    const uint16_t* __restrict__ w, int rows, int cols, int interleave, uint8_t* __restrict__ q,
    float* __restrict__ d) {
  __shared__ float wave_max[4];
  const int rb = blockIdx.y, cb = blockIdx.x, b = blockIdx.z;
  const int nrb = rows >> 7, ncb = cols >> 7;
  const int chunk = threadIdx.x & 15;   // 8-element chunk of the 128 columns
  const int row0 = threadIdx.x >> 4;    // 16 rows per pass, 8 passes
  const uint16_t* src = w + ((long long)b * rows + rb * 128) * cols + cb * 128 + chunk * 8;
  float v[8][8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    load8<uint16_t>(src + (long long)(row0 + 16 * p) * cols, v[p]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[p][i]));
  }
  amax = group_max<64>(amax);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  float m, dd;
  tile_scale(amax, m, dd);
  // output row block: with interleaving, gate block j -> 2j, up block j -> 2j+1
  int orb = rb;
  if (interleave) orb = rb < nrb / 2 ? 2 * rb : 2 * (rb - nrb / 2) + 1;
  uint8_t* dst = q + ((long long)b * rows + orb * 128) * cols + cb * 128 + chunk * 8;
#pragma unroll
  for (int p = 0; p < 8; ++p)
    *reinterpret_cast<uint2*>(dst + (long long)(row0 + 16 * p) * cols) = encode8(v[p], m);
  if (threadIdx.x == 0) d[((long long)b * nrb + orb) * ncb + cb] = dd;
}

}  // namespace

extern "C" moe_status_t fp8_quant_1x128(const void* x, moe_dtype_t dt, int rows, int cols,
                                        int ld, uint8_t* q, float* d, hipStream_t stream) {
  if (rows < 0 || cols < 0 || cols % 128 != 0 || ld < cols || ld % 8 != 0) return MOE_ERR_SHAPE;
  if (dt != MOE_BF16 && dt != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!x || !q || !d) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || (reinterpret_cast<uintptr_t>(d) & 3)) return MOE_ERR_ALIGN;
  if (moe_status_t s = check_device()) return s;
  const long long tiles = (long long)rows * (cols / 128);
  long long blocks = (tiles + 31) / 32;   // 16 groups of 16 lanes, two tiles each
  if (blocks > 65536) blocks = 65536;
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(quant_1x128_kernel<uint16_t>, dim3((unsigned)blocks), dim3(kQuantBlock), 0,
                       stream, static_cast<const uint16_t*>(x), rows, cols, ld, q, d);
  else
    hipLaunchKernelGGL(quant_1x128_kernel<float>, dim3((unsigned)blocks), dim3(kQuantBlock), 0,
                       stream, static_cast<const float*>(x), rows, cols, ld, q, d);
  return launch_status();
}

extern "C" moe_status_t fp8_quant_128x128(const void* w_bf16, int batch, int rows, int cols,
                                          int interleave_gate_up, uint8_t* q, float* d,
                                          hipStream_t stream) {
  if (batch < 0 || rows < 0 || cols < 0 || rows % 128 || cols % 128) return MOE_ERR_SHAPE;
  if (interleave_gate_up && rows % 256) return MOE_ERR_SHAPE;
  if (batch == 0 || rows == 0 || cols == 0) return MOE_OK;
  if (!w_bf16 || !q || !d) return MOE_ERR_NULL;
  if (!aligned16(w_bf16) || !aligned16(q) || (reinterpret_cast<uintptr_t>(d) & 3))
    return MOE_ERR_ALIGN;
  if (rows / 128 > 65535 || batch > 65535) return MOE_ERR_SHAPE;
  if (moe_status_t s = check_device()) return s;
  hipLaunchKernelGGL(quant_128x128_kernel, dim3(cols / 128, rows / 128, batch), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(w_bf16), rows, cols,
                     interleave_gate_up ? 1 : 0, q, d);
  return launch_status();
}

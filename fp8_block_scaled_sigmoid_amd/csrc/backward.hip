// FP8 backward GEMMs of a block-scaled linear layer Y = X W^T ("DeepSeek-V3:
// Auxiliary-Loss-Free MoE Load Balancing, Multi-Token Prediction, and FP8
// Training at 671B Scale", section V, Figure 6: the input-gradient (Dgrad) and
// weight-gradient (Wgrad) GEMMs take FP8 inputs and accumulate in FP32; detail
// 3: E4M3 on every tensor with fine-grained scales; detail 4 and "DeepSeek-V3
// Technical Report" (deepforge) part 1 "FP8 training, from first principles":
// gradients stay in higher precision).
//
//   Dgrad  dX = dY W: dY quantised 1x128 along its channels (the activation
//          rule), W in its forward 128x128 blocks used transposed.  The
//          transposed codes and scales are exact (a block transposes into a
//          block with the same scale); fp8_transpose_128x128 writes them and
//          the forward grouped GEMM does the product.
//   Wgrad  dW_g = dY_g^T X_g per expert g: the contraction runs over the
//          expert's tokens, so both operands are quantised in tiles of 128
//          consecutive tokens of one channel (fp8_quant_tokens_128, which also
//          transposes them so the contraction is contiguous), and
//          moe_grouped_wgrad_fp8 forms every expert's [N, K] product in float.
#include <type_traits>

#include "common.h"

namespace {

using namespace moe;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kMaxGroupsBw = 1025;

__device__ __forceinline__ int clampi_bw(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------
// exact transpose of block-quantised weights: 64 x 64-byte tiles through LDS

__global__ __launch_bounds__(256) void transpose_blocks_kernel(const uint8_t* __restrict__ w,
                                                               const float* __restrict__ wd,
                                                               int rows, int cols,
                                                               uint8_t* __restrict__ wt,
                                                               float* __restrict__ wtd) {
  __shared__ uint32_t tile[64][17];   // 64 rows of 64 bytes, one word of padding
  const long long b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const uint8_t* src = w + b * (long long)rows * cols;
  {
    const int r = t >> 2, c = (t & 3) * 16;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (long long)(r0 + r) * cols + c0 + c);
    tile[r][c / 4 + 0] = v.x;
    tile[r][c / 4 + 1] = v.y;
    tile[r][c / 4 + 2] = v.z;
    tile[r][c / 4 + 3] = v.w;
  }
  __syncthreads();
  {
    // output row c0 + c holds input column c0 + c; this thread writes its
    // input rows r .. r + 15 (16 bytes)
    const int c = t >> 2, r = (t & 3) * 16;
    const int word = c >> 2, sh = (c & 3) * 8;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t acc = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc |= ((tile[r + 4 * i + k][word] >> sh) & 0xFFu) << (8 * k);
      o[i] = acc;
    }
    *reinterpret_cast<uint4*>(wt + b * (long long)rows * cols + (long long)(c0 + c) * rows + r0 + r) =
        make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (t == 0 && (r0 & 127) == 0 && (c0 & 127) == 0) {
    const int rb = rows / 128, cb = cols / 128;
    wtd[b * rb * cb + (long long)(c0 / 128) * rb + r0 / 128] =
        wd[b * rb * cb + (long long)(r0 / 128) * cb + c0 / 128];
  }
}

// ---------------------------------------------------------------------------
// token-tile quantiser

// pad[g] = first padded token column of group g: the sum over earlier groups
// of 128 * ceil(rows_g / 128); pad[G] = the padded length.  One block.
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ off, int G,
                                                           int rows, int32_t* __restrict__ pad) {
  __shared__ int s_w[16];
  __shared__ int s_carry;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < G; base += 1024) {
    const int g = base + (int)threadIdx.x;
    int len = 0;
    if (g < G) {
      const int r0 = clampi_bw(off[g], 0, rows), r1 = clampi_bw(off[g + 1], 0, rows);
      len = r1 > r0 ? (r1 - r0 + 127) / 128 * 128 : 0;
    }
    int incl = len;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int pre = s_carry;
    for (int w = 0; w < wave; ++w) pre += s_w[w];
    if (g < G) pad[g] = pre + incl - len;
    __syncthreads();
    if (threadIdx.x == 1023) s_carry = pre + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) pad[G] = s_carry;
}

template <typename InT>
__device__ __forceinline__ void load8_bw(const InT* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8_bw<uint16_t>(const uint16_t* p, float (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
template <>
__device__ __forceinline__ void load8_bw<float>(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One block per (64 channels, padded token tile): the tile's 128 x 64 values
// are staged in LDS with coalesced row loads; then 4 lanes per channel take
// 32 tokens each, meet for the tile maximum with two xor shuffles, and each
// writes its 32 codes as two 16-byte stores (4 lanes cover one 128-byte row
// segment of the transposed output).
template <typename InT>
__global__ __launch_bounds__(256) void quant_tokens_kernel(
    const InT* __restrict__ x, int rows, long long ldx, const int32_t* __restrict__ off,
    const int32_t* __restrict__ pad, int G, uint8_t* __restrict__ xt, float* __restrict__ xtd,
    long long ldt) {
  __shared__ float tile[128][65];
  const int j = blockIdx.y;
  const int c0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const int total = pad[G];
  if (j * 128 >= total) return;
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pad[mid] <= j * 128) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int r0 = clampi_bw(off[g], 0, rows), r1 = clampi_bw(off[g + 1], 0, rows);
  const int t0 = r0 + (j * 128 - pad[g]);
  const int n = min(128, r1 - t0);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = p * 32 + (t >> 3), cc = (t & 7) * 8;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (row < n) load8_bw<InT>(x + (long long)(t0 + row) * ldx + c0 + cc, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[row][cc + i] = v[i];
  }
  __syncthreads();
  const int c = t >> 2, q = t & 3;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = tile[q * 32 + i][c];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  float m, d;
  tile_scale(amax, m, d);
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    w[k] = m == 0.0f ? 0u : e4m3_pack4(v[4 * k] * m, v[4 * k + 1] * m, v[4 * k + 2] * m, v[4 * k + 3] * m);
  uint8_t* dst = xt + (long long)(c0 + c) * ldt + (long long)j * 128 + q * 32;
  reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
  reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
  if (q == 0) xtd[(long long)(c0 + c) * (ldt / 128) + j] = d;
}

// ---------------------------------------------------------------------------
// Wgrad grouped GEMM

constexpr int kWM = 128, kWN = 128;                        // output tile: N rows x K columns
constexpr int kWThreads = 256;                             // 4 waves, 2 x 2 of 64 x 64
constexpr int kWStage = kWM * 128 + kWN * 128 + (kWM + kWN) * 4;   // codes, then A and B scales
constexpr int kWStages = 2;
constexpr int kWOutStride = kWN + 4;                       // float stride of the output staging
constexpr int kWLds = kWStages * kWStage > kWM * kWOutStride * 4 ? kWStages * kWStage
                                                                  : kWM * kWOutStride * 4;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_bw(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
template <int N>
__device__ __forceinline__ void wait_barrier_bw() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

struct WgradParams {
  const uint8_t* a_q;  // dY^T codes [N][lda]
  const float* a_d;    // [N][lda / 128]
  long long lda;
  const uint8_t* b_q;  // X^T codes [K][ldb]
  const float* b_d;    // [K][ldb / 128]
  long long ldb;
  const int32_t* pad;  // [G + 1], multiples of 128
  int G, N, K;
  float* out;          // [G][N][K]
};

// Tile (g, n-tile, k-tile) of the list, XCD-aware like the forward GEMM: each
// XCD takes a contiguous run, so one XCD works through one expert's operands.
// An expert's contraction is short (its tokens), so the float output write
// dominates: the tile is 128 x 128 with 4 waves and two stages (67.6 KiB of
// LDS), which lets two workgroups share a compute unit and overlap one's
// loads with the other's write; the output is written with streaming
// (non-temporal) stores.  Wave (wm, wn) owns 64 x 64 outputs; per 128-token
// block, 16 FP8 MFMAs into zero accumulators, then acc += part * (d_A[row] *
// d_B[col]).
__global__ __launch_bounds__(kWThreads, 2) void wgrad_kernel(WgradParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tn = p.N / kWM, tk = p.K / kWN;
  const int per_g = tn * tk;
  const long long total = (long long)p.G * per_g;
  const long long per_xcd = (total + 7) / 8;
  const long long slot = blockIdx.x >> 3, xcd = blockIdx.x & 7;
  const long long L = xcd * per_xcd + slot;
  if (slot >= per_xcd || L >= total) return;
  const int g = (int)(L / per_g);
  const int rem = (int)(L - (long long)g * per_g);
  const int n0 = (rem / tk) * kWM, k0 = (rem % tk) * kWN;
  const int lim = (int)min(p.lda, p.ldb) / 128 * 128;
  const int p0 = clampi_bw(p.pad[g], 0, lim), p1 = clampi_bw(p.pad[g + 1], p0, lim);
  const int nkb = (p1 - p0) / 128;

  // copies: load j of wave w fills 1 KiB block 4 j + w (rows 8 (4 j + w) ..);
  // lane l: row + (l >> 3), swizzled chunk (l & 7) ^ ((row >> 1) & 7)
  const int chunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow8 = 8 * wave + (lane >> 3);
  const int sa_stride = (int)(p.lda / 128), sb_stride = (int)(p.ldb / 128);
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc_bw(p.a_q, (int)(p.N * p.lda));
  const __amdgpu_buffer_rsrc_t rs_b = make_rsrc_bw(p.b_q, (int)(p.K * p.ldb));
  const __amdgpu_buffer_rsrc_t rs_sa = make_rsrc_bw(p.a_d, p.N * sa_stride * 4);
  const __amdgpu_buffer_rsrc_t rs_sb = make_rsrc_bw(p.b_d, p.K * sb_stride * 4);
  int a_off[4], b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a_off[j] = (n0 + 32 * j + lrow8) * (int)p.lda + p0 + chunk * 16;
    b_off[j] = (k0 + 32 * j + lrow8) * (int)p.ldb + p0 + chunk * 16;
  }
  // scales: waves 0-1 copy the 128 A-row scales, waves 2-3 the 128 B-row scales
  const int s_off = wave < 2 ? ((n0 + 64 * wave + lane) * sa_stride + p0 / 128) * 4
                             : ((k0 + 64 * (wave - 2) + lane) * sb_stride + p0 / 128) * 4;
  auto issue = [&](int kb, uint8_t* st) {
    const int ko = kb * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_ptr_t)(st + (4 * j + wave) * 1024), 16,
                                               a_off[j], ko, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_b, (lds_ptr_t)(st + kWM * 128 + (4 * j + wave) * 1024), 16, b_off[j], ko, 0, 0);
    if (wave < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_sa, (lds_ptr_t)(st + (kWM + kWN) * 128 + wave * 256), 4, s_off, kb * 4, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_sb, (lds_ptr_t)(st + (kWM + kWN) * 128 + kWM * 4 + (wave - 2) * 256), 4, s_off,
          kb * 4, 0, 0);
  };

  const int wm = wave & 1, wn = wave >> 1;
  const int lrow = lane & 15, lk = lane >> 4;
  const int sw = (lrow >> 1) & 7;
  const int frag_lo = lrow * 128 + ((lk ^ sw) << 4);
  const int frag_hi = lrow * 128 + (((lk + 4) ^ sw) << 4);
  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  // two stages: stage kb + 2 reuses kb's slot once every wave is done with it
  if (nkb > 0) issue(0, smem);
  if (nkb > 1) issue(1, smem + kWStage);
  for (int kb = 0; kb < nkb; ++kb) {
    if (kb + 1 < nkb) wait_barrier_bw<9>(); else wait_barrier_bw<0>();
    const uint8_t* st = smem + (kb % kWStages) * kWStage;
    const float* sA = reinterpret_cast<const float*>(st + (kWM + kWN) * 128) + wm * 64 + 4 * lk;
    const float* sB = reinterpret_cast<const float*>(st + (kWM + kWN) * 128 + kWM * 4) + wn * 64 + lrow;
    i32x8 af[4], bfr[4];
    f32x4 sa[4];
    float sbc[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const uint8_t* a = st + (wm * 64 + mi * 16) * 128;
      const i32x4 x0 = *reinterpret_cast<const i32x4*>(a + frag_lo);
      const i32x4 x1 = *reinterpret_cast<const i32x4*>(a + frag_hi);
      af[mi] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
      sa[mi] = *reinterpret_cast<const f32x4*>(sA + mi * 16);
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const uint8_t* b = st + kWM * 128 + (wn * 64 + ni * 16) * 128;
      const i32x4 y0 = *reinterpret_cast<const i32x4*>(b + frag_lo);
      const i32x4 y1 = *reinterpret_cast<const i32x4*>(b + frag_hi);
      bfr[ni] = __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
      sbc[ni] = sB[ni * 16];
    }
    if (kb + 2 < nkb) {
      // every wave's fragment reads of this slot are done before it is refilled
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      issue(kb + 2, smem + (kb % kWStages) * kWStage);
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[mi], bfr[ni], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[mi][ni][v] = __builtin_fmaf(part[v], sa[mi][v] * sbc[ni], acc[mi][ni][v]);
      }
  }
  __syncthreads();
  // stage the float tile in LDS (row stride 132 floats keeps the writes of a
  // wave on distinct banks), then stream whole 512-byte output rows
  float* o = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        o[(wm * 64 + mi * 16 + 4 * lk + v) * kWOutStride + wn * 64 + ni * 16 + lrow] = acc[mi][ni][v];
  __syncthreads();
  float* out = p.out + ((long long)g * p.N + n0) * p.K + k0;
#pragma unroll 4
  for (int q = tid; q < kWM * (kWN / 4); q += kWThreads) {
    const int r = q / (kWN / 4), c4 = (q % (kWN / 4)) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(o + r * kWOutStride + c4);
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(out + (long long)r * p.K + c4));
  }
}

}  // namespace

extern "C" moe_status_t fp8_transpose_128x128(const uint8_t* w_q, const float* w_d, int batch,
                                              int rows, int cols, uint8_t* wt_q, float* wt_d,
                                              hipStream_t stream) {
  if (batch < 0 || rows < 0 || cols < 0 || rows % 128 || cols % 128) return MOE_ERR_SHAPE;
  if (batch == 0 || rows == 0 || cols == 0) return MOE_OK;
  if (!w_q || !w_d || !wt_q || !wt_d) return MOE_ERR_NULL;
  if (!aligned16(w_q) || !aligned16(wt_q) || (reinterpret_cast<uintptr_t>(w_d) & 3) ||
      (reinterpret_cast<uintptr_t>(wt_d) & 3))
    return MOE_ERR_ALIGN;
  if (rows / 64 > 65535 || batch > 65535 || cols / 64 > 0x7FFFFFFF) return MOE_ERR_SHAPE;
  if (moe_status_t s = check_device()) return s;
  hipLaunchKernelGGL(transpose_blocks_kernel, dim3(cols / 64, rows / 64, batch), dim3(256), 0,
                     stream, w_q, w_d, rows, cols, wt_q, wt_d);
  return launch_status();
}

extern "C" moe_status_t fp8_quant_tokens_128(const void* x, moe_dtype_t dt, int rows, int cols,
                                             long long ldx, const int32_t* group_offsets,
                                             int num_groups, uint8_t* xt_q, float* xt_d,
                                             long long ldt, int32_t* pad_offsets,
                                             hipStream_t stream) {
  if (rows < 0 || cols < 0 || cols % 64 != 0 || ldx < cols || num_groups < 1 ||
      num_groups > kMaxGroupsBw || ldt % 128 != 0 || ldt < (long long)rows + 127LL * num_groups)
    return MOE_ERR_SHAPE;
  if (dt != MOE_BF16 && dt != MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (dt == MOE_BF16 ? ldx % 8 != 0 : ldx % 4 != 0) return MOE_ERR_SHAPE;
  if (!group_offsets || !pad_offsets) return MOE_ERR_NULL;
  if (cols > 0 && (!x || !xt_q || !xt_d)) return MOE_ERR_NULL;
  if ((cols > 0 && (!aligned16(x) || !aligned16(xt_q))) ||
      (reinterpret_cast<uintptr_t>(xt_d) & 3))
    return MOE_ERR_ALIGN;
  const long long tiles = ((long long)rows + 127) / 128 + num_groups;   // bound on the padded tiles
  if (tiles > 65535) return MOE_ERR_UNSUPPORTED;
  if (moe_status_t s = check_device()) return s;
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, stream, group_offsets,
                     num_groups, rows, pad_offsets);
  if (moe_status_t s = launch_status()) return s;
  if (rows == 0 || cols == 0) return MOE_OK;
  const dim3 grid(cols / 64, (unsigned)tiles);
  if (dt == MOE_BF16)
    hipLaunchKernelGGL(quant_tokens_kernel<uint16_t>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), rows, ldx, group_offsets, pad_offsets,
                       num_groups, xt_q, xt_d, ldt);
  else
    hipLaunchKernelGGL(quant_tokens_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float*>(x), rows, ldx, group_offsets, pad_offsets,
                       num_groups, xt_q, xt_d, ldt);
  return launch_status();
}

extern "C" moe_status_t moe_grouped_wgrad_fp8(const uint8_t* a_q, const float* a_d, long long lda,
                                              int n_rows, const uint8_t* b_q, const float* b_d,
                                              long long ldb, int k_rows,
                                              const int32_t* pad_offsets, int num_groups,
                                              float* out, hipStream_t stream) {
  if (n_rows < 0 || k_rows < 0 || n_rows % 128 != 0 || k_rows % 128 != 0 || lda < 128 ||
      ldb < 128 || lda % 128 != 0 || ldb % 128 != 0 || num_groups < 1 ||
      num_groups > kMaxGroupsBw)
    return MOE_ERR_SHAPE;
  if (n_rows == 0 || k_rows == 0) return MOE_OK;
  if ((long long)n_rows * lda >= (1LL << 31) || (long long)k_rows * ldb >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  if (!a_q || !a_d || !b_q || !b_d || !pad_offsets || !out) return MOE_ERR_NULL;
  if (!aligned16(a_q) || !aligned16(b_q) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(a_d) & 3) || (reinterpret_cast<uintptr_t>(b_d) & 3))
    return MOE_ERR_ALIGN;
  if (moe_status_t s = check_device()) return s;
  static std::atomic<uint64_t> lds_set{0};
  if (moe_status_t st = allow_dynamic_lds(reinterpret_cast<const void*>(&wgrad_kernel),
                                          kWLds, lds_set))
    return st;
  WgradParams p;
  p.a_q = a_q; p.a_d = a_d; p.lda = lda; p.b_q = b_q; p.b_d = b_d; p.ldb = ldb;
  p.pad = pad_offsets; p.G = num_groups; p.N = n_rows; p.K = k_rows; p.out = out;
  const long long tiles = (long long)num_groups * (n_rows / kWM) * (k_rows / kWN);
  const long long grid = (tiles + 7) / 8 * 8;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)grid), dim3(kWThreads), kWLds, stream, p);
  return launch_status();
}

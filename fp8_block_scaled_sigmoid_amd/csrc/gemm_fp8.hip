// Grouped block-scaled FP8 GEMM for the routed and shared experts.
//
// What it computes ("DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing,
// Multi-Token Prediction, and FP8 Training at 671B Scale", section V, Figure 6
// and FP8 details 1-2; "DeepSeek-V3, explained.", recipe step 7): E4M3
// operands with one scale per 1x128 activation tile and per 128x128 weight
// block, float accumulation, bf16 (or re-quantised E4M3) output.  The pages
// promote partial sums to FP32 every 128 products because their tensor cores
// accumulate with ~14 bits.  CDNA4 MFMA accumulates in fp32 already, but the
// scales still change every 128 elements of K, so each 128-deep block is one
// v_mfma_f32_16x16x128_f8f6f4 into a zero accumulator, folded into the running
// sum with one fused multiply-add by d_A[row, kb] * d_B[col block, kb].
//
// Layout and schedule:
//   * a workgroup of 8 waves (2 per SIMD) computes a 128 x 256 output tile of
//     one group (expert); wave (wm, wn) owns 64 rows x 64 columns = 4 x 4 MFMA
//     subtiles, all inside one 128x128 weight block, so each wave needs one B
//     scale per K block and its 64 float accumulators stay in VALU registers
//     for the per-block fused multiply-add;
//   * per 128-deep K block the A tile (128 x 128 B, rows gathered through
//     a_row_index), the B tile (256 x 128 B) and the 128 A scales are staged in
//     LDS, double-buffered through registers, 16-byte chunks XOR-swizzled by
//     row to spread LDS banks;
//   * with the SwiGLU epilogue the B tile is the interleaved pair (gate block j,
//     up block j) of W1: the "up" waves pass their accumulators to the "gate"
//     waves through LDS, and the 128 h columns of a row form exactly one 1x128
//     quantisation tile;
//   * every workgroup derives the tile list itself from the device-side group
//     offsets (tiles ordered group, column tile, row tile), so the call needs no
//     workspace and no host sync; consecutive row tiles of one (expert, column
//     tile) are mapped to the same XCD so their weight tile is fetched from HBM
//     once and re-read from that XCD's L2.
#include "common.h"

namespace {

using namespace moe;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int kThreads = 512;   // 8 waves, 2 per SIMD
constexpr int kMaxGroups = 2048;  // 4 per thread in the tile-list scan
constexpr int kABytes = BM * BK;                       // 16 KiB
constexpr int kBBytes = BN * BK;                       // 32 KiB
constexpr int kStage = kABytes + kBBytes + BM * 4;     // + A scales
constexpr int kLds = 2 * kStage;                       // 97 KiB

struct GemmParams {
  const uint8_t* a_q;
  const float* a_d;
  long long lda;
  int a_rows;
  const int32_t* a_row_index;
  const uint8_t* b_q;
  const float* b_d;
  const int32_t* offsets;
  int G;
  int total_rows;
  int n_out;
  int k_dim;
  void* out;
  float* out_d;
  long long ldo;
  const float* row_scale;
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_prefix[kMaxGroups + 1];
  __shared__ int s_tmp[kThreads];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = p.G;
  const int n_tiles = (p.n_out + BN - 1) / BN;   // the last tile may be 128 wide

  // ---- tile list: exclusive prefix of (row tiles x column tiles) per group
  {
    const int per = (G + kThreads - 1) / kThreads;   // <= 4
    int cnt[4];
    int run = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = tid * per + i;
      int c = 0;
      if (i < per && g < G) {
        const int r0 = clampi(p.offsets[g], 0, p.total_rows);
        const int r1 = clampi(p.offsets[g + 1], 0, p.total_rows);
        const int rows = r1 > r0 ? r1 - r0 : 0;
        c = ((rows + BM - 1) / BM) * n_tiles;
      }
      cnt[i] = c;
      run += c;
    }
    s_tmp[tid] = run;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
      const int v = tid >= o ? s_tmp[tid - o] : 0;
      __syncthreads();
      s_tmp[tid] += v;
      __syncthreads();
    }
    int base = s_tmp[tid] - run;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = tid * per + i;
      if (i < per && g < G) {
        s_prefix[g] = base;
        base += cnt[i];
      }
    }
    if (tid == kThreads - 1) s_prefix[G] = s_tmp[tid];
    __syncthreads();
  }
  const int total = s_prefix[G];
  // XCD-aware mapping: dispatch sends block b to XCD b % 8; give each XCD a
  // contiguous run of the tile list.
  const int per_xcd = (total + 7) / 8;
  const int slot = blockIdx.x >> 3, xcd = blockIdx.x & 7;
  if (slot >= per_xcd) return;
  const int L = xcd * per_xcd + slot;
  if (L >= total) return;
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_prefix[mid] <= L) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int row0 = clampi(p.offsets[g], 0, p.total_rows);
  const int rows_g = clampi(p.offsets[g + 1], 0, p.total_rows) - row0;
  const int mt = (rows_g + BM - 1) / BM;
  const int local = L - s_prefix[g];
  const int n_tile = local / mt;
  const int m0 = (local - n_tile * mt) * BM;
  const int nkb = p.k_dim / BK;

  // ---- per-thread global sources: A rows (tid>>3) and +64, B rows (tid>>3) + 64 j
  const int lrow_ld = tid >> 3, lchunk = tid & 7;
  const uint8_t* a_src0;
  const uint8_t* a_src1;
  {
    int r = row0 + min(m0 + lrow_ld, rows_g - 1);
    int src = p.a_row_index ? p.a_row_index[r] : r;
    src = clampi(src, 0, p.a_rows - 1);
    a_src0 = p.a_q + (long long)src * p.lda + lchunk * 16;
    r = row0 + min(m0 + lrow_ld + 64, rows_g - 1);
    src = p.a_row_index ? p.a_row_index[r] : r;
    src = clampi(src, 0, p.a_rows - 1);
    a_src1 = p.a_q + (long long)src * p.lda + lchunk * 16;
  }
  const float* sa_src = p.a_d;
  if (tid < BM) {
    const int r = row0 + min(m0 + tid, rows_g - 1);
    int src = p.a_row_index ? p.a_row_index[r] : r;
    src = clampi(src, 0, p.a_rows - 1);
    sa_src = p.a_d + (long long)src * nkb;
  }
  // B rows past n_out (a 128-wide last tile) re-read the last row; their
  // results are never stored
  const uint8_t* b_grp = p.b_q + (long long)g * p.n_out * p.k_dim + lchunk * 16;
  int b_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) b_off[j] = min(n_tile * BN + lrow_ld + 64 * j, p.n_out - 1) * p.k_dim;
  const int st_a0 = swz(lrow_ld, lchunk), st_a1 = swz(lrow_ld + 64, lchunk);
  const int st_b0 = kABytes + swz(lrow_ld, lchunk);

  // ---- wave tile: rows wm*64..+64, B-tile rows wn*64..+64 (one 128x128 weight
  // block per wave: wn < 2 -> block 0 (gate), wn >= 2 -> block 1 (up))
  const int wm = wave & 1, wn = wave >> 1;
  const int lrow = lane & 15, lk = lane >> 4;
  const int nb_w = min(2 * n_tile + (wn >> 1), p.n_out / 128 - 1);   // this wave's weight block
  const bool wave_cols = 2 * n_tile + (wn >> 1) < p.n_out / 128;    // false: past n_out
  const float* bd = p.b_d + ((long long)g * (p.n_out / 128) + nb_w) * nkb;

  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra0, ra1, rb0, rb1, rb2, rb3;
  float rsa = 0.0f;
#define MOE_GLOAD(kb)                                                               \
  {                                                                                 \
    const long long ko = (long long)(kb) * BK;                                      \
    ra0 = *reinterpret_cast<const uint4*>(a_src0 + ko);                             \
    ra1 = *reinterpret_cast<const uint4*>(a_src1 + ko);                             \
    rb0 = *reinterpret_cast<const uint4*>(b_grp + b_off[0] + ko);                   \
    rb1 = *reinterpret_cast<const uint4*>(b_grp + b_off[1] + ko);                   \
    rb2 = *reinterpret_cast<const uint4*>(b_grp + b_off[2] + ko);                   \
    rb3 = *reinterpret_cast<const uint4*>(b_grp + b_off[3] + ko);                   \
    if (tid < BM) rsa = sa_src[kb];                                                 \
  }
#define MOE_LSTORE(st)                                                              \
  {                                                                                 \
    *reinterpret_cast<uint4*>((st) + st_a0) = ra0;                                  \
    *reinterpret_cast<uint4*>((st) + st_a1) = ra1;                                  \
    *reinterpret_cast<uint4*>((st) + st_b0) = rb0;                                  \
    *reinterpret_cast<uint4*>((st) + st_b0 + 64 * 128) = rb1;                       \
    *reinterpret_cast<uint4*>((st) + st_b0 + 128 * 128) = rb2;                      \
    *reinterpret_cast<uint4*>((st) + st_b0 + 192 * 128) = rb3;                      \
    if (tid < BM) reinterpret_cast<float*>((st) + kABytes + kBBytes)[tid] = rsa;    \
  }

  MOE_GLOAD(0);
  MOE_LSTORE(smem);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    uint8_t* st = smem + (kb & 1) * kStage;
    if (kb + 1 < nkb) MOE_GLOAD(kb + 1);
    const float* sA = reinterpret_cast<const float*>(st + kABytes + kBBytes);
    const float sb = bd[kb];
    float s[16];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) s[mi * 4 + v] = sA[wm * 64 + mi * 16 + 4 * lk + v] * sb;
    i32x8 af[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int r = wm * 64 + mi * 16 + lrow;
      const uint4 x0 = *reinterpret_cast<const uint4*>(st + swz(r, 2 * lk));
      const uint4 x1 = *reinterpret_cast<const uint4*>(st + swz(r, 2 * lk + 1));
      af[mi] = i32x8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int r = wn * 64 + ni * 16 + lrow;
      const uint4 y0 = *reinterpret_cast<const uint4*>(st + kABytes + swz(r, 2 * lk));
      const uint4 y1 = *reinterpret_cast<const uint4*>(st + kABytes + swz(r, 2 * lk + 1));
      const i32x8 bf = i32x8{(int)y0.x, (int)y0.y, (int)y0.z, (int)y0.w,
                             (int)y1.x, (int)y1.y, (int)y1.z, (int)y1.w};
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[mi], bf, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[mi][ni][v] = __builtin_fmaf(part[v], s[mi * 4 + v], acc[mi][ni][v]);
      }
    }
    if (kb + 1 < nkb) MOE_LSTORE(smem + ((kb + 1) & 1) * kStage);
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_LSTORE

  // ---- epilogues (the staging buffers are free after the final barrier).
  // Lane value (mi, ni, v) sits at tile row wm*64 + mi*16 + 4*lk + v and
  // tile column wn*64 + ni*16 + lrow.
  if (EPI == MOE_EPI_SWIGLU_FP8) {
    // up waves (wn >= 2) hand their accumulators to the gate waves through LDS
    float* upt = reinterpret_cast<float*>(smem);             // [128][128 + 4]
    float* red = reinterpret_cast<float*>(smem + 128 * 132 * 4);  // [2][128]
    uint8_t* otile = smem + 128 * 132 * 4 + 1024;              // [128][128] codes
    constexpr int ldu = 132;
    if (wn >= 2) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            upt[(wm * 64 + mi * 16 + 4 * lk + v) * ldu + (wn - 2) * 64 + ni * 16 + lrow] =
                acc[mi][ni][v];
    }
    __syncthreads();
    float h[4][4][4];
    if (wn < 2) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float mx = 0.0f;
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const float gt = acc[mi][ni][v];
            const float u = upt[(wm * 64 + mi * 16 + 4 * lk + v) * ldu + wn * 64 + ni * 16 + lrow];
            const float e = expf(-gt);
            const float sg = 1.0f / (1.0f + e);
            const float silu = gt * sg;
            const float hv = silu * u;
            h[mi][ni][v] = hv;
            mx = fmaxf(mx, fabsf(hv));
          }
          mx = group_max<16>(mx);
          if (lrow == 0) red[wn * 128 + wm * 64 + mi * 16 + 4 * lk + v] = mx;
        }
    }
    __syncthreads();
    if (wn < 2) {
      const int ld_d = p.n_out / BN;  // h scale row stride (h has n_out/2 columns)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = wm * 64 + mi * 16 + 4 * lk + v;
          const float amax = fmaxf(red[row], red[128 + row]);
          float m, d;
          tile_scale(amax, m, d);
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            otile[row * 128 + wn * 64 + ni * 16 + lrow] = (uint8_t)quant_code(h[mi][ni][v], m);
          if (wn == 0 && lrow == 0 && m0 + row < rows_g)
            p.out_d[(long long)(row0 + m0 + row) * ld_d + n_tile] = d;
        }
    }
    __syncthreads();
    uint8_t* out = static_cast<uint8_t*>(p.out);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + kThreads * j;
      const int row = q >> 3, c = q & 7;
      if (m0 + row < rows_g)
        *reinterpret_cast<uint4*>(out + (long long)(row0 + m0 + row) * p.ldo + n_tile * 128 + c * 16) =
            *reinterpret_cast<const uint4*>(otile + row * 128 + c * 16);
    }
  } else if (EPI == MOE_EPI_BF16) {
    uint16_t* otile = reinterpret_cast<uint16_t*>(smem);   // [128][256] bf16
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 64 + mi * 16 + 4 * lk + v;
        float rs = 1.0f;
        if (p.row_scale) rs = p.row_scale[row0 + min(m0 + row, rows_g - 1)];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          const float val = p.row_scale ? acc[mi][ni][v] * rs : acc[mi][ni][v];
          otile[row * 256 + wn * 64 + ni * 16 + lrow] = (uint16_t)f32_to_bf16(val);
        }
      }
    __syncthreads();
    uint16_t* out = static_cast<uint16_t*>(p.out);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = tid + kThreads * j;
      const int row = q >> 5, c = q & 31;
      if (m0 + row < rows_g && n_tile * BN + c * 8 < p.n_out)
        *reinterpret_cast<uint4*>(out + (long long)(row0 + m0 + row) * p.ldo + n_tile * BN + c * 8) =
            *reinterpret_cast<const uint4*>(otile + row * 256 + c * 8);
    }
  } else {
    float* out = static_cast<float*>(p.out);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 64 + mi * 16 + 4 * lk + v;
        if (m0 + row < rows_g && wave_cols) {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            out[(long long)(row0 + m0 + row) * p.ldo + n_tile * BN + wn * 64 + ni * 16 + lrow] =
                acc[mi][ni][v];
        }
      }
  }
}

template <int EPI>
moe_status_t launch(const GemmParams& p, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&grouped_gemm_kernel<EPI>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return hip_fail(e);
    attr_set = true;
  }
  const long long n_tiles = (p.n_out + BN - 1) / BN;
  long long grid = ((long long)(p.total_rows + BM - 1) / BM + p.G) * n_tiles;
  grid = (grid + 7) / 8 * 8;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(grouped_gemm_kernel<EPI>, dim3((unsigned)grid), dim3(kThreads), kLds, stream, p);
  return launch_status();
}

}  // namespace

extern "C" moe_status_t moe_grouped_gemm_fp8(const moe_gemm_fp8_args* a, hipStream_t stream) {
  if (!a) return MOE_ERR_NULL;
  if (a->num_groups < 1 || a->num_groups > kMaxGroups || a->total_rows < 0 || a->n_out <= 0 ||
      a->k_dim <= 0 || a->k_dim % BK != 0 || a->n_out % 128 != 0 || a->lda < a->k_dim ||
      a->lda % 16 != 0 || a->a_rows < 0)
    return MOE_ERR_SHAPE;
  if (a->epilogue != MOE_EPI_BF16 && a->epilogue != MOE_EPI_SWIGLU_FP8 && a->epilogue != MOE_EPI_F32)
    return MOE_ERR_UNSUPPORTED;
  if (a->epilogue == MOE_EPI_SWIGLU_FP8 && a->n_out % BN != 0) return MOE_ERR_SHAPE;
  if (a->total_rows == 0) return MOE_OK;
  if (a->a_rows == 0) return MOE_ERR_SHAPE;
  if (!a->a_q || !a->a_d || !a->b_q || !a->b_d || !a->group_offsets || !a->out) return MOE_ERR_NULL;
  if (a->epilogue == MOE_EPI_SWIGLU_FP8 && !a->out_d) return MOE_ERR_NULL;
  const long long min_ldo = a->epilogue == MOE_EPI_SWIGLU_FP8 ? a->n_out / 2 : a->n_out;
  if (a->ldo < min_ldo) return MOE_ERR_SHAPE;
  if (a->epilogue == MOE_EPI_SWIGLU_FP8 ? (a->ldo % 16 != 0) : (a->ldo % 8 != 0))
    return MOE_ERR_SHAPE;
  if (!aligned16(a->a_q) || !aligned16(a->b_q) || !aligned16(a->out)) return MOE_ERR_ALIGN;
  if (moe_status_t s = check_device()) return s;
  GemmParams p;
  p.a_q = a->a_q; p.a_d = a->a_d; p.lda = a->lda; p.a_rows = a->a_rows;
  p.a_row_index = a->a_row_index; p.b_q = a->b_q; p.b_d = a->b_d;
  p.offsets = a->group_offsets; p.G = a->num_groups; p.total_rows = a->total_rows;
  p.n_out = a->n_out; p.k_dim = a->k_dim; p.out = a->out; p.out_d = a->out_d;
  p.ldo = a->ldo; p.row_scale = a->row_scale;
  switch (a->epilogue) {
    case MOE_EPI_SWIGLU_FP8: return launch<MOE_EPI_SWIGLU_FP8>(p, stream);
    case MOE_EPI_BF16: return launch<MOE_EPI_BF16>(p, stream);
    default: return launch<MOE_EPI_F32>(p, stream);
  }
}

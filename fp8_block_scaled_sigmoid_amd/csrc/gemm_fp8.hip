// Grouped block-scaled FP8 GEMM for the routed and shared experts.
//
// What it computes ("DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing,
// Multi-Token Prediction, and FP8 Training at 671B Scale", section V, Figure 6
// and FP8 details 1-2; "DeepSeek-V3, explained.", recipe step 7): E4M3
// operands with one scale per 1x128 activation tile and per 128x128 weight
// block, float accumulation, bf16 (or re-quantised E4M3) output.  The pages
// promote partial sums to FP32 every 128 products because their tensor cores
// accumulate with ~14 bits.  CDNA4 has the same kind of limit inside one MFMA
// (each group of 8 products is summed on a grid 2^-13 below its largest
// product), and the scales change every 128 elements of K anyway, so each
// 128-deep block is one v_mfma_f32_16x16x128_f8f6f4 into a zero accumulator,
// folded into the float running sum with one fused multiply-add by
// d_A[row, kb] * d_B[col block, kb].
//
// Two kernels compute it, with the same per-output arithmetic (so the same
// results bit for bit): grouped_gemm256_kernel (256 x 256 tiles, below the
// 128-row kernel) for the SwiGLU and bf16 epilogues when the groups hold at
// least 128 rows on average, and grouped_gemm_kernel (128 x 256 tiles) for
// small groups and the float32 epilogue.
//
// Layout and schedule of the 128-row kernel:
//   * a workgroup of 8 waves (two per SIMD, so one wave's LDS reads overlap
//     the other's MFMAs) computes a 128 x 256 output tile of one group
//     (expert); wave (wm, wn) owns 64 rows x 64 columns = 4 x 4 MFMA subtiles,
//     inside one 128x128 weight block, so it needs one B scale per K block;
//     its 64 float accumulators stay in VALU registers;
//   * the A tile (128 rows x 128 B, gathered through a_row_index) and the B
//     tile (256 x 128 B) of a K block are copied global -> LDS by
//     buffer-resource direct-to-LDS loads whose per-lane offset is fixed and
//     whose K position is the scalar offset, three stages deep: stage kb + 2
//     is requested in parts spread over the MFMAs of stage kb, and each wave
//     waits with an explicit vmcnt for exactly the stage it needs next; the A
//     scales come 8 K blocks at a time (a [128 rows][8] window, two windows
//     double-buffered), one 16-byte copy per lane pair of waves 0-3 riding
//     with the first stage of each window, so a copy touches 32 rows' cache
//     lines once per 8 K blocks instead of 64 every K block;
//   * LDS rows are 128 B; 16-byte chunk c of row r sits at chunk position
//     c ^ ((r >> 1) & 7), and each direct-to-LDS load writes 1 KiB of
//     consecutive LDS (8 rows); MFMA lane group lk reads K chunks lk and lk + 4
//     (the same permutation of K for A and B), which keeps every ds_read_b128
//     free of bank conflicts;
//   * with the SwiGLU epilogue the B tile is the interleaved pair (gate block j,
//     up block j) of W1: waves wn < 2 hold gate, wn >= 2 hold up; each gate
//     wave and its up partner swap half of their subtiles through LDS so all
//     8 waves form h, and the 128 h columns of a row (one 1x128 quantisation
//     tile) meet in LDS for the tile maximum;
//   * two K-loop schedules (each measured faster for its case), chosen per
//     launch: the "ping-pong" loop, two wave groups alternating MFMA and
//     VALU/memory phases, for the SwiGLU epilogue (GEMM1) and contractions
//     longer than 2048; the single-group loop for the short ones (GEMM2),
//     where a workgroup may compute two adjacent column tiles of the same rows
//     one after the other, the second reusing the group lookup and the row
//     map, its first stage requested before the first tile's epilogue;
//   * every workgroup derives the tile list itself from the device-side group
//     offsets (tiles ordered group, column tile (or pair), row tile), so the
//     call needs no workspace and no host sync; consecutive row tiles of one
//     (expert, column tile) are mapped to the same XCD so their weight tile is
//     fetched from HBM once and re-read from that XCD's L2, and the last
//     group (the shared expert) is cut into 8 column parts spread over the 8
//     XCDs' runs so that no XCD gets all its full tiles; in a group's last
//     row tile, 16-row subtiles past the group's end skip their MFMAs (the K
//     loop is compiled for each count of live subtiles).
#include <type_traits>

#include "common.h"

namespace {

using namespace moe;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int kThreads = 512;                           // 8 waves, two per SIMD
constexpr int kMaxGroups = 1025;                        // up to 1024 experts + shared
constexpr int kMaxKb = 128;                             // K <= 16384
constexpr int kABytes = BM * BK;                        // 16 KiB
constexpr int kBBytes = BN * BK;                        // 32 KiB
constexpr int kStage = kABytes + kBBytes;               // 48 KiB
constexpr int kStages = 3;
constexpr int kSWin = 8;                                // K blocks per A-scale window
constexpr int kSWinBytes = BM * kSWin * 4;              // 4 KiB: [128 rows][8 K blocks]
constexpr int kSWinOff = kStages * kStage;              // A scales after the ring
// The single-group K loop keeps one K block's 128 A scales at the end of each
// of its stages instead: its reads are four 16-byte loads per K block, where
// the window's [row][8] layout would take sixteen 4-byte ones.
constexpr int kSStageBytes = BM * 4;
constexpr int kStageSG = kStage + kSStageBytes;          // single-group stage: + its 128 A scales
// dynamic LDS of each schedule: the ring and the two windows, or the ring of
// single-group stages
constexpr int lds_bytes(bool ping_pong) { return ping_pong ? kSWinOff + 2 * kSWinBytes : kStages * kStageSG; }

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
  int cols_per_wg;          // column tiles a workgroup computes one after the other (1 or 2)
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// A-scale window slot of a tile row and back (bits 0-1 and 2-3 swapped)
__device__ __forceinline__ int win_slot(int r) {
  return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3);
}

// Direct-to-LDS copies through a buffer resource: the per-lane byte offset is
// fixed for the whole K loop and the K position is the scalar offset, so
// issuing a copy costs no vector instructions.  Offsets past num_records read
// as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint8_t* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)l, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint8_t* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)l, 4, voff, soff, 0, 0);
}

// Wait until at most N of this wave's direct-to-LDS loads are outstanding and
// its LDS reads are done, then meet the other waves.  (The compiler does not
// track the LDS side of these loads, so the wait is explicit.)
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Row maxima of 16 values per lane (a[r], r = 0..15) over the 16 lanes of
// each row group, by recursive halving: at each of four exchanges (partner
// lane = lane ^ 15, ^ 7, ^ 2, ^ 1 within the 16) a lane keeps the half of its
// values picked by one bit of its lane index and sends the other half, so the
// lane with row-group index r ends with the maximum of value r over all 16
// lanes (60 instructions instead of 16 separate reductions).  The values are
// bit patterns of non-negative floats, whose order is the unsigned order.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t row_max16_halving(const uint32_t (&a)[16], int lrow) {
  uint32_t b[8], c[4], d[2];
  const bool s3 = lrow & 8, s2 = lrow & 4, s1 = lrow & 2, s0 = lrow & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    b[i] = max(s3 ? a[i + 8] : a[i], dpp<0x140>(s3 ? a[i] : a[i + 8]));    // row mirror: ^15
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c[i] = max(s2 ? b[i + 4] : b[i], dpp<0x141>(s2 ? b[i] : b[i + 4]));    // half mirror: ^7
#pragma unroll
  for (int i = 0; i < 2; ++i)
    d[i] = max(s1 ? c[i + 2] : c[i], dpp<0x4E>(s1 ? c[i] : c[i + 2]));     // quad perm: ^2
  return max(s0 ? d[1] : d[0], dpp<0xB1>(s0 ? d[0] : d[1]));               // quad perm: ^1
}

// ---- the tile list.  Tiles are ordered (group, column tile, row tile): group
// g owns ceil(rows_g / BMt) row tiles for each of its n_cols column tiles,
// and consecutive row tiles of one column tile are consecutive in the list.
// Dispatch sends workgroup b to XCD b % 8, and each XCD takes a contiguous
// run of the list, so the row tiles that share a weight tile run on one XCD
// and re-read it from that XCD's L2.  The last group (the shared expert of
// the layer: T rows, every one a full tile) would put all its tiles on the
// last XCD, which would then finish last; with at least 8 other groups and 8
// column tiles it is cut into 8 parts of n_cols / 8 column tiles, part j
// placed after group (j + 1) (G - 1) / 8 - 1, so every XCD's run holds one
// part.  Thread t counts the tiles that follow groups t * per .. t * per +
// per - 1 in the list (per <= 3); a wave-level scan and one pass over the 8
// wave totals give every thread the exclusive prefix of its groups, and the
// thread whose range holds this workgroup's tile publishes the group, the
// tile's index inside the group's part, and the part's first column tile.
// Returns false when this workgroup has no tile (the same in all its
// threads).
template <int BMt>
__device__ __forceinline__ bool find_tile(const GemmParams& p, int n_cols, int* s_tmp, int tid,
                                          int lane, int wave, int& g, int& local, int& col0) {
  const int G = p.G;
  const bool split = G >= 9 && n_cols >= 8;
  const int last = G - 1;
  int last_mt = 0;
  if (split) {
    const int r0 = clampi(p.offsets[last], 0, p.total_rows);
    const int r1 = clampi(p.offsets[last + 1], 0, p.total_rows);
    last_mt = ((r1 > r0 ? r1 - r0 : 0) + BMt - 1) / BMt;
  }
  const int per = (G + kThreads - 1) / kThreads;   // <= 3
  int cnt[3], own[3], part[3];
  int run = 0;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int gi = tid * per + i;
    int c = 0, pj = -1;
    if (i < per && gi < G && !(split && gi == last)) {
      const int r0 = clampi(p.offsets[gi], 0, p.total_rows);
      const int r1 = clampi(p.offsets[gi + 1], 0, p.total_rows);
      const int rows = r1 > r0 ? r1 - r0 : 0;
      c = ((rows + BMt - 1) / BMt) * n_cols;
      if (split) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (((j + 1) * last) / 8 - 1 == gi) pj = j;
      }
    }
    own[i] = c;
    part[i] = pj;
    if (pj >= 0) c += last_mt * ((pj + 1) * n_cols / 8 - pj * n_cols / 8);
    cnt[i] = c;
    run += c;
  }
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s_tmp[wave] = incl;
  __syncthreads();
  int base = incl - run, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int t = s_tmp[w];
    if (w < wave) base += t;
    total += t;
  }
  const int per_xcd = (total + 7) / 8;
  const int slot = blockIdx.x >> 3, xcd = blockIdx.x & 7;
  const int L = xcd * per_xcd + slot;
  if (slot >= per_xcd || L >= total) return false;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int gi = tid * per + i;
    if (i < per && gi < G && L >= base && L < base + cnt[i]) {
      const bool in_part = L >= base + own[i];
      s_tmp[8] = in_part ? last : gi;
      s_tmp[9] = in_part ? L - base - own[i] : L - base;
      s_tmp[10] = in_part ? part[i] * n_cols / 8 : 0;
    }
    base += cnt[i];
  }
  __syncthreads();
  g = __builtin_amdgcn_readfirstlane(s_tmp[8]);
  local = __builtin_amdgcn_readfirstlane(s_tmp[9]);
  col0 = __builtin_amdgcn_readfirstlane(s_tmp[10]);
  return true;
}

template <int EPI, bool PING_PONG>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(GemmParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_tmp[kThreads];
  __shared__ float s_bd[2][kMaxKb];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int n_tiles = (p.n_out + BN - 1) / BN;   // the last tile may be 128 wide
  // PING_PONG: the ping-pong K loop on one column tile; otherwise the
  // single-group K loop on one column tile or (cols_per_wg = 2, chosen by
  // the host) two adjacent ones of the same rows, one after the other (the
  // second reuses the group lookup and the row map, so it starts with its
  // copies)
  constexpr bool kPingPong = PING_PONG;
  constexpr int kMaxPer = kPingPong ? 1 : 2;
  const int per = kPingPong ? 1 : (p.cols_per_wg == 2 ? 2 : 1);
  const int n_cols = (n_tiles + per - 1) / per;

  int g, local, col0;
  if (!find_tile<BM>(p, n_cols, s_tmp, tid, lane, wave, g, local, col0)) return;
  const int row0 = clampi(p.offsets[g], 0, p.total_rows);
  const int rows_g = clampi(p.offsets[g + 1], 0, p.total_rows) - row0;
  const int mt = (rows_g + BM - 1) / BM;
  const int col_l = local / mt;
  const int col = col0 + col_l;                         // column tile (or pair)
  const int m0 = (local - col_l * mt) * BM;
  const int rows_valid = min(BM, rows_g - m0);
  const int nkb = p.k_dim / BK;
  const int n_here = min(per, n_tiles - per * col);     // column tiles of this workgroup

  // ---- direct-to-LDS sources.  Load j of wave w writes 1 KiB block
  // b = 8 j + w (rows 8 b .. 8 b + 7); lane l fills row 8 b + (l >> 3) at chunk
  // position l & 7, i.e. it fetches chunk (l & 7) ^ ((row >> 1) & 7), which
  // is the same for every j of this lane.
  const int chunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow8 = 8 * wave + (lane >> 3);            // row inside each 64-row band
  const int nkb_all = p.k_dim / BK;
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.a_q, (int)(p.a_rows * p.lda));
  const __amdgpu_buffer_rsrc_t rs_sa = make_rsrc(p.a_d, p.a_rows * nkb_all * 4);
  int a_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = row0 + min(m0 + 64 * j + lrow8, rows_g - 1);
    int src = p.a_row_index ? p.a_row_index[r] : r;
    src = clampi(src, 0, p.a_rows - 1);
    a_off[j] = (int)((long long)src * p.lda) + chunk * 16;
  }
  // A scales.  Ping-pong loop: 8 K blocks at a time (32 contiguous bytes of a
  // row of a_d): waves 0-3 each load 32 window slots with one 16-byte copy,
  // lane l filling slot 32 w + l / 2 with K blocks 4 (l & 1) .. + 3 (LDS
  // [slot][8]).  Slot and row differ by a swap of the two lowest 2-bit fields
  // (win_slot, its own inverse), so the rows 4 apart that the four MFMA lane
  // groups read together sit 8 floats apart in LDS, in different banks (in
  // row order they would be 128 bytes apart, on the same banks).
  // Single-group loop: waves 0-1 load one K block's scale of 64 rows each
  // with one 4-byte copy per lane, every K block.
  int sw_off = 0;
  if (kPingPong ? wave < 4 : wave < 2) {
    const int r = kPingPong ? row0 + min(m0 + win_slot(32 * wave + (lane >> 1)), rows_g - 1)
                            : row0 + min(m0 + 64 * wave + lane, rows_g - 1);
    int src = p.a_row_index ? p.a_row_index[r] : r;
    src = clampi(src, 0, p.a_rows - 1);
    sw_off = src * nkb_all * 4 + (kPingPong ? (lane & 1) * 16 : 0);
  }
  // The B side of column tile n: the block scales of both of its weight
  // blocks for every K block (into s_bd), its buffer resource and the lanes'
  // offsets.  Set per column tile; the copy lambdas read them.
  __amdgpu_buffer_rsrc_t rs_b = make_rsrc(p.b_q, 0);
  int b_off[4];
  auto setup_b = [&](int n) {
    const bool half = p.n_out - n * BN < BN;              // only 128 columns exist
    for (int i = tid; i < 2 * nkb; i += kThreads) {
      const int blk = i / nkb, kb = i - blk * nkb;
      const int nb = min(2 * n + blk, p.n_out / 128 - 1);
      s_bd[blk][kb] = p.b_d[((long long)g * (p.n_out / 128) + nb) * nkb + kb];
    }
    const int b_rows = half ? 128 : BN;
    rs_b = make_rsrc(p.b_q + ((long long)g * p.n_out + (long long)n * BN) * p.k_dim, b_rows * p.k_dim);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int jj = half ? (j & 1) : j;                  // past n_out: repeat valid rows
      b_off[j] = (lrow8 + 64 * jj) * p.k_dim + chunk * 16;
    }
  };
  // The single-group schedule with the bf16 epilogue requests the first
  // stage of a workgroup's second column tile before the first tile's
  // epilogue, so its latency hides behind it (the epilogue then stages its
  // output through ring slots 1-2 only).
  bool prefetched = false;
#pragma unroll
  for (int hh = 0; hh < kMaxPer; ++hh) {
  if (hh >= n_here) break;
  const int n_tile = per * col + hh;
  const bool half_tile = p.n_out - n_tile * BN < BN;   // only 128 columns exist
  if (hh > 0) __syncthreads();   // the previous tile's epilogue is done with LDS
  if (!prefetched) setup_b(n_tile);

  // the copies of one stage, in four parts so they can be spread over a K
  // block's MFMAs: part 0 the A tile, parts 1-2 the B tile, part 3 the A scales
  auto issue_part = [&](int kb, uint8_t* st, int part) {
    const int ko = kb * BK;
    if (part == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) dma16(rs_a, a_off[j], ko, st + (8 * j + wave) * 1024);
    } else if (part < 3) {
#pragma unroll
      for (int j = 2 * part - 2; j < 2 * part; ++j)
        dma16(rs_b, b_off[j], ko, st + kABytes + (8 * j + wave) * 1024);
    } else if constexpr (kPingPong) {
      if (wave < 4 && kb % kSWin == 0)
        dma16(rs_sa, sw_off, kb * 4, smem + kSWinOff + ((kb / kSWin) & 1) * kSWinBytes + wave * 1024);
    } else if (wave < 2) {
      dma4(rs_sa, sw_off, kb * 4, st + kABytes + kBBytes + wave * 256);
    }
  };
  auto issue = [&](int kb, uint8_t* st) {
#pragma unroll
    for (int part = 0; part < 4; ++part) issue_part(kb, st, part);
  };
  // copy i (0-5) of this wave's A and B share of a stage: A loads 0-1, B loads 0-3
  auto issue_one = [&](int kb, uint8_t* st, int i) {
    const int ko = kb * BK;
    if (i < 2) dma16(rs_a, a_off[i], ko, st + (8 * i + wave) * 1024);
    else dma16(rs_b, b_off[i - 2], ko, st + kABytes + (8 * (i - 2) + wave) * 1024);
  };

  // ---- wave tile: rows wm*64..+64, B-tile rows wn*64..+64; wn < 2 lies in
  // weight block 0 (gate), wn >= 2 in block 1 (up)
  const int wm = wave & 1, wn = wave >> 1;
  const int lrow = lane & 15, lk = lane >> 4;
  // byte offset of this lane's K chunks lk and lk + 4 in row lrow of a
  // 16-row subtile (swz() of that row and chunk)
  const int frag_lo = lrow * 128 + ((lk ^ ((lrow >> 1) & 7)) << 4);
  const int frag_hi = lrow * 128 + (((lk + 4) ^ ((lrow >> 1) & 7)) << 4);
  const int wave_rows = rows_valid - wm * 64;          // <= 0: nothing to compute
  const bool wave_cols = !(half_tile && wn >= 2);

  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The K loop, for a wave whose first NMI 16-row subtiles hold valid rows
  // (the others are padding of a group's last row tile and skip their MFMAs).
  //
  // Two wave groups take turns ("ping-pong"): waves 0-3 and waves 4-7 each
  // hold one wave per SIMD.  Every K block kb has two phases; in each phase
  // one group issues the 16 MFMAs of its
  // K block while the other, on the same SIMDs, runs the VALU and memory work:
  // the scale FMAs of its previous MFMAs, its share of the copies of a later
  // stage, and the LDS reads of its next fragments.  So the MFMA pipe and the
  // VALU / LDS / TA paths of every SIMD are busy at the same time.
  //   phase E_kb: group 0 MFMAs of kb;  group 1 FMAs of kb-1, copies of stage
  //               kb+2, reads of kb;  then every wave waits for its copies of
  //               stage kb+1 and its LDS reads;
  //   phase O_kb: group 1 MFMAs of kb;  group 0 FMAs of kb, copies of stage
  //               kb+3, reads of kb+1.
  // Stage kb (ring slot kb % 3) is read by group 0 in O_kb-1 and by group 1
  // in E_kb, so its slot is free from O_kb on.  Only the end of E_kb is a
  // workgroup barrier.  The end of O_kb needs none: group 1 may start
  // E_kb+1 while group 0 is still in O_kb, and what both then do is read
  // stage kb + 1 (landed at the barrier) and copy into slot kb % 3 (free since
  // that barrier); the scale window a group-0 copy refills was last read eight
  // K blocks earlier.
  auto kloop = [&](auto nmi_c) {
    constexpr int NMI = decltype(nmi_c)::value;
    const bool g1 = wave >= 4;
    // copies this wave issues for stage s: 6, plus the scale window (waves 0-3)
    // when s starts a window
    auto n_of = [&](int s) { return 6 + ((wave < 4 && s % kSWin == 0) ? 1 : 0); };
    i32x8 af[4], bfr[4];
    f32x4 part[4][4], sc[4];
    float sbv = 0.0f;
    // MFMA lane group lk takes the 16-byte K chunks lk and lk + 4 of its row,
    // for A and B alike (a fixed permutation of K inside the block, so the
    // dot product is unchanged); this keeps each ds_read_b128 free of LDS bank
    // conflicts, which chunks 2 lk and 2 lk + 1 are not.  Subtile rows differ
    // by multiples of 16, so a lane's swizzle term is the same in every
    // subtile: one lane offset per chunk half.
    auto read_frags = [&](int kb) {
      const uint8_t* st = smem + (kb % kStages) * kStage;
      const uint8_t* a_lo = st + wm * 64 * 128 + frag_lo;
      const uint8_t* a_hi = st + wm * 64 * 128 + frag_hi;
      const uint8_t* b_lo = st + kABytes + wn * 64 * 128 + frag_lo;
      const uint8_t* b_hi = st + kABytes + wn * 64 * 128 + frag_hi;
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) {
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(a_lo + mi * 16 * 128);
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(a_hi + mi * 16 * 128);
        af[mi] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const i32x4 y0 = *reinterpret_cast<const i32x4*>(b_lo + ni * 16 * 128);
        const i32x4 y1 = *reinterpret_cast<const i32x4*>(b_hi + ni * 16 * 128);
        bfr[ni] = __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    // the row scales of every accumulator row of this lane, and the block
    // scale; they are multiplied in the next MFMA phase (scale_rows), so no
    // phase waits for these reads
    auto read_scales = [&](int kb) {
      // row wm 64 + mi 16 + 4 lk + v lives in window slot wm 64 + mi 16 + 4 v + lk
      const float* sA = reinterpret_cast<const float*>(smem + kSWinOff + ((kb / kSWin) & 1) * kSWinBytes) +
                        (wm * 64 + lk) * kSWin + (kb % kSWin);
      sbv = s_bd[wn >> 1][kb];
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[mi][v] = sA[(mi * 16 + 4 * v) * kSWin];
    };
    auto scale_rows = [&]() {
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) sc[mi] = sc[mi] * sbv;
    };
    auto mfma = [&]() {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int mi = 0; mi < NMI; ++mi)
          part[ni][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[mi], bfr[ni], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
    };
    auto fma = [&]() {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[mi][ni][v] = __builtin_fmaf(part[ni][mi][v], sc[mi][v], acc[mi][ni][v]);
    };
    // scale FMAs of (column subtile, row subtile) pairs q0 .. q1 - 1
    auto fma_pairs = [&](int q0, int q1) {
#pragma unroll
      for (int q = 0; q < 4 * NMI; ++q) {
        if (q < q0 || q >= q1) continue;
        const int ni = q / (NMI > 0 ? NMI : 1), mi = q - ni * NMI;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[mi][ni][v] = __builtin_fmaf(part[ni][mi][v], sc[mi][v], acc[mi][ni][v]);
      }
    };
    // The VALU / memory phase, in segments the compiler may not reorder:
    // eight slices of the scale FMAs, with one copy of a later stage before
    // each of the first six (so the address unit drains while the FMAs run)
    // and the fragment reads of K block kb_read spread over the first four
    // (A and B fragment i in slice i: their registers are free once the
    // MFMAs are issued; spread out, the LDS queue drains behind the FMAs
    // instead of stalling the wave, and the last reads still land before the
    // phase ends); last the row scales of kb_read, into the registers the
    // FMAs free (nothing in this phase waits for them).
    auto xphase = [&](auto issue_c, auto fma_c, int kb_issue, uint8_t* slot, int kb_read) {
      constexpr bool ISSUE = decltype(issue_c)::value, FMA = decltype(fma_c)::value;
      if (ISSUE && wave < 4) issue_part(kb_issue, slot, 3);
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* rst = smem + (kb_read % kStages) * kStage;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (ISSUE) {
          if (i < 6) issue_one(kb_issue, slot, i);
        }
        if constexpr (NMI > 0) {
          if (i < 4) {
            if (i < NMI) {
              const i32x4 x0 = *reinterpret_cast<const i32x4*>(rst + wm * 64 * 128 + frag_lo + i * 16 * 128);
              const i32x4 x1 = *reinterpret_cast<const i32x4*>(rst + wm * 64 * 128 + frag_hi + i * 16 * 128);
              af[i] = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            const i32x4 y0 = *reinterpret_cast<const i32x4*>(rst + kABytes + wn * 64 * 128 + frag_lo + i * 16 * 128);
            const i32x4 y1 = *reinterpret_cast<const i32x4*>(rst + kABytes + wn * 64 * 128 + frag_hi + i * 16 * 128);
            bfr[i] = __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
        if constexpr (FMA && NMI > 0) fma_pairs(i * 4 * NMI / 8, (i + 1) * 4 * NMI / 8);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NMI > 0) read_scales(kb_read);
      __builtin_amdgcn_sched_barrier(0);
    };
    // end of an E phase: this wave's copies of stage kb + 1 have landed
    // (those of stage kb + 2 may be in flight) and its LDS reads are done.
    // (After E_0 the copies still in flight are the A part of stage 2 only:
    // the prologue requests the B parts of stages 0-2 first.)
    auto end_e = [&](int kb) {
      __builtin_amdgcn_sched_barrier(0);
      if (kb + 2 >= nkb) {
        wait_and_barrier<0>();
      } else if (kb == 0) {
        wait_and_barrier<2>();
      } else {
        if (n_of(kb + 2) == 7) wait_and_barrier<7>(); else wait_and_barrier<6>();
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    auto end_o = [&]() {
      __builtin_amdgcn_sched_barrier(0);
    };
    // every wave requests stages 0-2 (the B parts first: they do not wait
    // for the row map), then waits for stage 0
    const int npro = min(nkb, kStages);
    for (int st = 0; st < npro; ++st) {
      issue_part(st, smem + st * kStage, 1);
      issue_part(st, smem + st * kStage, 2);
    }
    for (int st = 0; st < npro; ++st) {
      issue_part(st, smem + st * kStage, 0);
      issue_part(st, smem + st * kStage, 3);
    }
    if (nkb > 2) {
      wait_and_barrier<4>();
    } else if (nkb > 1) {
      wait_and_barrier<2>();
    } else {
      wait_and_barrier<0>();
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    // (The loops are split where the copies stop, so no phase holds a branch;
    // after the last K block, group 0 reads a stale stage it does not use.)
    if (!g1) {
      if constexpr (NMI > 0) {
        read_frags(0);
        read_scales(0);
      }
      int kb = 0;
      for (; kb + 3 < nkb; ++kb) {
        mfma();                                                         // E_kb
        scale_rows();
        end_e(kb);
        xphase(yes, yes, kb + 3, smem + (kb % kStages) * kStage, kb + 1);   // O_kb
        end_o();
      }
      for (; kb < nkb; ++kb) {
        mfma();
        scale_rows();
        end_e(kb);
        xphase(no, yes, 0, smem, min(kb + 1, nkb - 1));
        end_o();
      }
    } else {
      xphase(no, no, 0, smem, 0);                                       // E_0
      end_e(0);
      mfma();                                                           // O_0
      scale_rows();
      end_o();
      int kb = 1;
      for (; kb + 2 < nkb; ++kb) {
        xphase(yes, yes, kb + 2, smem + ((kb + 2) % kStages) * kStage, kb);   // E_kb
        end_e(kb);
        mfma();                                                         // O_kb
        scale_rows();
        end_o();
      }
      for (; kb < nkb; ++kb) {
        xphase(no, yes, 0, smem, kb);
        end_e(kb);
        mfma();
        scale_rows();
        end_o();
      }
      fma();
    }
  };
  // The single-group K loop (bf16 and float32 epilogues): every wave runs
  // every K block; after one barrier per block it reads its fragments, and
  // for each column subtile issues the 4 MFMAs while the scale FMAs of the
  // previous subtile and one part of the copies of stage kb + 2 run behind
  // them.
  auto kloop_sg = [&](auto nmi_c, bool pre) {
    constexpr int NMI = decltype(nmi_c)::value;
    // one K block.  MORE: stage kb + 2 exists and is requested meanwhile;
    // LAST: no stage follows this one.
    auto kblock = [&](int kb, auto more_c, auto last_c) {
      constexpr bool more = decltype(more_c)::value, last = decltype(last_c)::value;
      // stage kb must have landed; stage kb + 1 may still be in flight (and,
      // when stage 0 was requested before the previous tile's epilogue, that
      // epilogue's 8 stores, which came between stages 0 and 1)
      if (!last) {
        if (pre && kb == 0) {
          if (wave < 2) wait_and_barrier<15>(); else wait_and_barrier<14>();
        } else {
          if (wave < 2) wait_and_barrier<7>(); else wait_and_barrier<6>();
        }
      } else {
        wait_and_barrier<0>();
      }
      uint8_t* st_next = smem + ((kb + 2) % kStages) * kStageSG;
      if (NMI == 0) {
        if (more) issue(kb + 2, st_next);
        return;
      }
      // MFMA lane group lk takes the 16-byte K chunks lk and lk + 4 of its
      // row, for A and B alike (a fixed permutation of K inside the block,
      // so the dot product is unchanged); this keeps each ds_read_b128 free
      // of LDS bank conflicts, which chunks 2 lk and 2 lk + 1 are not.
      // The A fragments, row scales and the first B fragment are read first;
      // then for each column subtile ni: the next B fragment is read and one
      // part of stage kb + 2 is requested while the 4 MFMAs of ni run, with
      // the scale FMAs of subtile ni - 1 behind them (no FMA waits on a
      // fresh result).
      // Subtile rows differ by multiples of 16, so a lane's swizzle term is
      // the same in every subtile: one lane offset per chunk half, and the
      // subtiles sit at constant offsets from it.
      const uint8_t* st = smem + (kb % kStages) * kStageSG;
      const float* sA = reinterpret_cast<const float*>(st + kABytes + kBBytes) + wm * 64 + 4 * lk;
      const float sb = s_bd[wn >> 1][kb];
      const uint8_t* a_lo = st + wm * 64 * 128 + frag_lo;
      const uint8_t* a_hi = st + wm * 64 * 128 + frag_hi;
      const uint8_t* b_lo = st + kABytes + wn * 64 * 128 + frag_lo;
      const uint8_t* b_hi = st + kABytes + wn * 64 * 128 + frag_hi;
      auto read_b = [&](int ni) {
        const i32x4 y0 = *reinterpret_cast<const i32x4*>(b_lo + ni * 16 * 128);
        const i32x4 y1 = *reinterpret_cast<const i32x4*>(b_hi + ni * 16 * 128);
        return __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      // read order = use order: A0 and B0 first, so the first MFMA waits for
      // four reads only, then the other A fragments, then the row scales
      // (first needed by the FMAs behind the second column subtile)
      f32x4 sc[4];
      i32x8 af[4], bfr[2];
      auto read_a = [&](int mi) {
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(a_lo + mi * 16 * 128);
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(a_hi + mi * 16 * 128);
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      af[0] = read_a(0);
      bfr[0] = read_b(0);
#pragma unroll
      for (int mi = 1; mi < NMI; ++mi) af[mi] = read_a(mi);
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) sc[mi] = *reinterpret_cast<const f32x4*>(sA + mi * 16);
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) sc[mi] = sc[mi] * sb;
      f32x4 part[2][4];
#pragma unroll
      for (int ni = 0; ni < 5; ++ni) {
        if (ni < 3) bfr[(ni + 1) & 1] = read_b(ni + 1);
        if (ni < 4 && more) issue_part(kb + 2, st_next, ni);
#pragma unroll
        for (int mi = 0; mi < NMI; ++mi) {
          if (ni < 4)
            part[ni & 1][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af[mi], bfr[ni & 1], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          if (ni > 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[mi][ni - 1][v] =
                  __builtin_fmaf(part[(ni - 1) & 1][mi][v], sc[mi][v], acc[mi][ni - 1][v]);
          }
        }
      }
    };
    if (!pre) issue(0, smem);
    if (nkb > 1) issue(1, smem + kStageSG);
    int kb = 0;
    for (; kb + 2 < nkb; ++kb) kblock(kb, std::true_type{}, std::false_type{});
    if (kb + 1 < nkb) kblock(kb++, std::false_type{}, std::false_type{});
    kblock(kb, std::false_type{}, std::true_type{});
  };
  const int nmi = wave_cols ? clampi((wave_rows + 15) >> 4, 0, 4) : 0;
  if constexpr (kPingPong) {
    switch (__builtin_amdgcn_readfirstlane(nmi)) {
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }
  } else {
    switch (__builtin_amdgcn_readfirstlane(nmi)) {
      case 4: kloop_sg(std::integral_constant<int, 4>{}, prefetched); break;
      case 3: kloop_sg(std::integral_constant<int, 3>{}, prefetched); break;
      case 2: kloop_sg(std::integral_constant<int, 2>{}, prefetched); break;
      case 1: kloop_sg(std::integral_constant<int, 1>{}, prefetched); break;
      default: kloop_sg(std::integral_constant<int, 0>{}, prefetched); break;
    }
  }
  __syncthreads();   // every wave is done with the stages before they are reused
  prefetched = false;
  if constexpr (!kPingPong && EPI == MOE_EPI_BF16) {
    if (hh + 1 < n_here && !p.row_scale) {
      setup_b(n_tile + 1);
      issue(0, smem);
      prefetched = true;
    }
  }

  // ---- epilogues.  Lane value (mi, ni, v) sits at tile row
  // wm*64 + mi*16 + 4*lk + v and tile column wn*64 + ni*16 + lrow.
  if (EPI == MOE_EPI_SWIGLU_FP8) {
    // Gate wave (wm, wn < 2) and up wave (wm, wn + 2) hold the same rows and
    // h columns.  Each hands the other half of its subtiles through LDS (gate
    // columns 2-3 to the up wave, up columns 0-1 to the gate wave), so all 8
    // waves form h = SiLU(gate) * up for two column subtiles each.  A row's
    // 128 h values (one 1x128 tile) then lie in 4 waves; their maxima meet in
    // LDS.
    float* ex = reinterpret_cast<float*>(smem);                   // [8 waves][32][64]
    float* red = reinterpret_cast<float*>(smem + 65536);          // [4][128] row maxima
    uint8_t* otile = smem + 65536 + 2048;                          // [128][128] codes
    const bool gate_wave = wn < 2;
    const int partner = gate_wave ? wave + 4 : wave - 4;           // wn +- 2
    const int keep0 = gate_wave ? 0 : 2;                           // subtiles kept
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          ex[(wave * 32 + (mi * 2 + j) * 4 + v) * 64 + lane] =
              gate_wave ? acc[mi][2 + j][v] : acc[mi][j][v];   // static indices: acc stays in registers
    __syncthreads();
    // 16-row subtiles past the group's end (wave-uniform) form no h
    float h[4][2][4];
    uint32_t mxb[16];   // per (mi, v): bits of max |h| over this lane's two columns
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const bool live = wm * 64 + mi * 16 < rows_valid;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          h[mi][j][v] = 0.0f;
          if (live) {
            const float mine = gate_wave ? acc[mi][j][v] : acc[mi][2 + j][v];
            const float other = ex[(partner * 32 + (mi * 2 + j) * 4 + v) * 64 + lane];
            const float gt = gate_wave ? mine : other;
            const float u = gate_wave ? other : mine;
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
            h[mi][j][v] = gt * sg * u;
            mx = fmaxf(mx, fabsf(h[mi][j][v]));
          }
        }
        mxb[mi * 4 + v] = __float_as_uint(mx);
      }
    }
    {
      // lane (lk, lrow) ends with the maximum of row (mi, v) = (lrow / 4, lrow % 4)
      const uint32_t mx = row_max16_halving(mxb, lrow);
      red[wn * 128 + wm * 64 + (lrow >> 2) * 16 + 4 * lk + (lrow & 3)] = __uint_as_float(mx);
    }
    __syncthreads();
    // one thread per row forms the tile's scale (two divisions) and stores d
    const int ld_d = p.n_out / BN;  // h scale row stride (h has n_out/2 columns)
    float* s_m = reinterpret_cast<float*>(smem + 65536 + 2048 + 16384);   // [128] multipliers
    if (tid < BM) {
      float m, d;
      tile_scale(fmaxf(fmaxf(red[tid], red[128 + tid]), fmaxf(red[256 + tid], red[384 + tid])), m, d);
      s_m[tid] = m;
      if (tid < rows_valid) p.out_d[(long long)(row0 + m0 + tid) * ld_d + n_tile] = d;
    }
    __syncthreads();
    const int hc = (wn & 1) * 64;   // this wave's 64-column half of the h tile
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (wm * 64 + mi * 16 >= rows_valid) continue;   // rows that are not stored
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 64 + mi * 16 + 4 * lk + v;
        const float m = s_m[row];
#pragma unroll
        for (int j = 0; j < 2; ++j)
          otile[row * 128 + hc + (keep0 + j) * 16 + lrow] = (uint8_t)quant_code(h[mi][j][v], m);
      }
    }
    __syncthreads();
    uint8_t* out = static_cast<uint8_t*>(p.out);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + kThreads * j;
      const int row = q >> 3, c = q & 7;
      if (row < rows_valid)
        *reinterpret_cast<i32x4*>(out + (long long)(row0 + m0 + row) * p.ldo + n_tile * 128 + c * 16) =
            *reinterpret_cast<const i32x4*>(otile + row * 128 + c * 16);
    }
  } else if (EPI == MOE_EPI_BF16) {
    // Staged through ring slots 1-2 (slot 0 may be receiving the next column
    // tile's first stage).  Every wave issues exactly 8 buffer stores; a lane
    // whose row or column lies outside the tile points past the buffer's end,
    // where the store is dropped.
    uint16_t* otile = reinterpret_cast<uint16_t*>(smem + (kPingPong ? 0 : kStageSG));   // [128][256] bf16
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      if (wm * 64 + mi * 16 >= rows_valid) continue;   // rows that are not stored
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
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rs_o =
        make_rsrc(static_cast<uint16_t*>(p.out) + (long long)(row0 + m0) * p.ldo, rows_valid * (int)p.ldo * 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = tid + kThreads * j;
      const int row = q >> 5, c = q & 31;
      const int colx = n_tile * BN + c * 8;
      const int off = colx < p.n_out ? (row * (int)p.ldo + colx) * 2 : 0x7FFFFFF0;
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const i32x4*>(otile + row * 256 + c * 8),
                                             rs_o, off, 0, 0);
    }
  } else {
    float* out = static_cast<float*>(p.out);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 64 + mi * 16 + 4 * lk + v;
        if (row < rows_valid && wave_cols) {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni)
            out[(long long)(row0 + m0 + row) * p.ldo + n_tile * BN + wn * 64 + ni * 16 + lrow] =
                acc[mi][ni][v];
        }
      }
  }

  }
}

// ---- 256-row tiles for the SwiGLU and bf16 epilogues -----------------------
// A workgroup of 8 waves computes a 256 x 256 tile: up to 256 rows of one
// group (its rows split evenly over its row tiles) by two 128-column weight
// blocks (with the SwiGLU epilogue the interleaved gate/up pair); wave
// (wm, wn) owns rows wm*64..+64 and the 128 columns of weight block wn: 4 x 8
// MFMA subtiles, 128 float accumulators.  Per 8.4 MFLOP it moves 16 KiB of A and 16 KiB of B
// through the compute unit's L1 instead of the 128-row tile's 16 + 32 KiB:
// each weight line is read once per 256 rows, not twice.
//   * LDS: two 64 KiB stages (A 256 x 128 B, B 256 x 128 B, rows laid out as
//     in the 128-row kernel), two A-scale windows [256 slots][8 K blocks] and a
//     dummy block; 152 KiB.
//   * Each stage is requested in two parts, by when its slot becomes free.
//     During K block kb the slot of stage kb holds A (read at the block's
//     start) and B (read one column subtile at a time).  After a mid-block
//     barrier (every wave has read A and B rows 0-63 of both weight blocks),
//     those rows of the slot take stage kb + 2 (the early part: B rows 0-63
//     and 128-191, A, the scale window); at the start of K block kb + 1 the
//     rest (B rows 64-127, 192-255) follows.  So one and a half stages are in
//     flight, which the two-stage ring could not give with whole stages.
//   * Every stage issues the same number of copies in every wave (the window
//     copy goes out of range into the dummy block off the first K block of a
//     window, and the A copies of a 64-row band wholly past the group's end go
//     out of range), so each wait has a fixed count.
//   * Inside a column subtile each MFMA is followed by the 4 scale FMAs of the
//     previous subtile's same row subtile, so the VALU works while the wave's
//     own MFMAs run (the partials are double-buffered).
//   * The two waves of a row band are adjacent (wm = (w >> 1) & 3, wn = w & 1),
//     so they run on different SIMDs (wave w runs on SIMD w % 4) and a tile
//     with few live rows still uses two SIMDs per band.
//   * Epilogues: SwiGLU + 1x128 requantisation (the gate and up waves of a
//     band swap half their columns through LDS) or bf16 (staged through LDS);
//     both write with coalesced 16-byte stores.
constexpr int BM256 = 256;
constexpr int kA256 = BM256 * BK;                       // 32 KiB
constexpr int kStage256 = kA256 + kBBytes;              // 64 KiB
constexpr int kSWin256 = BM256 * kSWin * 4;             // 8 KiB
constexpr int kSWinOff256 = 2 * kStage256;              // 128 KiB
constexpr int kDummy256 = kSWinOff256 + 2 * kSWin256;   // takes the dropped window copies
constexpr int kLds256 = kDummy256 + 8 * 1024;           // 152 KiB
static_assert(256 * 264 * 2 <= kLds256, "the bf16 epilogue's staging tile fits");

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm256_kernel(GemmParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_tmp[kThreads];
  __shared__ float s_bd[2][kMaxKb];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int n_tiles = p.n_out / BN;
  int g, local, col0;
  if (!find_tile<BM256>(p, n_tiles, s_tmp, tid, lane, wave, g, local, col0)) return;
  const int row0 = clampi(p.offsets[g], 0, p.total_rows);
  const int rows_g = clampi(p.offsets[g + 1], 0, p.total_rows) - row0;
  // A group's rows are split evenly over its ceil(rows / 256) row tiles (291
  // rows: 146 + 145, not 256 + 35).  The row tiles of one weight tile run
  // side by side on one XCD and share its lines in L2 only while they stay in
  // step; a nearly empty last tile would run ahead and fetch them again.
  const int mt = (rows_g + BM256 - 1) / BM256;
  const int n_tile_l = local / mt;
  const int n_tile = col0 + n_tile_l;
  const int rt = local - n_tile_l * mt;
  const int m0 = (int)((long long)rt * rows_g / mt);
  const int rows_valid = (int)((long long)(rt + 1) * rows_g / mt) - m0;   // <= 256
  const int nkb = p.k_dim / BK;

  // ---- direct-to-LDS sources: copy j of wave w fills rows 64 j + 8 w .. + 7
  // of the A or B tile (1 KiB), as in the 128-row kernel
  const int chunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow8 = 8 * wave + (lane >> 3);
  const __amdgpu_buffer_rsrc_t rs_a = make_rsrc(p.a_q, (int)(p.a_rows * p.lda));
  const __amdgpu_buffer_rsrc_t rs_sa = make_rsrc(p.a_d, p.a_rows * nkb * 4);
  int a_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = row0 + min(m0 + 64 * j + lrow8, rows_g - 1);
    int src = p.a_row_index ? p.a_row_index[r] : r;
    src = clampi(src, 0, p.a_rows - 1);
    a_off[j] = (int)((long long)src * p.lda) + chunk * 16;
    // a band wholly past the group's end is read by no wave: out of range
    // (dropped without a fetch; K block offsets stay below 2^14)
    if (64 * j >= rows_valid) a_off[j] = 0x7FFFFFF0 - 16384;
  }
  // A-scale window of 8 K blocks: lane pair (2 s, 2 s + 1) of wave w fills
  // slot 32 w + s with K blocks 0-3 / 4-7 of row win_slot(32 w + s)
  int sw_off;
  {
    const int r = row0 + min(m0 + win_slot(32 * wave + (lane >> 1)), rows_g - 1);
    int src = p.a_row_index ? p.a_row_index[r] : r;
    src = clampi(src, 0, p.a_rows - 1);
    sw_off = src * nkb * 4 + (lane & 1) * 16;
  }
  for (int i = tid; i < 2 * nkb; i += kThreads) {
    const int blk = i / nkb, kb = i - blk * nkb;
    s_bd[blk][kb] = p.b_d[((long long)g * (p.n_out / 128) + 2 * n_tile + blk) * nkb + kb];
  }
  const __amdgpu_buffer_rsrc_t rs_b =
      make_rsrc(p.b_q + ((long long)g * p.n_out + (long long)n_tile * BN) * p.k_dim, BN * p.k_dim);
  const int b_off = lrow8 * p.k_dim + chunk * 16;   // copy j adds 64 j rows in the scalar offset

  auto cp_a = [&](int kb, int j) {
    dma16(rs_a, a_off[j], kb * BK, smem + (kb & 1) * kStage256 + (8 * j + wave) * 1024);
  };
  auto cp_b = [&](int kb, int j) {
    dma16(rs_b, b_off, kb * BK + 64 * j * p.k_dim, smem + (kb & 1) * kStage256 + kA256 + (8 * j + wave) * 1024);
  };
  auto cp_w = [&](int kb) {
    const bool w = kb % kSWin == 0;
    dma16(rs_sa, sw_off, w ? kb * 4 : 0x7FFFFFF0,
          smem + (w ? kSWinOff256 + ((kb / kSWin) & 1) * kSWin256 : kDummy256) + wave * 1024);
  };
  // copy i of this wave's share of stage kb: the early part is i 0-6 (B rows
  // 0-63, B rows 128-191, A 0-3, the window), the late part i 7-8 (B rows
  // 64-127, 192-255)
  auto cp = [&](int kb, int i) {
    if (i == 0) cp_b(kb, 0);
    else if (i == 1) cp_b(kb, 2);
    else if (i < 6) cp_a(kb, i - 2);
    else if (i == 6) cp_w(kb);
    else if (i == 7) cp_b(kb, 1);
    else cp_b(kb, 3);
  };

  const int wm = (wave >> 1) & 3, wn = wave & 1;
  const int lrow = lane & 15, lk = lane >> 4;
  const int frag_lo = lrow * 128 + ((lk ^ ((lrow >> 1) & 7)) << 4);
  const int frag_hi = lrow * 128 + (((lk + 4) ^ ((lrow >> 1) & 7)) << 4);
  const int wave_rows = rows_valid - wm * 64;

  f32x4 acc[4][8];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The K loop for a wave whose first NMI 16-row subtiles hold valid rows.
  // NEXT1 / NEXT2: stages kb + 1 / kb + 2 exist (compile-time, so the loop
  // body has no branch for the compiler to sink the FMAs behind).
  auto kloop = [&](auto nmi_c) {
    constexpr int NMI = decltype(nmi_c)::value;
    auto kblock = [&](int kb, auto next1_c, auto next2_c) {
      constexpr bool next1 = decltype(next1_c)::value, next2 = decltype(next2_c)::value;
      // stage kb has landed; the early part of kb + 1 (7 copies) may be in flight
      if constexpr (next1) wait_and_barrier<7>();
      else wait_and_barrier<0>();
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* st = smem + (kb & 1) * kStage256;
      // row wm 64 + mi 16 + 4 lk + v lives in window slot wm 64 + mi 16 + 4 v + lk
      const float* sA = reinterpret_cast<const float*>(smem + kSWinOff256 + ((kb / kSWin) & 1) * kSWin256) +
                        (wm * 64 + lk) * kSWin + (kb % kSWin);
      const float sb = s_bd[wn][kb];
      const uint8_t* a_lo = st + wm * 64 * 128 + frag_lo;
      const uint8_t* a_hi = st + wm * 64 * 128 + frag_hi;
      const uint8_t* b_lo = st + kA256 + wn * 128 * 128 + frag_lo;
      const uint8_t* b_hi = st + kA256 + wn * 128 * 128 + frag_hi;
      auto read_b = [&](int ni) {
        const i32x4 y0 = *reinterpret_cast<const i32x4*>(b_lo + ni * 16 * 128);
        const i32x4 y1 = *reinterpret_cast<const i32x4*>(b_hi + ni * 16 * 128);
        return __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      auto read_a = [&](int mi) {
        const i32x4 x0 = *reinterpret_cast<const i32x4*>(a_lo + mi * 16 * 128);
        const i32x4 x1 = *reinterpret_cast<const i32x4*>(a_hi + mi * 16 * 128);
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      // the copies issued with column subtile ni: the late part of kb + 1 with
      // subtiles 0-1 (its rows' slot is free since this block's barrier), the
      // early part of kb + 2 with subtiles 4-7 (after the mid-block barrier)
      auto copies_at = [&](int ni) {
        if (ni < 2) {
          if (next1) cp(kb + 1, 7 + ni);
        } else if (ni >= 4 && next2) {
          if (ni == 4) { cp(kb + 2, 0); cp(kb + 2, 1); }
          else if (ni == 5) { cp(kb + 2, 2); cp(kb + 2, 3); }
          else if (ni == 6) { cp(kb + 2, 4); cp(kb + 2, 5); }
          else cp(kb + 2, 6);
        }
      };
      auto mid_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      };
      if constexpr (NMI == 0) {
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) {
          if (ni == 4) mid_barrier();
          copies_at(ni);
        }
        return;
      }
      f32x4 sc[4];
      i32x8 af[4], bfr[2];
      af[0] = read_a(0);
      bfr[0] = read_b(0);
#pragma unroll
      for (int mi = 1; mi < NMI; ++mi) af[mi] = read_a(mi);
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[mi][v] = sA[(mi * 16 + 4 * v) * kSWin];
#pragma unroll
      for (int mi = 0; mi < NMI; ++mi) sc[mi] = sc[mi] * sb;
      f32x4 part[2][4];
#pragma unroll
      for (int ni = 0; ni < 9; ++ni) {
        // every wave's reads of A and of B rows 0-63 of both blocks are done
        if (ni == 4) mid_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (ni < 7) bfr[(ni + 1) & 1] = read_b(ni + 1);
        if (ni < 8) copies_at(ni);
#pragma unroll
        for (int mi = 0; mi < NMI; ++mi) {
          if (ni < 8)
            part[ni & 1][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                af[mi], bfr[ni & 1], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
          if (ni > 0) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[mi][ni - 1][v] = __builtin_fmaf(part[(ni - 1) & 1][mi][v], sc[mi][v], acc[mi][ni - 1][v]);
          }
        }
        // issue order: the next B fragment's reads, the copies, then each
        // MFMA followed by the previous subtile's 4 FMAs of the same rows
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // vector memory reads
#pragma unroll
        for (int mi = 0; mi < NMI; ++mi) {
          if (ni < 8) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          if (ni > 0) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
        }
      }
    };
    // stage 0 whole, then the early part of stage 1
#pragma unroll
    for (int i = 0; i < 9; ++i) cp(0, i);
    if (nkb > 1) {
#pragma unroll
      for (int i = 0; i < 7; ++i) cp(1, i);
    }
    constexpr std::true_type yes{};
    constexpr std::false_type no{};
    int kb = 0;
    for (; kb + 2 < nkb; ++kb) kblock(kb, yes, yes);
    if (kb + 1 < nkb) kblock(kb++, yes, no);
    kblock(kb, no, no);
  };
  switch (__builtin_amdgcn_readfirstlane(clampi((wave_rows + 15) >> 4, 0, 4))) {
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }
  __syncthreads();   // every wave is done with the stages and windows (no copy is in flight)

  if constexpr (EPI == MOE_EPI_BF16) {
    // ---- bf16 epilogue: staged through LDS ([256][264] bf16 over both stage
    // slots and the windows; the 8 pad columns put the rows that four lane
    // groups write together, 4 rows apart, on different banks), then 16
    // coalesced 16-byte buffer stores per thread; a row past the tile's valid
    // rows points past the buffer's end, where the store is dropped.  Lane value (mi, ni, v) sits at tile row wm*64 + mi*16 + 4*lk + v
    // and column wn*128 + ni*16 + lrow.
    uint16_t* otile = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 64 + mi * 16 + 4 * lk + v;
        float rs = 1.0f;
        if (p.row_scale) rs = p.row_scale[row0 + min(m0 + row, rows_g - 1)];
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) {
          const float val = p.row_scale ? acc[mi][ni][v] * rs : acc[mi][ni][v];
          otile[row * 264 + wn * 128 + ni * 16 + lrow] = (uint16_t)f32_to_bf16(val);
        }
      }
    __syncthreads();
    // 256 rows of ldo <= 2^21 bf16: the resource and every offset stay below 2^31
    const __amdgpu_buffer_rsrc_t rs_o =
        make_rsrc(static_cast<uint16_t*>(p.out) + (long long)(row0 + m0) * p.ldo, rows_valid * (int)p.ldo * 2);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int q = tid + kThreads * j;
      const int row = q >> 5, c = q & 31;
      const int off = row < rows_valid ? (row * (int)p.ldo + n_tile * BN + c * 8) * 2 : 0x7FFFFFF0;
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const i32x4*>(otile + row * 264 + c * 8), rs_o,
                                             off, 0, 0);
    }
  } else {
  // ---- SwiGLU epilogue.  Lane value (mi, ni, v) sits at tile row
  // wm*64 + mi*16 + 4*lk + v and column ni*16 + lrow of weight block wn.  The
  // gate wave keeps columns 0-63 and hands 64-127 to its up partner (wave ^ 1),
  // which hands back its columns 0-63; each forms h for 64 columns.
  f32x4* ex = reinterpret_cast<f32x4*>(smem);                          // [8 waves][16][64]
  float* red = reinterpret_cast<float*>(smem + kSWinOff256);             // [2][256] row maxima
  float* s_m = reinterpret_cast<float*>(smem + kSWinOff256 + 2048);      // [256] multipliers
  uint8_t* otile = smem;                                                 // [256][128] codes, after ex
  const int partner = wave ^ 1;
  // The gate / up role is fixed per wave, so each phase is compiled for both
  // roles and a wave-uniform branch picks one (a role chosen per element
  // costs a select and register moves for each of the 128 values); the
  // barriers stay outside the branches.
  auto hand_over = [&](auto gate_c) {
    constexpr bool GATE = decltype(gate_c)::value;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int j = 0; j < 4; ++j) ex[(wave * 16 + mi * 4 + j) * 64 + lane] = GATE ? acc[mi][4 + j] : acc[mi][j];
  };
  if (wn == 0) hand_over(std::true_type{});
  else hand_over(std::false_type{});
  __syncthreads();
  // Subtiles past the group's end had no MFMAs, so both partners' values
  // there are +0 and h is +0: every row is formed without a branch, the row
  // maxima of stored rows are unchanged, and those rows are never stored.
  float h[4][4][4];
  auto form_h = [&](auto gate_c) {
    constexpr bool GATE = decltype(gate_c)::value;
    uint32_t mxb[16];   // per (mi, v): bits of max |h| over this lane's four columns
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      f32x4 oth[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) oth[j] = ex[(partner * 16 + mi * 4 + j) * 64 + lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float mine = GATE ? acc[mi][j][v] : acc[mi][4 + j][v];
          const float other = oth[j][v];
          const float gt = GATE ? mine : other;
          const float u = GATE ? other : mine;
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
          h[mi][j][v] = gt * sg * u;
          mx = fmaxf(mx, fabsf(h[mi][j][v]));
        }
        mxb[mi * 4 + v] = __float_as_uint(mx);
      }
    }
    // lane (lk, lrow) ends with the maximum of row (mi, v) = (lrow / 4, lrow % 4)
    const uint32_t mx = row_max16_halving(mxb, lrow);
    red[wn * 256 + wm * 64 + (lrow >> 2) * 16 + 4 * lk + (lrow & 3)] = __uint_as_float(mx);
  };
  if (wn == 0) form_h(std::true_type{});
  else form_h(std::false_type{});
  __syncthreads();
  // one thread per row forms the tile's scale (two divisions) and stores d
  const int ld_d = p.n_out / BN;
  if (tid < BM256) {
    float m, d;
    tile_scale(fmaxf(red[tid], red[256 + tid]), m, d);
    s_m[tid] = m;
    if (tid < rows_valid) p.out_d[(long long)(row0 + m0 + tid) * ld_d + n_tile] = d;
  }
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = wm * 64 + mi * 16 + 4 * lk + v;
      const float m = s_m[row];
#pragma unroll
      for (int j = 0; j < 4; ++j) otile[row * 128 + wn * 64 + j * 16 + lrow] = (uint8_t)quant_code(h[mi][j][v], m);
    }
  }
  __syncthreads();
  uint8_t* out = static_cast<uint8_t*>(p.out);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = tid + kThreads * j;
    const int row = q >> 3, c = q & 7;
    if (row < rows_valid)
      *reinterpret_cast<i32x4*>(out + (long long)(row0 + m0 + row) * p.ldo + n_tile * 128 + c * 16) =
          *reinterpret_cast<const i32x4*>(otile + row * 128 + c * 16);
  }
  }
}

template <int EPI>
moe_status_t launch256(const GemmParams& p, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  if (moe_status_t st = allow_dynamic_lds(reinterpret_cast<const void*>(&grouped_gemm256_kernel<EPI>),
                                          kLds256, lds_set))
    return st;
  const long long n_tiles = p.n_out / BN;
  const long long row_tiles = (long long)(p.total_rows + BM256 - 1) / BM256 + p.G;   // an upper bound
  long long grid = row_tiles * n_tiles;
  grid = (grid + 7) / 8 * 8;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(grouped_gemm256_kernel<EPI>, dim3((unsigned)grid), dim3(kThreads), kLds256, stream, p);
  return launch_status();
}

template <int EPI, bool PING_PONG>
moe_status_t launch_schedule(const GemmParams& q, long long grid, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  if (moe_status_t st = allow_dynamic_lds(
          reinterpret_cast<const void*>(&grouped_gemm_kernel<EPI, PING_PONG>), lds_bytes(PING_PONG), lds_set))
    return st;
  hipLaunchKernelGGL((grouped_gemm_kernel<EPI, PING_PONG>), dim3((unsigned)grid), dim3(kThreads),
                     lds_bytes(PING_PONG), stream, q);
  return launch_status();
}

// The schedule by measurement: the ping-pong K loop for the SwiGLU epilogue
// and for contractions longer than 16 K blocks; the single-group loop for the
// short ones (K <= 2048, where the per-tile work weighs most), with two column
// tiles per workgroup as long as the grid still holds at least 32 workgroups
// per compute unit (so the last, partly filled round stays a small share).
template <int EPI>
moe_status_t launch(const GemmParams& p, int tile_rows, hipStream_t stream) {
  const bool ping_pong = EPI == MOE_EPI_SWIGLU_FP8 || p.k_dim / BK > 16;
  const long long n_tiles = (p.n_out + BN - 1) / BN;
  const long long row_tiles = (long long)(p.total_rows + BM - 1) / BM + p.G;   // an upper bound
  const long long cus = cu_count();
  if (cus <= 0) return MOE_ERR_HIP;
  GemmParams q = p;
  q.cols_per_wg = (!ping_pong && row_tiles * ((n_tiles + 1) / 2) >= 32 * cus) ? 2 : 1;
  const long long n_cols = (n_tiles + q.cols_per_wg - 1) / q.cols_per_wg;
  long long grid = row_tiles * n_cols;
  grid = (grid + 7) / 8 * 8;
  if (grid > 0x7FFFFFFFLL) return MOE_ERR_SHAPE;
  // 256-row tiles (SwiGLU and bf16 epilogues) unless the groups are small
  // (fewer than 128 rows on average, as in decoding), where a 256-row tile
  // would be mostly padding; the bf16 one also needs whole 256-column tiles
  // and ldo <= 2^21 (its store offsets over 256 rows are 32-bit)
  if constexpr (EPI != MOE_EPI_F32) {
    const bool fits = EPI == MOE_EPI_SWIGLU_FP8 || (p.n_out % BN == 0 && p.ldo <= (1 << 21));
    if (tile_rows == 256 || (tile_rows == 0 && fits && (long long)p.total_rows >= 128LL * p.G))
      return launch256<EPI>(p, stream);
  }
  if constexpr (EPI == MOE_EPI_SWIGLU_FP8) {
    return launch_schedule<EPI, true>(q, grid, stream);
  } else {
    return ping_pong ? launch_schedule<EPI, true>(q, grid, stream)
                     : launch_schedule<EPI, false>(q, grid, stream);
  }
}

moe_status_t grouped_gemm(const moe_gemm_fp8_args* a, int tile_rows, hipStream_t stream) {
  if (!a) return MOE_ERR_NULL;
  if (tile_rows != 0 && tile_rows != 128 && tile_rows != 256) return MOE_ERR_UNSUPPORTED;
  if (tile_rows == 256 && a->epilogue == MOE_EPI_F32) return MOE_ERR_UNSUPPORTED;
  if (tile_rows == 256 && a->epilogue == MOE_EPI_BF16 && (a->n_out % BN != 0 || a->ldo > (1 << 21)))
    return MOE_ERR_UNSUPPORTED;
  if (a->num_groups < 1 || a->num_groups > kMaxGroups || a->total_rows < 0 || a->n_out <= 0 ||
      a->k_dim <= 0 || a->k_dim % BK != 0 || a->n_out % 128 != 0 || a->lda < a->k_dim ||
      a->lda % 16 != 0 || a->a_rows < 0)
    return MOE_ERR_SHAPE;
  if (a->epilogue != MOE_EPI_BF16 && a->epilogue != MOE_EPI_SWIGLU_FP8 && a->epilogue != MOE_EPI_F32)
    return MOE_ERR_UNSUPPORTED;
  if (a->epilogue == MOE_EPI_SWIGLU_FP8 && a->n_out % BN != 0) return MOE_ERR_SHAPE;
  if (a->k_dim / BK > kMaxKb) return MOE_ERR_UNSUPPORTED;
  // in-kernel offsets are 32-bit: A must span less than 2 GiB
  if ((long long)a->a_rows * a->lda >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  // the bf16 epilogue stores through a buffer resource over the tile's rows
  // with 32-bit byte offsets: 128 rows of ldo bf16 must stay below 2^31 bytes
  if (a->epilogue == MOE_EPI_BF16 && a->ldo > (1 << 22)) return MOE_ERR_UNSUPPORTED;
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
    case MOE_EPI_SWIGLU_FP8: return launch<MOE_EPI_SWIGLU_FP8>(p, tile_rows, stream);
    case MOE_EPI_BF16: return launch<MOE_EPI_BF16>(p, tile_rows, stream);
    default: return launch<MOE_EPI_F32>(p, tile_rows, stream);
  }
}

}  // namespace

extern "C" moe_status_t moe_grouped_gemm_fp8(const moe_gemm_fp8_args* a, hipStream_t stream) {
  return grouped_gemm(a, 0, stream);
}

extern "C" moe_status_t moe_grouped_gemm_fp8_tiles(const moe_gemm_fp8_args* a, int tile_rows,
                                                   hipStream_t stream) {
  return grouped_gemm(a, tile_rows, stream);
}

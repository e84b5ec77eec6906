// Sigmoid router with auxiliary-loss-free biased top-k ("DeepSeek-V3:
// Auxiliary-Loss-Free MoE Load Balancing, Multi-Token Prediction, and FP8
// Training at 671B Scale", section III: affinity s = Sigmoid(u . e_i), chosen
// set = TopK of s + b, gate = s normalised over the chosen set, the bias never
// touching the gate; "DeepSeek-V3, explained.", recipe step 4).  The router
// stays in bf16 with float accumulation by default, as the pages keep the
// gating network out of FP8 (same page, section V, FP8 detail 4);
// moe_route_topk_fp8 is an opt-in variant on block-scaled FP8 operands.
//
// moe_route_topk in two launches.  The router GEMM x [T,H] . Wr^T [H,N] is
// split along H into S slices so that about one workgroup per compute unit
// exists; a workgroup computes the partial logits of 128 tokens x all N
// experts over its slice with bf16 MFMA (16x16x32) from LDS tiles filled by
// direct-to-LDS copies three stages deep, and writes them to the workspace.
// The second launch takes one wave per token: it sums the S partial logits in
// slice order (so the result does not depend on timing), applies the
// sigmoid, and selects the top k by k rounds of a wave-wide maximum of the
// keys as order-preserving integers, a ballot giving ties to the lower index.
#include <type_traits>

#include "common.h"

namespace {

using namespace moe;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kMaxN = 256;
constexpr int kRT = 128;                        // tokens per workgroup
constexpr int kRStage = (kRT + kMaxN) * 128;    // 48 KiB: x rows, then Wr rows
constexpr int kRStages = 3;
constexpr int kRLds = kRStages * kRStage;       // 144 KiB
constexpr int kRThreads = 512;                  // 8 waves: 2 token bands x 4 expert bands

__device__ __forceinline__ uint32_t sortable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One step of a 64-bit maximum across lanes: (hi, lo) takes the DPP-moved
// neighbour's pair when that pair is larger.
template <int CTRL>
__device__ __forceinline__ void dpp_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t oh = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, 0xF, 0xF, false);
  const uint32_t ol = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, 0xF, 0xF, false);
  const bool take = oh > hi || (oh == hi && ol > lo);
  hi = take ? oh : hi;
  lo = take ? ol : lo;
}

// Wave-wide maximum of a 64-bit value (uniform result): within each row of 16
// lanes by DPP (swap neighbours, swap pairs, mirror the halves, mirror the
// row), then the four row maxima read out to scalar registers and compared.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  dpp_max_step<0xB1>(hi, lo);
  dpp_max_step<0x4E>(hi, lo);
  dpp_max_step<0x141>(hi, lo);
  dpp_max_step<0x140>(hi, lo);
  unsigned long long best = 0ull;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const unsigned long long c =
        ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
        (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
    best = c > best ? c : best;
  }
  return best;
}

// Wave-wide maximum of a 32-bit unsigned value (uniform result): the row
// maxima by the same four DPP steps, then row 0's maximum broadcast into row
// 1 and row 2's into row 3, then row 1's into rows 2 and 3, so that lane 63
// holds the maximum of the wave.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t o;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v = o > v ? o : v;
  o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  v = o > v ? o : v;
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// k rounds of wave-wide argmax over keys held PER slots per lane, expert
// e = lane * PER + slot (each lane holds PER consecutive experts).  On return
// lane j < k holds the j-th chosen expert in sel_idx and its unbiased score in
// sel_s; `sum` (wave-uniform) is the float sum of the chosen scores in
// selection order.
//
// Each slot holds its key as an order-preserving 32-bit integer (at least 1;
// 0 marks a slot that is taken, excluded or beyond N).  A round takes the
// wave maximum m; the lowest lane whose own maximum equals m (a ballot) holds
// the lowest expert index with key m, at its lowest slot equal to m, so ties
// go to the lower index as in a (key, -index) argmax.  Equal integers are
// equal keys, except that the two most negative NaN patterns share the value
// 1.  The rounds run on the vector unit but for the ballot and two reads of
// one lane.
template <int PER>
__device__ __forceinline__ void wave_topk(const float (&key)[PER], const float (&score)[PER],
                                          int N, int k, int lane, int& sel_idx, float& sel_s,
                                          float& sum, uint32_t excluded = 0u) {
  uint32_t cand[PER];
#pragma unroll
  for (int s = 0; s < PER; ++s) {
    const uint32_t u = sortable(key[s]);
    cand[s] = (lane * PER + s < N && !((excluded >> s) & 1u)) ? (u > 1u ? u : 1u) : 0u;
  }
  sel_idx = -1;
  for (int r = 0; r < k; ++r) {
    uint32_t best = cand[0];
#pragma unroll
    for (int s = 1; s < PER; ++s) best = cand[s] > best ? cand[s] : best;
    const uint32_t m = wave_max_u32(best);
    // k never exceeds the eligible experts, so some lane's maximum equals m
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(best == m);
    const int owner = (int)__builtin_ctzll(hit | (1ull << 63));
    int first = PER - 1;
#pragma unroll
    for (int s = PER - 2; s >= 0; --s) first = cand[s] == m ? s : first;
    const int e = owner * PER + __builtin_amdgcn_readlane(first, owner);
#pragma unroll
    for (int s = 0; s < PER; ++s) cand[s] = lane * PER + s == e ? 0u : cand[s];
    if (lane == r) sel_idx = e;
  }
  // lane j < k fetches its expert's score from the lane that holds it
  const int src = sel_idx < 0 ? lane : sel_idx / PER;
  const int slot = sel_idx < 0 ? 0 : sel_idx % PER;
  float got = 0.0f;
#pragma unroll
  for (int s = 0; s < PER; ++s) {
    const float v = __shfl(score[s], src, 64);
    got = slot == s ? v : got;
  }
  sel_s = sel_idx < 0 ? 0.0f : got;
  sum = 0.0f;
  for (int r = 0; r < k; ++r)
    sum = sum + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sel_s), r));
}

__device__ __forceinline__ float unsortable(uint32_t v) {
  return __uint_as_float((v & 0x80000000u) ? (v & 0x7FFFFFFFu) : ~v);
}

// Group-limited routing ("DeepSeek-V3, explained.", recipe step 5; "DeepSeek-V3
// Technical Report" (deepforge), "Balancing without a balance loss"): the N
// experts form G groups of N / G consecutive indices; a group's score is the
// float sum of its r largest keys, added in descending order; only the M best
// groups (score descending, group index ascending) are eligible.  Returns the
// slots of this lane (expert lane * PER + p) that are NOT eligible, as a bit
// mask.  Requires G <= 64.
template <int PER>
__device__ __forceinline__ uint32_t group_excluded(const float (&key)[PER], int N, int G, int M,
                                                   int r, int lane) {
  const int gs = N / G;
  float my_score = 0.0f;                    // lane g < G: score of group g
  for (int g = 0; g < G; ++g) {
    uint32_t taken = 0;
    float acc = 0.0f;
    for (int j = 0; j < r; ++j) {
      unsigned long long best = 0ull;
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int e = lane * PER + p;
        if (e < N && e / gs == g && !((taken >> p) & 1u)) {
          const unsigned long long c =
              ((unsigned long long)sortable(key[p]) << 32) | (0xFFFFFFFFu - (uint32_t)e);
          best = c > best ? c : best;
        }
      }
      best = wave_max_u64(best);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
      if (lane == e / PER) taken |= 1u << (e % PER);
      const float kv = unsortable((uint32_t)(best >> 32));
      acc = j == 0 ? kv : acc + kv;
    }
    if (lane == g) my_score = acc;
  }
  int rank = 0;
  for (int g = 0; g < G; ++g) {
    const float sg = __shfl(my_score, g, 64);
    if (sg > my_score || (sg == my_score && g < lane)) ++rank;
  }
  const int chosen = (lane < G && rank < M) ? 1 : 0;
  uint32_t excluded = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int e = lane * PER + p;
    const int g = e < N ? e / gs : 0;
    const int ok = __shfl(chosen, g, 64);
    if (e >= N || !ok) excluded |= 1u << p;
  }
  return excluded;
}

__device__ __forceinline__ float sigmoidf_acc(float z) { return 1.0f / (1.0f + expf(-z)); }

// Number of H slices for T tokens: enough workgroups for about one per
// compute unit, at most one slice per 128-wide block of H (a slice holds
// whole 1x128 tiles of x, which the quantising variant needs), and at most
// 16 (the partial logits, S * T * N floats written and read back, must stay
// small next to x when T is small).
int route_splits(int T, int H) {
  const int nb = H / 128;
  const int tiles = (T + kRT - 1) / kRT;
  int S = (256 + tiles - 1) / tiles;
  if (S > 16) S = 16;
  if (S > nb) S = nb;
  return S < 1 ? 1 : S;
}

__device__ __forceinline__ int clampi_dev(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Wait until at most N of this wave's direct-to-LDS copies are outstanding
// and its LDS reads are done, then meet the other waves (the compiler does
// not track the LDS side of these copies).
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Partial router logits: ws[s][t][e] = sum over the H slice s of
// x[t,h] * Wr[e,h] (bf16 products, float accumulation in the MFMA).
// Workgroup layout: the (slice, token tile) list is slice-major and each XCD
// takes a contiguous run of it, so one XCD mostly reads one slice of Wr.
// LDS rows are 128 B; 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7).
// A slice holds whole 128-wide blocks of H (two K chunks each).
//
// With QX the kernel also writes the 1x128 FP8 codes and scales of the x
// tiles it holds (the activation quantisation of the expert GEMM, section V
// of the same page, FP8 detail 1 and Figure 6), so x is read once for both:
// the four threads of a token row each take 16 values of both K chunks of a
// block (the first chunk's kept in registers until the second lands), the
// block maximum is a 4-lane reduction, and the codes leave in two 16-byte
// buffer stores per thread, the scales of four blocks of a row in one
// 16-byte write by its four threads; rows past T point past the buffers'
// ends, where the stores are dropped.  The stores go out before the next
// stage's copies, so the copy waits cover them.  The codes and scales are
// those of fp8_quant_1x128 (the same scale rule and encoder).
template <bool QX>
__global__ __launch_bounds__(kRThreads, 1) void route_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int N, int S,
    float* __restrict__ ws, uint8_t* __restrict__ xq, float* __restrict__ xd) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles = (T + kRT - 1) / kRT;
  const int total = tiles * S;
  const int per_xcd = (total + 7) / 8;
  const int slot = blockIdx.x >> 3, xcd = blockIdx.x & 7;
  const int L = xcd * per_xcd + slot;
  if (slot >= per_xcd || L >= total) return;
  const int s = L / tiles, tile = L - s * tiles;
  const int t0 = tile * kRT;
  const int nb = H / 128;
  const int c0 = 2 * (int)((long long)s * nb / S), c1 = 2 * (int)((long long)(s + 1) * nb / S);
  const int nck = c1 - c0;

  // copies: load j of wave w fills the 1 KiB block 8 j + w of the stage
  // (rows 64 j + 8 w + (lane >> 3)); x has 2 loads per wave, Wr 4.
  const int chunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow8 = 8 * wave + (lane >> 3);
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(x, (int)((long long)T * H * 2));
  const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(wr, N * H * 2);
  int x_off[2], w_off[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = min(t0 + 64 * j + lrow8, T - 1);
    x_off[j] = t * H * 2 + chunk * 16;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = min(64 * j + lrow8, N - 1);
    w_off[j] = e * H * 2 + chunk * 16;
  }
  auto issue = [&](int i, uint8_t* st) {
    const int ko = (c0 + i) * 128;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_x, (lds_ptr_t)(st + (8 * j + wave) * 1024), 16,
                                               x_off[j], ko, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_w, (lds_ptr_t)(st + kRT * 128 + (8 * j + wave) * 1024), 16, w_off[j], ko, 0, 0);
  };

  // wave tile: tokens wm*64..+64, experts wn*64..+64 (NI valid 16-expert
  // subtiles); lane l reads row l & 15 of a subtile, K chunk 4 ks + (l >> 4)
  const int wm = wave & 1, wn = wave >> 1;
  const int lrow = lane & 15, lk = lane >> 4;
  const int ni_valid = clampi_dev((N - wn * 64) >> 4, 0, 4);
  const int sw = (lrow >> 1) & 7;
  const int frag0 = lrow * 128 + ((lk ^ sw) << 4);         // ks = 0
  const int frag1 = lrow * 128 + (((lk + 4) ^ sw) << 4);   // ks = 1
  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  // quantiser: thread (row qr, part qp) holds x values 16 qp .. 16 qp + 15 of
  // each K chunk of the row's current 128-wide block
  const int qr = tid >> 2, qp = tid & 3;
  const int qsw = (qr >> 1) & 7;
  const int qpos0 = qr * 128 + (((2 * qp) ^ qsw) << 4);
  const int qpos1 = qr * 128 + (((2 * qp + 1) ^ qsw) << 4);
  const bool q_live = t0 + qr < T;
  const int q_row = q_live ? (t0 + qr) * H : T * H;        // past the end: dropped
  const int d_row = q_live ? (t0 + qr) * nb * 4 : T * nb * 4;
  const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(xq, QX ? T * H : 0);
  const __amdgpu_buffer_rsrc_t rs_qd = make_rsrc(xd, QX ? T * nb * 4 : 0);
  float qu[16];                                             // first chunk's 16 values
#pragma unroll
  for (int e = 0; e < 16; ++e) qu[e] = 0.0f;
  float qmax = 0.0f;
  i32x4 q_lo = i32x4{0, 0, 0, 0}, q_hi = q_lo;              // a finished block, not yet stored
  // scales: thread qp of a row keeps the scale of the slice's blocks 4 m + qp,
  // and the row's four threads store four blocks' scales as 16 contiguous
  // bytes (one write, not four)
  float q_d = 1.0f;
  const int blk0 = c0 >> 1, nblk = nck >> 1;
  // the first K chunk of a block (P = 0): keep its values, start the maximum;
  // the second (P = 1): finish the maximum over the 4 threads of the row,
  // form the scale and encode both chunks
  auto quant_chunk = [&](auto p_c, const uint4& a, const uint4& b, int blk_done) {
    constexpr int P = decltype(p_c)::value;
    float v[16];
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
    v[8] = bf16_lo(b.x); v[9] = bf16_hi(b.x); v[10] = bf16_lo(b.y); v[11] = bf16_hi(b.y);
    v[12] = bf16_lo(b.z); v[13] = bf16_hi(b.z); v[14] = bf16_lo(b.w); v[15] = bf16_hi(b.w);
    float m = P ? qmax : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
    if constexpr (P == 0) {
#pragma unroll
      for (int e = 0; e < 16; ++e) qu[e] = v[e];
      qmax = m;
    } else {
      m = group_max<4>(m);
      float mul, dd;
      tile_scale(m, mul, dd);
      const float (&u)[16] = qu;
      i32x4 c_lo, c_hi;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        c_lo[w4] = (int)e4m3_pack4(u[4 * w4] * mul, u[4 * w4 + 1] * mul, u[4 * w4 + 2] * mul,
                                   u[4 * w4 + 3] * mul);
        c_hi[w4] = (int)e4m3_pack4(v[4 * w4] * mul, v[4 * w4 + 1] * mul, v[4 * w4 + 2] * mul,
                                   v[4 * w4 + 3] * mul);
      }
      const bool zero = mul == 0.0f;        // the zero-tile rule: all codes +0
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        q_lo[w4] = zero ? 0 : c_lo[w4];
        q_hi[w4] = zero ? 0 : c_hi[w4];
      }
      q_d = (blk_done & 3) == qp ? dd : q_d;
    }
  };
  // the codes of the block completed in K chunk i, and after every fourth
  // block of the slice (and its last) the scales of up to four blocks
  auto quant_store = [&](int i) {
    const int blk = (c0 + i) >> 1, lb = blk - blk0;
    __builtin_amdgcn_raw_buffer_store_b128(q_lo, rs_q, q_row + blk * 128 + 16 * qp, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(q_hi, rs_q, q_row + blk * 128 + 64 + 16 * qp, 0, 0);
    if ((lb & 3) == 3 || lb == nblk - 1) {
      const int first = lb & ~3;                 // slice-local block of this thread: first + qp
      __builtin_amdgcn_raw_buffer_store_b32(
          __float_as_int(q_d), rs_qd,
          first + qp <= lb ? d_row + (blk0 + first + qp) * 4 : T * nb * 4, 0, 0);
    }
  };

  auto kloop = [&](auto ni_c) {
    constexpr int NI = decltype(ni_c)::value;
    issue(0, smem);
    if (nck > 1) issue(1, smem + kRStage);
    // one K chunk; P is its position in its 128-wide block (nck is even, so
    // chunk i has P = i & 1)
    auto chunk = [&](int i, auto p_c) {
      constexpr int P = decltype(p_c)::value;
      // The quantiser's stores of the block finished in chunk i - 1 go out
      // before the copies of chunk i + 2, so the next wait, which allows 6
      // operations (those copies) to be outstanding, also covers them,
      // whatever order loads and stores complete in.
      if (i + 1 < nck) wait_and_barrier<6>(); else wait_and_barrier<0>();
      if (QX && P == 0 && i > 0) quant_store(i - 1);
      if (i + 2 < nck) issue(i + 2, smem + ((i + 2) % kRStages) * kRStage);
      const uint8_t* st = smem + (i % kRStages) * kRStage;
      uint4 qa = make_uint4(0u, 0u, 0u, 0u), qb = qa;
      if (QX) {
        qa = *reinterpret_cast<const uint4*>(st + qpos0);
        qb = *reinterpret_cast<const uint4*>(st + qpos1);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (NI == 0) break;
        const int fo = ks ? frag1 : frag0;
        bf16x8 af[4], bfr[NI > 0 ? NI : 1];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
          af[mi] = *reinterpret_cast<const bf16x8*>(st + (wm * 64 + mi * 16) * 128 + fo);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          bfr[ni] = *reinterpret_cast<const bf16x8*>(st + (kRT + wn * 64 + ni * 16) * 128 + fo);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
            acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
      }
      if (QX) {
        quant_chunk(p_c, qa, qb, ((c0 + i) >> 1) - blk0);
        // the quantiser's vector work between the MFMAs, so that it runs
        // while they do
        if (NI > 0) {
#pragma unroll
          for (int m = 0; m < 8 * NI; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, P ? 5 : 2, 0);
          }
        }
      }
    };
    for (int i = 0; i < nck; i += 2) {
      chunk(i, std::integral_constant<int, 0>{});
      chunk(i + 1, std::integral_constant<int, 1>{});
    }
    if (QX) quant_store(nck - 1);
    if (NI == 0) return;
    // lane value (mi, ni, v): token wm*64 + mi*16 + 4*lk + v, expert
    // wn*64 + ni*16 + lrow
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + wm * 64 + mi * 16 + 4 * lk + v;
        if (t < T) {
          float* row = ws + ((long long)s * T + t) * N + wn * 64 + lrow;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) row[ni * 16] = acc[mi][ni][v];
        }
      }
  };
  switch (__builtin_amdgcn_readfirstlane(ni_valid)) {
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }
}

// The same partial logits from FP8 operands, for the opt-in FP8 router: x
// quantised with one scale per 1x128 tile, Wr with one per 128x128 block.
// One K chunk is one 128-wide scale block: one 16x16x128 FP8 MFMA per
// subtile into a zero accumulator, folded into the float sum with one FMA by
// d_x[t, c] * d_W[e / 128, c] (the block-scaled product of section V of the
// same page, FP8 details 1-2, applied to the gating GEMM, which that section
// otherwise keeps in higher precision: detail 4).
typedef int i32x8_r __attribute__((ext_vector_type(8)));
constexpr int kRStageF = (kRT + kMaxN) * 128 + kRT * 4;   // + the chunk's 128 x scales
constexpr int kRLdsF = kRStages * kRStageF;

__global__ __launch_bounds__(kRThreads, 1) void route_partial_fp8_kernel(
    const uint8_t* __restrict__ xq, const float* __restrict__ xd, const uint8_t* __restrict__ wq,
    const float* __restrict__ wd, int T, int H, int N, int S, float* __restrict__ ws) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tiles = (T + kRT - 1) / kRT;
  const int total = tiles * S;
  const int per_xcd = (total + 7) / 8;
  const int slot = blockIdx.x >> 3, xcd = blockIdx.x & 7;
  const int L = xcd * per_xcd + slot;
  if (slot >= per_xcd || L >= total) return;
  const int s = L / tiles, tile = L - s * tiles;
  const int t0 = tile * kRT;
  const int nc = H / 128;
  const int c0 = (int)((long long)s * nc / S), c1 = (int)((long long)(s + 1) * nc / S);
  const int nck = c1 - c0;

  // row copies as in the bf16 kernel (one row = 128 codes = 128 B); waves 0
  // and 1 also copy the chunk's x scales, 64 tokens each
  const int chunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int lrow8 = 8 * wave + (lane >> 3);
  const __amdgpu_buffer_rsrc_t rs_x = make_rsrc(xq, (int)((long long)T * H));
  const __amdgpu_buffer_rsrc_t rs_w = make_rsrc(wq, N * H);
  const __amdgpu_buffer_rsrc_t rs_d = make_rsrc(xd, T * nc * 4);
  int x_off[2], w_off[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = min(t0 + 64 * j + lrow8, T - 1);
    x_off[j] = t * H + chunk * 16;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = min(64 * j + lrow8, N - 1);
    w_off[j] = e * H + chunk * 16;
  }
  const int d_off = min(t0 + 64 * (wave & 1) + lane, T - 1) * nc * 4;
  auto issue = [&](int i, uint8_t* st) {
    const int ko = (c0 + i) * 128;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_x, (lds_ptr_t)(st + (8 * j + wave) * 1024), 16,
                                               x_off[j], ko, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_w, (lds_ptr_t)(st + kRT * 128 + (8 * j + wave) * 1024), 16, w_off[j], ko, 0, 0);
    if (wave < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs_d, (lds_ptr_t)(st + (kRT + kMaxN) * 128 + wave * 256), 4, d_off, (c0 + i) * 4, 0, 0);
  };

  // wave tile and fragments as in the bf16 kernel; a lane's 32 codes of a
  // row are 16-byte chunks lk and lk + 4 (the same K order for x and Wr)
  const int wm = wave & 1, wn = wave >> 1;
  const int lrow = lane & 15, lk = lane >> 4;
  const int ni_valid = clampi_dev((N - wn * 64) >> 4, 0, 4);
  const int sw = (lrow >> 1) & 7;
  const int frag_lo = lrow * 128 + ((lk ^ sw) << 4);
  const int frag_hi = lrow * 128 + (((lk + 4) ^ sw) << 4);
  const float* wd_row = wd + (long long)((wn * 64) >> 7) * nc;   // the wave's 64 experts share a block
  f32x4 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto kloop = [&](auto ni_c) {
    constexpr int NI = decltype(ni_c)::value;
    issue(0, smem);
    if (nck > 1) issue(1, smem + kRStageF);
    for (int i = 0; i < nck; ++i) {
      if (i + 1 < nck) {
        if (wave < 2) wait_and_barrier<7>();
        else wait_and_barrier<6>();
      } else {
        wait_and_barrier<0>();
      }
      if (i + 2 < nck) issue(i + 2, smem + ((i + 2) % kRStages) * kRStageF);
      if (NI == 0) continue;
      const uint8_t* st = smem + (i % kRStages) * kRStageF;
      const float* sx = reinterpret_cast<const float*>(st + (kRT + kMaxN) * 128) + wm * 64 + 4 * lk;
      const float sw_blk = wd_row[c0 + i];
      i32x8_r af[4], bfr[NI > 0 ? NI : 1];
      f32x4 sc[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const uint8_t* a = st + (wm * 64 + mi * 16) * 128;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(a + frag_lo);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(a + frag_hi);
        af[mi] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        sc[mi] = *reinterpret_cast<const f32x4*>(sx + mi * 16) * sw_blk;
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const uint8_t* b = st + (kRT + wn * 64 + ni * 16) * 128;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(b + frag_lo);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(b + frag_hi);
        bfr[ni] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[mi], bfr[ni], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[mi][ni][v] = __builtin_fmaf(part[v], sc[mi][v], acc[mi][ni][v]);
        }
    }
    if (NI == 0) return;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + wm * 64 + mi * 16 + 4 * lk + v;
        if (t < T) {
          float* row = ws + ((long long)s * T + t) * N + wn * 64 + lrow;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) row[ni * 16] = acc[mi][ni][v];
        }
      }
  };
  switch (__builtin_amdgcn_readfirstlane(ni_valid)) {
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }
}

// One wave per token, each lane holding PER consecutive experts: logits = sum
// of the S partials in slice order, scores = sigmoid, then the biased top k
// and the unbiased gates.  A lane's PER partials, biases and scores are
// adjacent, so each is one wide access.
template <int PER>
__global__ __launch_bounds__(256) void route_finish_kernel(const float* __restrict__ ws, int S,
                                                           const float* __restrict__ bias, int T,
                                                           int N, int k, int G, int M,
                                                           float* __restrict__ scores,
                                                           int32_t* __restrict__ idx,
                                                           float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int e0 = lane * PER;
  float key[PER], scr[PER];
  // N is a multiple of 16, so a lane holds all PER of its experts or none
  if (e0 < N) {
    float z[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) z[p] = ws[(long long)t * N + e0 + p];
    for (int s = 1; s < S; ++s) {
#pragma unroll
      for (int p = 0; p < PER; ++p) z[p] += ws[((long long)s * T + t) * N + e0 + p];
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      scr[p] = sigmoidf_acc(z[p]);
      key[p] = scr[p] + bias[e0 + p];
    }
    if (scores) {
#pragma unroll
      for (int p = 0; p < PER; ++p) scores[(long long)t * N + e0 + p] = scr[p];
    }
  } else {
#pragma unroll
    for (int p = 0; p < PER; ++p) scr[p] = key[p] = 0.0f;
  }
  const uint32_t excluded = G > 1 ? group_excluded<PER>(key, N, G, M, k / M, lane) : 0u;
  int sel;
  float s_sel, sum;
  wave_topk<PER>(key, scr, N, k, lane, sel, s_sel, sum, excluded);
  if (lane < k) {
    idx[(long long)t * k + lane] = sel;
    gate[(long long)t * k + lane] = sum > 0.0f ? s_sel / sum : 1.0f / (float)k;
  }
}

// One wave per token over a given score tensor (N <= 64 * PER), each lane
// holding PER consecutive experts.
template <int PER>
__global__ __launch_bounds__(256) void topk_scores_kernel(const float* __restrict__ scores,
                                                          const float* __restrict__ bias, int T,
                                                          int N, int k, int G, int M,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float key[PER], scr[PER];
#pragma unroll
  for (int s = 0; s < PER; ++s) {
    const int e = lane * PER + s;
    scr[s] = e < N ? scores[(long long)t * N + e] : 0.0f;
    key[s] = e < N ? scr[s] + bias[e] : 0.0f;
  }
  const uint32_t excluded = G > 1 ? group_excluded<PER>(key, N, G, M, k / M, lane) : 0u;
  int sel;
  float s_sel, sum;
  wave_topk<PER>(key, scr, N, k, lane, sel, s_sel, sum, excluded);
  if (lane < k) {
    idx[(long long)t * k + lane] = sel;
    gate[(long long)t * k + lane] = sum > 0.0f ? s_sel / sum : 1.0f / (float)k;
  }
}

// group-limited routing arguments: G <= 1 disables it; otherwise G divides N,
// 1 <= M <= G, M divides k and each group holds at least k / M experts
bool groups_ok(int N, int k, int G, int M) {
  if (G <= 1) return true;
  if (G > 64 || N % G != 0 || M < 1 || M > G || k % M != 0) return false;
  return k / M <= N / G && k <= M * (N / G);
}

// The finish launch shared by both routers: PER = ceil(N / 64) slots per lane.
void launch_finish(const float* part, int S, const float* bias, int T, int N, int k, int G, int M,
                   float* scores, int32_t* idx, float* gate, hipStream_t stream) {
  const int blocks = (T + 3) / 4;
  const int per = (N + 63) / 64;
#define MOE_FINISH_LAUNCH(P)                                                                  \
  hipLaunchKernelGGL(route_finish_kernel<P>, dim3(blocks), dim3(256), 0, stream, part, S, bias, \
                     T, N, k, G, M, scores, idx, gate)
  if (per <= 1) MOE_FINISH_LAUNCH(1);
  else if (per <= 2) MOE_FINISH_LAUNCH(2);
  else MOE_FINISH_LAUNCH(4);
#undef MOE_FINISH_LAUNCH
}

}  // namespace

extern "C" size_t moe_route_workspace_bytes(int T, int H, int N) {
  if (T <= 0 || H <= 0 || H % 128 != 0 || N <= 0) return 0;
  return (size_t)route_splits(T, H) * (size_t)T * (size_t)N * sizeof(float);
}

namespace {

// moe_route_topk, and with qx also the 1x128 quantisation of x into x_q / x_d
// (moe_route_topk_quant_x).
moe_status_t route_topk_bf16(const void* x_bf16, const void* w_router_bf16, const float* bias,
                             int T, int H, int N, int k, int n_groups, int topk_groups,
                             float* scores, int32_t* topk_idx, float* topk_gate, bool qx,
                             uint8_t* x_q, float* x_d, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  if (T < 0 || H < 0 || H % 128 != 0 || N < 16 || N > kMaxN || N % 16 != 0 || k < 1 ||
      k > 32 || k > N || !groups_ok(N, k, n_groups, topk_groups))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (H == 0) return MOE_ERR_SHAPE;
  // in-kernel byte offsets are 32-bit
  if ((long long)T * H * 2 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (!x_bf16 || !w_router_bf16 || !bias || !topk_idx || !topk_gate) return MOE_ERR_NULL;
  if (qx && (!x_q || !x_d)) return MOE_ERR_NULL;
  if (!ws || ws_bytes < moe_route_workspace_bytes(T, H, N)) return MOE_ERR_WORKSPACE;
  if (!aligned16(x_bf16) || !aligned16(w_router_bf16) || !aligned16(ws)) return MOE_ERR_ALIGN;
  if (qx && (!aligned16(x_q) || (reinterpret_cast<uintptr_t>(x_d) & 3))) return MOE_ERR_ALIGN;
  if (moe_status_t st = check_device()) return st;
  const void* kern = qx ? reinterpret_cast<const void*>(&route_partial_kernel<true>)
                        : reinterpret_cast<const void*>(&route_partial_kernel<false>);
  static std::atomic<uint64_t> lds_set[2] = {0, 0};
  if (moe_status_t st = allow_dynamic_lds(kern, kRLds, lds_set[qx ? 1 : 0])) return st;
  const int S = route_splits(T, H);
  const int tiles = (T + kRT - 1) / kRT;
  const int grid = (tiles * S + 7) / 8 * 8;
  float* part = static_cast<float*>(ws);
  if (qx)
    hipLaunchKernelGGL(route_partial_kernel<true>, dim3(grid), dim3(kRThreads), kRLds, stream,
                       static_cast<const uint16_t*>(x_bf16),
                       static_cast<const uint16_t*>(w_router_bf16), T, H, N, S, part, x_q, x_d);
  else
    hipLaunchKernelGGL(route_partial_kernel<false>, dim3(grid), dim3(kRThreads), kRLds, stream,
                       static_cast<const uint16_t*>(x_bf16),
                       static_cast<const uint16_t*>(w_router_bf16), T, H, N, S, part,
                       (uint8_t*)nullptr, (float*)nullptr);
  if (moe_status_t st = launch_status()) return st;
  launch_finish(part, S, bias, T, N, k, n_groups, topk_groups, scores, topk_idx, topk_gate,
                stream);
  return launch_status();
}

}  // namespace

extern "C" moe_status_t moe_route_topk(const void* x_bf16, const void* w_router_bf16,
                                       const float* bias, int T, int H, int N, int k,
                                       int n_groups, int topk_groups, float* scores,
                                       int32_t* topk_idx, float* topk_gate, void* ws,
                                       size_t ws_bytes, hipStream_t stream) {
  return route_topk_bf16(x_bf16, w_router_bf16, bias, T, H, N, k, n_groups, topk_groups, scores,
                         topk_idx, topk_gate, false, nullptr, nullptr, ws, ws_bytes, stream);
}

extern "C" moe_status_t moe_route_topk_quant_x(const void* x_bf16, const void* w_router_bf16,
                                               const float* bias, int T, int H, int N, int k,
                                               int n_groups, int topk_groups, float* scores,
                                               int32_t* topk_idx, float* topk_gate,
                                               uint8_t* x_q, float* x_d, void* ws,
                                               size_t ws_bytes, hipStream_t stream) {
  return route_topk_bf16(x_bf16, w_router_bf16, bias, T, H, N, k, n_groups, topk_groups, scores,
                         topk_idx, topk_gate, true, x_q, x_d, ws, ws_bytes, stream);
}

extern "C" moe_status_t moe_route_topk_fp8(const uint8_t* x_q, const float* x_d,
                                           const uint8_t* w_router_q, const float* w_router_d,
                                           const float* bias, int T, int H, int N, int k,
                                           int n_groups, int topk_groups, float* scores,
                                           int32_t* topk_idx, float* topk_gate, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || H < 0 || H % 128 != 0 || N < 128 || N > kMaxN || N % 128 != 0 || k < 1 ||
      k > 32 || k > N || !groups_ok(N, k, n_groups, topk_groups))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (H == 0) return MOE_ERR_SHAPE;
  // in-kernel byte offsets are 32-bit
  if ((long long)T * H >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (!x_q || !x_d || !w_router_q || !w_router_d || !bias || !topk_idx || !topk_gate)
    return MOE_ERR_NULL;
  // this path splits H as the bf16 one does, so the bf16 size fits it
  if (!ws || ws_bytes < moe_route_workspace_bytes(T, H, N)) return MOE_ERR_WORKSPACE;
  if (!aligned16(x_q) || !aligned16(w_router_q) || !aligned16(ws) ||
      (reinterpret_cast<uintptr_t>(x_d) & 3) || (reinterpret_cast<uintptr_t>(w_router_d) & 3))
    return MOE_ERR_ALIGN;
  if (moe_status_t st = check_device()) return st;
  static std::atomic<uint64_t> lds_set{0};
  if (moe_status_t st = allow_dynamic_lds(reinterpret_cast<const void*>(&route_partial_fp8_kernel),
                                          kRLdsF, lds_set))
    return st;
  const int S = route_splits(T, H);
  const int tiles = (T + kRT - 1) / kRT;
  const int grid = (tiles * S + 7) / 8 * 8;
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(route_partial_fp8_kernel, dim3(grid), dim3(kRThreads), kRLdsF, stream, x_q,
                     x_d, w_router_q, w_router_d, T, H, N, S, part);
  if (moe_status_t st = launch_status()) return st;
  launch_finish(part, S, bias, T, N, k, n_groups, topk_groups, scores, topk_idx, topk_gate,
                stream);
  return launch_status();
}

extern "C" moe_status_t moe_topk_from_scores(const float* scores, const float* bias, int T, int N,
                                             int k, int n_groups, int topk_groups,
                                             int32_t* topk_idx, float* topk_gate,
                                             hipStream_t stream) {
  if (T < 0 || N < 1 || N > 1024 || k < 1 || k > 32 || k > N ||
      !groups_ok(N, k, n_groups, topk_groups))
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!scores || !bias || !topk_idx || !topk_gate) return MOE_ERR_NULL;
  if (moe_status_t s = check_device()) return s;
  const int blocks = (T + 3) / 4;
  const int per = (N + 63) / 64;
#define MOE_TOPK_LAUNCH(P)                                                                      \
  hipLaunchKernelGGL(topk_scores_kernel<P>, dim3(blocks), dim3(256), 0, stream, scores, bias, T, \
                     N, k, n_groups, topk_groups, topk_idx, topk_gate)
  if (per <= 1) MOE_TOPK_LAUNCH(1);
  else if (per <= 2) MOE_TOPK_LAUNCH(2);
  else if (per <= 4) MOE_TOPK_LAUNCH(4);
  else if (per <= 8) MOE_TOPK_LAUNCH(8);
  else MOE_TOPK_LAUNCH(16);
#undef MOE_TOPK_LAUNCH
  return launch_status();
}

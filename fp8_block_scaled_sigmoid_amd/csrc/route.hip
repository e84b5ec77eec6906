// Sigmoid router with auxiliary-loss-free biased top-k ("DeepSeek-V3:
// Auxiliary-Loss-Free MoE Load Balancing, Multi-Token Prediction, and FP8
// Training at 671B Scale", section III: affinity s = Sigmoid(u . e_i), chosen
// set = TopK of s + b, gate = s normalised over the chosen set, the bias never
// touching the gate; "DeepSeek-V3, explained.", recipe step 4).  The router
// stays in bf16 with float accumulation, as the pages keep the gating network
// out of FP8 (same page, section V, FP8 detail 4).
//
// moe_route_topk: one workgroup owns 32 tokens and every expert (N <= 256), so
// a token's whole score row stays on chip: a bf16 MFMA GEMM (16x16x32) over
// LDS-staged, double-buffered 64-wide K chunks, the sigmoid in the epilogue,
// then each wave selects the top k of 8 tokens by k rounds of a wave-wide
// argmax on a (key, -index) composite, which gives ties to the lower index.
#include "common.h"

namespace {

using namespace moe;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBT = 32;    // tokens per workgroup
constexpr int kKC = 64;    // K chunk, bf16 elements (128 bytes per row)
constexpr int kMaxN = 256;

__device__ __forceinline__ uint32_t sortable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// k rounds of wave-wide argmax over keys held PER lane-slots per lane (expert
// e = lane + 64 * slot).  On return lane j < k holds the j-th chosen expert in
// sel_idx and its unbiased score in sel_s; `sum` (wave-uniform) is the float
// sum of the chosen scores in selection order.
template <int PER>
__device__ __forceinline__ void wave_topk(const float (&key)[PER], const float (&score)[PER],
                                          int N, int k, int lane, int& sel_idx, float& sel_s,
                                          float& sum) {
  uint32_t taken = 0;
  sum = 0.0f;
  sel_idx = -1;
  sel_s = 0.0f;
  for (int r = 0; r < k; ++r) {
    unsigned long long best = 0ull;
#pragma unroll
    for (int s = 0; s < PER; ++s) {
      const int e = lane + 64 * s;
      if (e < N && !((taken >> s) & 1u)) {
        const unsigned long long c =
            ((unsigned long long)sortable(key[s]) << 32) | (0xFFFFFFFFu - (uint32_t)e);
        best = c > best ? c : best;
      }
    }
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    const int owner = e & 63, slot = e >> 6;
    float s_e = 0.0f;
#pragma unroll
    for (int s = 0; s < PER; ++s)
      if (s == slot) s_e = score[s];
    s_e = __shfl(s_e, owner, 64);
    if (lane == owner) taken |= 1u << slot;
    sum = sum + s_e;
    if (lane == r) {
      sel_idx = e;
      sel_s = s_e;
    }
  }
}

__device__ __forceinline__ float sigmoidf_acc(float z) { return 1.0f / (1.0f + expf(-z)); }

// x [T,H] bf16, wr [N,H] bf16, bias [N]; outputs scores [T,N] (optional),
// idx [T,k], gate [T,k].
__global__ __launch_bounds__(256) void route_topk_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int T, int H, int N, int k, float* __restrict__ scores,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  // staging: [2][kBT + kMaxN][kKC] bf16 = 2 * 288 * 128 B = 72 KiB; reused for
  // the score tile [kBT][kMaxN + 4] float after the K loop
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kBT;
  // the stage always holds kBT + kMaxN rows; rows past kBT + N repeat the last
  // expert row and are never read
  constexpr int stage_bytes = (kBT + kMaxN) * 128;

  // global chunk assignment: row rr of the stage (x rows first, then wr rows),
  // 16-byte chunk c (0..7), stored at chunk position c ^ (rr & 7)
  const uint16_t* src_ptr[9];
  int dst_off[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int q = tid + 256 * i;
    const int rr = q >> 3, c = q & 7;
    if (rr < kBT) {
      int t = t0 + rr;
      t = t < T ? t : T - 1;
      src_ptr[i] = x + (long long)t * H + c * 8;
    } else {
      const int e = rr - kBT < N ? rr - kBT : N - 1;
      src_ptr[i] = wr + (long long)e * H + c * 8;
    }
    dst_off[i] = rr * 128 + ((c ^ (rr & 7)) << 4);
  }
  const int NS = N >> 4;  // expert subtiles of 16
  f32x4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x4 reg[9];
#pragma unroll
  for (int i = 0; i < 9; ++i)
    reg[i] = *reinterpret_cast<const i32x4*>(src_ptr[i]);
#pragma unroll
  for (int i = 0; i < 9; ++i)
    *reinterpret_cast<i32x4*>(smem + dst_off[i]) = reg[i];
  __syncthreads();
  const int nkc = H / kKC;
  for (int kc = 0; kc < nkc; ++kc) {
    const int cur = kc & 1;
    const bool more = kc + 1 < nkc;
    if (more) {
#pragma unroll
      for (int i = 0; i < 9; ++i)
        reg[i] = *reinterpret_cast<const i32x4*>(src_ptr[i] + (kc + 1) * kKC);
    }
    const uint8_t* sb = smem + cur * stage_bytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {         // two 32-deep MFMA slices
      const int cpos = 4 * ks + (lane >> 4);  // 16-byte chunk of this lane
      bf16x8 af[2];
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
        const int rr = ti * 16 + (lane & 15);
        af[ti] = *reinterpret_cast<const bf16x8*>(sb + rr * 128 + ((cpos ^ (rr & 7)) << 4));
      }
#pragma unroll
      for (int ei = 0; ei < 4; ++ei) {
        const int es = wave + 4 * ei;
        if (es < NS) {
          const int rr = kBT + es * 16 + (lane & 15);
          const bf16x8 bfr =
              *reinterpret_cast<const bf16x8*>(sb + rr * 128 + ((cpos ^ (rr & 7)) << 4));
#pragma unroll
          for (int ti = 0; ti < 2; ++ti)
            acc[ti][ei] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ti], bfr, acc[ti][ei], 0, 0, 0);
        }
      }
    }
    uint8_t* nb = smem + (cur ^ 1) * stage_bytes;
    if (more) {
#pragma unroll
      for (int i = 0; i < 9; ++i) *reinterpret_cast<i32x4*>(nb + dst_off[i]) = reg[i];
    }
    __syncthreads();
  }

  // epilogue: sigmoid -> score tile in LDS (and global)
  float* sc = reinterpret_cast<float*>(smem);
  const int ldsc = kMaxN + 4;
#pragma unroll
  for (int ei = 0; ei < 4; ++ei) {
    const int es = wave + 4 * ei;
    if (es < NS) {
      const int e = es * 16 + (lane & 15);
#pragma unroll
      for (int ti = 0; ti < 2; ++ti) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tl = ti * 16 + 4 * (lane >> 4) + v;
          const float s = sigmoidf_acc(acc[ti][ei][v]);
          sc[tl * ldsc + e] = s;
          if (scores && t0 + tl < T) scores[(long long)(t0 + tl) * N + e] = s;
        }
      }
    }
  }
  __syncthreads();

  float b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane + 64 * s;
    b[s] = e < N ? bias[e] : 0.0f;
  }
  for (int tl = wave; tl < kBT; tl += 4) {
    const int t = t0 + tl;
    if (t >= T) break;
    float key[4], scr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = lane + 64 * s;
      scr[s] = e < N ? sc[tl * ldsc + e] : 0.0f;
      key[s] = scr[s] + b[s];
    }
    int sel;
    float s_sel, sum;
    wave_topk<4>(key, scr, N, k, lane, sel, s_sel, sum);
    if (lane < k) {
      topk_idx[(long long)t * k + lane] = sel;
      topk_gate[(long long)t * k + lane] = sum > 0.0f ? s_sel / sum : 1.0f / (float)k;
    }
  }
}

// One wave per token over a given score tensor (N <= 64 * PER).
template <int PER>
__global__ __launch_bounds__(256) void topk_scores_kernel(const float* __restrict__ scores,
                                                          const float* __restrict__ bias, int T,
                                                          int N, int k, int32_t* __restrict__ idx,
                                                          float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float key[PER], scr[PER];
#pragma unroll
  for (int s = 0; s < PER; ++s) {
    const int e = lane + 64 * s;
    scr[s] = e < N ? scores[(long long)t * N + e] : 0.0f;
    key[s] = e < N ? scr[s] + bias[e] : 0.0f;
  }
  int sel;
  float s_sel, sum;
  wave_topk<PER>(key, scr, N, k, lane, sel, s_sel, sum);
  if (lane < k) {
    idx[(long long)t * k + lane] = sel;
    gate[(long long)t * k + lane] = sum > 0.0f ? s_sel / sum : 1.0f / (float)k;
  }
}

}  // namespace

extern "C" moe_status_t moe_route_topk(const void* x_bf16, const void* w_router_bf16,
                                       const float* bias, int T, int H, int N, int k,
                                       float* scores, int32_t* topk_idx, float* topk_gate,
                                       hipStream_t stream) {
  if (T < 0 || H < 0 || H % 128 != 0 || N < 16 || N > kMaxN || N % 16 != 0 || k < 1 ||
      k > 32 || k > N)
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (H == 0) return MOE_ERR_SHAPE;
  if (!x_bf16 || !w_router_bf16 || !bias || !topk_idx || !topk_gate) return MOE_ERR_NULL;
  if (!aligned16(x_bf16) || !aligned16(w_router_bf16)) return MOE_ERR_ALIGN;
  if (moe_status_t s = check_device()) return s;
  const size_t lds = 2 * (size_t)(kBT + kMaxN) * 128;   // >= the score tile
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_topk_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return hip_fail(e);
    attr_set = true;
  }
  const int blocks = (T + kBT - 1) / kBT;
  hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(256), lds, stream,
                     static_cast<const uint16_t*>(x_bf16),
                     static_cast<const uint16_t*>(w_router_bf16), bias, T, H, N, k, scores,
                     topk_idx, topk_gate);
  return launch_status();
}

extern "C" moe_status_t moe_topk_from_scores(const float* scores, const float* bias, int T, int N,
                                             int k, int32_t* topk_idx, float* topk_gate,
                                             hipStream_t stream) {
  if (T < 0 || N < 1 || N > 1024 || k < 1 || k > 32 || k > N) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!scores || !bias || !topk_idx || !topk_gate) return MOE_ERR_NULL;
  if (moe_status_t s = check_device()) return s;
  const int blocks = (T + 3) / 4;
  const int per = (N + 63) / 64;
#define MOE_TOPK_LAUNCH(P)                                                                      \
  hipLaunchKernelGGL(topk_scores_kernel<P>, dim3(blocks), dim3(256), 0, stream, scores, bias, T, \
                     N, k, topk_idx, topk_gate)
  if (per <= 1) MOE_TOPK_LAUNCH(1);
  else if (per <= 2) MOE_TOPK_LAUNCH(2);
  else if (per <= 4) MOE_TOPK_LAUNCH(4);
  else if (per <= 8) MOE_TOPK_LAUNCH(8);
  else MOE_TOPK_LAUNCH(16);
#undef MOE_TOPK_LAUNCH
  return launch_status();
}

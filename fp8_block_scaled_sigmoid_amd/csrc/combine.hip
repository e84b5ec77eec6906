// Gate-weighted combine and the sign-based bias update.
//
// Combine ("DeepSeek-V3, explained.", glossary: routed weights sum to 1, the
// shared expert is added at full weight; "DeepSeek-V3: Auxiliary-Loss-Free MoE
// Load Balancing, ...", Figure 2: expert outputs are summed into the block
// output).  An HBM stream: each lane owns 8 columns of one token, issues the
// k + 1 independent 16-byte row loads together, and accumulates in float with
// one fused multiply-add per slot in slot order, so the result does not depend
// on the launch shape.
//
// Bias update (same page, section III "How the bias is set"; "DeepSeek-V3,
// explained.", recipe step 4): overloaded experts lose gamma, underloaded ones
// gain gamma, judged by an exact integer comparison of N * count with T * k.
#include <type_traits>

#include "common.h"

namespace {

using namespace moe;

constexpr int kCombineBlock = 256;

// 16 bytes read once: a non-temporal load keeps them out of the caches' way
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__global__ __launch_bounds__(kCombineBlock) void combine_kernel(
    const uint16_t* __restrict__ out, const float* __restrict__ gate,
    const int32_t* __restrict__ row_of, int shared_row0, int T, int H, int k,
    const uint16_t* __restrict__ residual, uint16_t* __restrict__ y) {
  // one work item = one token x one 8-column chunk, flattened so every lane
  // of every block has work whatever H is
  const int chunks = H >> 3;
  const long long items = (long long)T * chunks;
  // When a row has a multiple of 64 chunks, a wave's 64 items share one token:
  // that copy of the loop reads its slot rows and gates with scalar loads.
  auto run = [&](auto uniform_c) {
    constexpr bool UNIFORM = decltype(uniform_c)::value;
    for (long long item = (long long)blockIdx.x * kCombineBlock + threadIdx.x; item < items;
         item += (long long)gridDim.x * kCombineBlock) {
      int t = (int)(item / chunks);
      if (UNIFORM) t = __builtin_amdgcn_readfirstlane(t);
      const int c8 = (int)(item - (long long)t * chunks);
      float acc[8];
      const long long col = (long long)c8 * 8;
      uint4 base = make_uint4(0, 0, 0, 0);
      if (shared_row0 >= 0)
        base = load_stream(out + (long long)(shared_row0 + t) * H + col);
      const uint32_t bw[4] = {base.x, base.y, base.z, base.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = bf16_lo(bw[i]);
        acc[2 * i + 1] = bf16_hi(bw[i]);
      }
      if (residual) {
        const uint4 r = *reinterpret_cast<const uint4*>(residual + (long long)t * H + col);
        const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = bf16_lo(rw[i]) + acc[2 * i];
          acc[2 * i + 1] = bf16_hi(rw[i]) + acc[2 * i + 1];
        }
      }
      for (int j0 = 0; j0 < k; j0 += 8) {
        const int jn = min(8, k - j0);
        uint4 rows[8];
        float g[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < jn) {
            const int r = row_of[(long long)t * k + j0 + j];
            g[j] = gate[(long long)t * k + j0 + j];
            rows[j] = load_stream(out + (long long)r * H + col);
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (j < jn) {
            const uint32_t w[4] = {rows[j].x, rows[j].y, rows[j].z, rows[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[2 * i] = __builtin_fmaf(g[j], bf16_lo(w[i]), acc[2 * i]);
              acc[2 * i + 1] = __builtin_fmaf(g[j], bf16_hi(w[i]), acc[2 * i + 1]);
            }
          }
        }
      }
      uint4 o;
      o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
      o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
      o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
      o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
      *reinterpret_cast<uint4*>(y + (long long)t * H + col) = o;
    }
  };
  if ((chunks & 63) == 0) run(std::true_type{});
  else run(std::false_type{});
}

__global__ __launch_bounds__(256) void bias_update_kernel(float* __restrict__ bias,
                                                           const int32_t* __restrict__ counts,
                                                           int N, long long target, float gamma) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < N; i += gridDim.x * 256) {
    const long long load = (long long)N * counts[i];
    float step = 0.0f;
    if (load > target) step = -gamma;
    if (load < target) step = gamma;
    bias[i] = bias[i] + step;
  }
}

// Sequence-wise balance statistic ("DeepSeek-V3: Auxiliary-Loss-Free MoE Load
// Balancing, ...", section III, "The one small loss that remains"): per
// sequence s of T_s tokens, L = alpha * sum_i f_i P_i with f_i = N / (k T_s) *
// count_i (normalised load) and P_i = (1 / T_s) * sum of the gates expert i
// received (mean gate mass).  One workgroup per sequence; counts and gate
// masses are integers (gates in units of 2^-32), so the LDS atomics give the
// same sums in any order, and the final sum over experts is a fixed tree in
// double.
__global__ __launch_bounds__(256) void seq_balance_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ gate,
    const int32_t* __restrict__ seq_off, int T, int N, int k, float alpha,
    float* __restrict__ loss) {
  extern __shared__ __align__(16) uint8_t smem[];
  unsigned long long* mass = reinterpret_cast<unsigned long long*>(smem);   // [N]
  uint32_t* cnt = reinterpret_cast<uint32_t*>(smem + (size_t)N * 8);      // [N]
  __shared__ double wsum[4];
  const int s = blockIdx.x, tid = threadIdx.x;
  int t0 = seq_off[s], t1 = seq_off[s + 1];
  t0 = t0 < 0 ? 0 : (t0 > T ? T : t0);
  t1 = t1 < t0 ? t0 : (t1 > T ? T : t1);
  for (int e = tid; e < N; e += 256) {
    mass[e] = 0ull;
    cnt[e] = 0u;
  }
  __syncthreads();
  const long long n = (long long)(t1 - t0) * k;
  for (long long i = tid; i < n; i += 256) {
    const long long a = (long long)t0 * k + i;
    int e = idx[a];
    e = e < 0 ? 0 : (e >= N ? N - 1 : e);
    const double g = (double)gate[a];
    atomicAdd(&cnt[e], 1u);
    atomicAdd(&mass[e], (unsigned long long)__builtin_rint(g * 4294967296.0));
  }
  __syncthreads();
  double term = 0.0;
  for (int e = tid; e < N; e += 256) term += (double)cnt[e] * (double)mass[e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) term += __shfl_xor(term, o, 64);
  if ((tid & 63) == 0) wsum[tid >> 6] = term;
  __syncthreads();
  if (tid == 0) {
    const double tot = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    const int Ts = t1 - t0;
    loss[s] = Ts > 0 ? (float)((double)alpha * N / ((double)k * Ts) * (tot * 0x1p-32) / Ts) : 0.0f;
  }
}

}  // namespace

extern "C" moe_status_t moe_seq_balance_loss(const int32_t* topk_idx, const float* topk_gate,
                                             const int32_t* seq_offsets, int n_seq, int T, int N,
                                             int k, float alpha, float* loss, hipStream_t stream) {
  if (n_seq < 0 || T < 0 || N < 1 || N > 1024 || k < 1 || k > 32) return MOE_ERR_SHAPE;
  if (n_seq == 0) return MOE_OK;
  if (!seq_offsets || !loss || (T > 0 && (!topk_idx || !topk_gate))) return MOE_ERR_NULL;
  if (moe_status_t st = check_device()) return st;
  hipLaunchKernelGGL(seq_balance_kernel, dim3(n_seq), dim3(256), (size_t)N * 12, stream, topk_idx,
                     topk_gate, seq_offsets, T, N, k, alpha, loss);
  return launch_status();
}

extern "C" moe_status_t moe_combine(const void* out_rows_bf16, const float* gate,
                                    const int32_t* row_of, int shared_row0, int T, int H, int k,
                                    const void* residual_bf16, void* y_bf16, hipStream_t stream) {
  if (T < 0 || H < 0 || k < 0 || H % 8 != 0) return MOE_ERR_SHAPE;
  if (T == 0 || H == 0) return MOE_OK;
  if (!out_rows_bf16 || !y_bf16 || (k > 0 && (!gate || !row_of))) return MOE_ERR_NULL;
  if (!aligned16(out_rows_bf16) || !aligned16(y_bf16) ||
      (residual_bf16 && !aligned16(residual_bf16)))
    return MOE_ERR_ALIGN;
  if (moe_status_t s = check_device()) return s;
  const long long items = (long long)T * (H / 8);
  long long blocks = (items + kCombineBlock - 1) / kCombineBlock;
  if (blocks > (1LL << 20)) blocks = 1LL << 20;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kCombineBlock), 0, stream,
                     static_cast<const uint16_t*>(out_rows_bf16), gate, row_of, shared_row0, T, H,
                     k, static_cast<const uint16_t*>(residual_bf16), static_cast<uint16_t*>(y_bf16));
  return launch_status();
}

extern "C" moe_status_t moe_bias_update(float* bias, const int32_t* counts, int N, int T, int k,
                                        float gamma, hipStream_t stream) {
  if (N < 0 || T < 0 || k < 0) return MOE_ERR_SHAPE;
  if (N == 0) return MOE_OK;
  if (!bias || !counts) return MOE_ERR_NULL;
  if (moe_status_t s = check_device()) return s;
  const int blocks = (N + 255) / 256;
  hipLaunchKernelGGL(bias_update_kernel, dim3(blocks), dim3(256), 0, stream, bias, counts, N,
                     (long long)T * k, gamma);
  return launch_status();
}

// Per-expert counts and the token permutation: every (token, slot) assignment
// gets its own row, nothing is dropped ("DeepSeek-V3, explained.", recipe
// step 5), and the counts are the per-expert load the bias controller reads
// ("DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, ...", section III
// flowchart).
//
// A deterministic counting sort in three small launches, with no atomic
// deciding any order:
//   1. per block of 256 tokens: an LDS bit matrix mask[expert][token] (atomic
//      OR only sets bits, so it is order-free); the block's count per expert is
//      a popcount of its row, and an assignment's rank inside the block is the
//      popcount of the bits of earlier tokens;
//   2. one block scans the block counts per expert (block-major), then the
//      expert totals, giving counts, offsets and each block's base row;
//   3. row = offsets[e] + block base + in-block rank; token_of[row] = t, and the
//      shared group's rows T*k + t -> t.
// Rows of one group therefore come in token order.  The k experts of a token
// must be distinct (as top-k makes them); otherwise rows are unspecified but
// stay in bounds.
#include <atomic>

#include "common.h"

// The allocation-free variant's scratch: the per-block expert counts of the
// counting sort, in a file-scope device array of at most kScratchInts ints
// (1 MiB) that each GPU the library runs on holds until the process ends.
// Host code never passes the array's name to a kernel: it looks up the
// array's address on each device once (hipGetSymbolAddress) and uses that.
constexpr size_t kScratchInts = size_t{1} << 18;
static __device__ __align__(256) int32_t scratch[kScratchInts];

namespace {

using namespace moe;

constexpr int kTokPerBlock = 256;
constexpr int kWords = kTokPerBlock / 32;
constexpr int kMaxExperts = 1024;

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                             int T, int N, int k,
                                                             int32_t* __restrict__ blk_counts,
                                                             int32_t* __restrict__ rank) {
  __shared__ uint32_t mask[kMaxExperts * kWords];
  const int b = blockIdx.x;
  const int t0 = b * kTokPerBlock;
  for (int i = threadIdx.x; i < N * kWords; i += 256) mask[i] = 0u;
  __syncthreads();
  const int t = t0 + threadIdx.x;
  const int w = threadIdx.x >> 5, bit = threadIdx.x & 31;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      int e = idx[(long long)t * k + j];
      e = e < 0 ? 0 : (e >= N ? N - 1 : e);
      atomicOr(&mask[e * kWords + w], 1u << bit);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < kWords; ++i) c += __popc(mask[e * kWords + i]);
    blk_counts[(long long)b * N + e] = c;
  }
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      int e = idx[(long long)t * k + j];
      e = e < 0 ? 0 : (e >= N ? N - 1 : e);
      int r = __popc(mask[e * kWords + w] & ((1u << bit) - 1u));
      for (int i = 0; i < w; ++i) r += __popc(mask[e * kWords + i]);
      rank[(long long)t * k + j] = r;
    }
  }
}

// One block of 1024 threads: per-expert scan over blocks, then over experts.
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ blk_counts,
                                                            int n_blocks, int N, int T, int k,
                                                            int with_shared,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[kMaxExperts];
  const int e = threadIdx.x;
  int run = 0;
  if (e < N) {
    // 16 block counts in flight at a time (the loads of one batch are issued
    // before any base row of it is written back)
    for (int b0 = 0; b0 < n_blocks; b0 += 16) {
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        c[i] = b0 + i < n_blocks ? blk_counts[(long long)(b0 + i) * N + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (b0 + i < n_blocks) blk_counts[(long long)(b0 + i) * N + e] = run;  // the block's base row
        run += c[i];
      }
    }
    counts[e] = run;
  }
  tot[e] = e < N ? run : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over the 1024 totals
  for (int o = 1; o < 1024; o <<= 1) {
    const int v = e >= o ? tot[e - o] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < N) offsets[e + 1] = tot[e];
  if (e == 0) {
    offsets[0] = 0;
    offsets[N + 1] = T * k + (with_shared ? T : 0);
  }
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int T, int N, int k, int with_shared,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of, int32_t* __restrict__ token_of) {
  const int t = blockIdx.x * kTokPerBlock + threadIdx.x;
  if (t >= T) return;
  const int b = blockIdx.x;
  for (int j = 0; j < k; ++j) {
    const long long a = (long long)t * k + j;
    int e = idx[a];
    e = e < 0 ? 0 : (e >= N ? N - 1 : e);
    int row = offsets[e] + blk_base[(long long)b * N + e] + row_of[a];  // row_of holds the rank
    row = row < 0 ? 0 : (row >= T * k ? T * k - 1 : row);
    row_of[a] = row;
    token_of[row] = t;
  }
  if (with_shared) token_of[(long long)T * k + t] = t;
}

}  // namespace

extern "C" size_t moe_permute_workspace_bytes(int T, int N, int k) {
  (void)k;
  if (T <= 0 || N <= 0) return 0;
  const size_t blocks = (size_t)(T + kTokPerBlock - 1) / kTokPerBlock;
  return blocks * (size_t)N * sizeof(int32_t);
}

namespace {

moe_status_t check_permute_args(const int32_t* topk_idx, int T, int N, int k, int32_t* counts,
                                int32_t* offsets, int32_t* row_of, int32_t* token_of) {
  if (T < 0 || N < 1 || N > kMaxExperts || k < 1 || k > 32) return MOE_ERR_SHAPE;
  if ((long long)T * (k + 1) > 0x7FFFFFFFLL) return MOE_ERR_SHAPE;
  if (!counts || !offsets) return MOE_ERR_NULL;
  if (T > 0 && (!topk_idx || !row_of || !token_of)) return MOE_ERR_NULL;
  return MOE_OK;
}

moe_status_t launch_permute(const int32_t* topk_idx, int T, int N, int k, int with_shared,
                            int32_t* counts, int32_t* offsets, int32_t* row_of,
                            int32_t* token_of, int32_t* blk, hipStream_t stream) {
  const int n_blocks = (T + kTokPerBlock - 1) / kTokPerBlock;
  if (T > 0)
    hipLaunchKernelGGL(permute_count_kernel, dim3(n_blocks), dim3(256), 0, stream, topk_idx, T, N,
                       k, blk, row_of);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, blk, n_blocks, N, T, k,
                     with_shared ? 1 : 0, counts, offsets);
  if (T > 0)
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(n_blocks), dim3(256), 0, stream, topk_idx, T,
                       N, k, with_shared ? 1 : 0, blk, offsets, row_of, token_of);
  return launch_status();
}

// Device address of `scratch` on the current device, looked up once per
// device (devices 0-63; others on every call).
constexpr int kMaxScratchDevices = 64;
std::atomic<int32_t*> g_scratch_ptr[kMaxScratchDevices];

moe_status_t scratch_on_device(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev >= 0 && dev < kMaxScratchDevices) {
    if (int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire)) {
      *out = p;
      return MOE_OK;
    }
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e);
  if (!p) return MOE_ERR_HIP;
  if (dev >= 0 && dev < kMaxScratchDevices)
    g_scratch_ptr[dev].store(static_cast<int32_t*>(p), std::memory_order_release);
  *out = static_cast<int32_t*>(p);
  return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_permute(const int32_t* topk_idx, int T, int N, int k, int with_shared,
                                    int32_t* counts, int32_t* offsets, int32_t* row_of,
                                    int32_t* token_of, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  if (moe_status_t s = check_permute_args(topk_idx, T, N, k, counts, offsets, row_of, token_of))
    return s;
  const size_t need = moe_permute_workspace_bytes(T, N, k);
  if (T > 0 && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if (moe_status_t s = check_device()) return s;
  return launch_permute(topk_idx, T, N, k, with_shared, counts, offsets, row_of, token_of,
                        static_cast<int32_t*>(ws), stream);
}

extern "C" size_t moe_permute_noalloc_max_scratch_bytes(void) {
  return kScratchInts * sizeof(int32_t);
}

extern "C" moe_status_t moe_permute_noalloc(const int32_t* topk_idx, int T, int N, int k,
                                            int with_shared, int32_t* counts, int32_t* offsets,
                                            int32_t* row_of, int32_t* token_of,
                                            hipStream_t stream) {
  if (moe_status_t s = check_permute_args(topk_idx, T, N, k, counts, offsets, row_of, token_of))
    return s;
  if (moe_permute_workspace_bytes(T, N, k) > kScratchInts * sizeof(int32_t))
    return MOE_ERR_UNSUPPORTED;
  if (moe_status_t s = check_device()) return s;
  int32_t* blk = nullptr;
  if (moe_status_t s = scratch_on_device(&blk)) return s;
  return launch_permute(topk_idx, T, N, k, with_shared, counts, offsets, row_of, token_of, blk,
                        stream);
}

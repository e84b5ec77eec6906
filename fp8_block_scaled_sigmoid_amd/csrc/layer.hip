// The whole forward pass of one DeepSeekMoE layer behind one call.
//
// The steps are the library's own entry points, enqueued in order on one
// stream ("DeepSeek-V3: Auxiliary-Loss-Free MoE Load Balancing, ...", section
// III flowchart and Figure 2; "DeepSeek-V3, explained.", recipe steps 4-7):
// sigmoid router and biased top-k (which also writes the 1x128 activation
// quantisation), counts and permutation, the grouped FP8 GEMM with the SwiGLU + requantisation
// epilogue, the grouped FP8 down projection, the gate-weighted combine and,
// last, the sign-based bias update from this batch's counts.  Every
// intermediate lives in one caller-provided workspace, carved here into
// 256-byte-aligned pieces, so a call allocates nothing and a caller can
// capture it in a HIP graph.  All shape checks run before the first launch:
// a rejected call enqueues nothing.
#include "common.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Byte offsets of the intermediates inside the workspace.
struct LayerCarve {
  size_t idx, gate, counts, offsets, row_of, token_of, perm_ws, route_ws, xq, xd, hq, hd, out_rows;
  size_t route_ws_bytes, perm_ws_bytes;
  size_t total;
};

LayerCarve carve(int T, int H, int N, int k, int I, int with_shared) {
  const size_t t = (size_t)T, h = (size_t)H, n = (size_t)N, kk = (size_t)k, i = (size_t)I;
  const size_t R = t * kk + (with_shared ? t : 0);
  LayerCarve c{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t here = at;
    at += round_up(bytes);
    return here;
  };
  c.idx = take(t * kk * 4);
  c.gate = take(t * kk * 4);
  c.counts = take(n * 4);
  c.offsets = take((n + 2) * 4);
  c.row_of = take(t * kk * 4);
  c.token_of = take(R * 4);
  c.perm_ws_bytes = moe_permute_workspace_bytes(T, N, k);
  c.perm_ws = take(c.perm_ws_bytes);
  c.route_ws_bytes = moe_route_workspace_bytes(T, H, N);
  c.route_ws = take(c.route_ws_bytes);
  c.xq = take(t * h);
  c.xd = take(t * (h / 128) * 4);
  c.hq = take(R * i);
  c.hd = take(R * (i / 128) * 4);
  c.out_rows = take(R * h * 2);
  c.total = at;
  return c;
}

bool layer_shape_ok(const moe_layer_args& a) {
  const int T = a.T, H = a.H, N = a.N, k = a.k, I = a.I;
  if (T < 0 || H <= 0 || H % 128 != 0 || I <= 0 || I % 128 != 0) return false;
  if (H > 16384 || I > 16384) return false;                      // K of either GEMM
  if (k < 1 || k > 32 || k > N || N % 16 != 0 || N < 16 || N > 256) return false;
  if (a.router_fp8 && (N < 128 || N % 128 != 0)) return false;
  if (a.n_groups > 1) {
    const int g = a.n_groups, tg = a.topk_groups;
    if (g > 64 || N % g != 0 || tg < 1 || tg > g || k % tg != 0 || k / tg > N / g) return false;
  }
  return true;
}

bool layer_sizes_supported(const moe_layer_args& a) {
  const long long T = a.T, H = a.H, I = a.I, k = a.k;
  const long long R = T * k + (a.with_shared ? T : 0);
  // 32-bit buffer-resource offsets: x (router, quantiser), the permutation's
  // row numbers and h (GEMM2's A operand).  The expert rows [R, H] are
  // addressed with 64-bit offsets everywhere (GEMM2 epilogue, combine).
  return T * H * 2 < (1LL << 31) && T * (k + 1) <= 0x7FFFFFFFLL && R * I < (1LL << 31);
}

}  // namespace

extern "C" size_t moe_layer_workspace_bytes(int T, int H, int N, int k, int I, int with_shared) {
  if (T < 0 || H <= 0 || H % 128 != 0 || N <= 0 || k <= 0 || I <= 0 || I % 128 != 0) return 0;
  return carve(T, H, N, k, I, with_shared).total;
}

extern "C" moe_status_t moe_layer_forward(const moe_layer_args* args, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  if (!args) return MOE_ERR_NULL;
  const moe_layer_args& a = *args;
  if (!layer_shape_ok(a)) return MOE_ERR_SHAPE;
  if (!layer_sizes_supported(a)) return MOE_ERR_UNSUPPORTED;
  const int T = a.T, H = a.H, N = a.N, k = a.k, I = a.I;
  if (!a.bias || !a.w1_q || !a.w1_d || !a.w2_q || !a.w2_d) return MOE_ERR_NULL;
  if (a.router_fp8 ? (!a.w_router_q || !a.w_router_d) : !a.w_router) return MOE_ERR_NULL;
  if (T > 0 && (!a.x || !a.y)) return MOE_ERR_NULL;
  const LayerCarve c = carve(T, H, N, k, I, a.with_shared);
  if (!ws || ws_bytes < c.total) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_ERR_ALIGN;
  if (T > 0 && (!aligned16(a.x) || !aligned16(a.y) ||
                (a.residual && !aligned16(a.residual))))
    return MOE_ERR_ALIGN;
  if (!aligned16(a.w1_q) || !aligned16(a.w2_q) ||
      (a.router_fp8 ? (!aligned16(a.w_router_q) ||
                       (reinterpret_cast<uintptr_t>(a.w_router_d) & 3))
                    : !aligned16(a.w_router)))
    return MOE_ERR_ALIGN;
  if (moe_status_t st = check_device()) return st;

  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* idx = a.topk_idx ? a.topk_idx : reinterpret_cast<int32_t*>(base + c.idx);
  float* gate = a.topk_gate ? a.topk_gate : reinterpret_cast<float*>(base + c.gate);
  int32_t* counts = a.counts ? a.counts : reinterpret_cast<int32_t*>(base + c.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + c.offsets);
  int32_t* row_of = reinterpret_cast<int32_t*>(base + c.row_of);
  int32_t* token_of = reinterpret_cast<int32_t*>(base + c.token_of);
  uint8_t* xq = base + c.xq;
  float* xd = reinterpret_cast<float*>(base + c.xd);
  uint8_t* hq = base + c.hq;
  float* hd = reinterpret_cast<float*>(base + c.hd);
  void* out_rows = base + c.out_rows;
  const int G = a.with_shared ? N + 1 : N;
  const int R = T * k + (a.with_shared ? T : 0);

  moe_status_t st;
  // x is quantised first when the FP8 router reads the codes; otherwise the
  // bf16 router quantises the x tiles it reads on the way
  if (a.router_fp8) {
    if ((st = fp8_quant_1x128(a.x, MOE_BF16, T, H, H, xq, xd, stream))) return st;
    if ((st = moe_route_topk_fp8(xq, xd, a.w_router_q, a.w_router_d, a.bias, T, H, N, k,
                                 a.n_groups, a.topk_groups, a.scores, idx, gate,
                                 base + c.route_ws, c.route_ws_bytes, stream)))
      return st;
  } else {
    if ((st = moe_route_topk_quant_x(a.x, a.w_router, a.bias, T, H, N, k, a.n_groups,
                                     a.topk_groups, a.scores, idx, gate, xq, xd,
                                     base + c.route_ws, c.route_ws_bytes, stream)))
      return st;
  }
  if ((st = moe_permute(idx, T, N, k, a.with_shared ? 1 : 0, counts, offsets, row_of, token_of,
                        base + c.perm_ws, c.perm_ws_bytes, stream)))
    return st;

  moe_gemm_fp8_args g1{};
  g1.a_q = xq; g1.a_d = xd; g1.lda = H; g1.a_rows = T; g1.a_row_index = token_of;
  g1.b_q = a.w1_q; g1.b_d = a.w1_d; g1.group_offsets = offsets; g1.num_groups = G;
  g1.total_rows = R; g1.n_out = 2 * I; g1.k_dim = H; g1.epilogue = MOE_EPI_SWIGLU_FP8;
  g1.out = hq; g1.out_d = hd; g1.ldo = I; g1.row_scale = nullptr;
  if ((st = moe_grouped_gemm_fp8(&g1, stream))) return st;

  moe_gemm_fp8_args g2{};
  g2.a_q = hq; g2.a_d = hd; g2.lda = I; g2.a_rows = R; g2.a_row_index = nullptr;
  g2.b_q = a.w2_q; g2.b_d = a.w2_d; g2.group_offsets = offsets; g2.num_groups = G;
  g2.total_rows = R; g2.n_out = H; g2.k_dim = I; g2.epilogue = MOE_EPI_BF16;
  g2.out = out_rows; g2.out_d = nullptr; g2.ldo = H; g2.row_scale = nullptr;
  if ((st = moe_grouped_gemm_fp8(&g2, stream))) return st;

  if ((st = moe_combine(out_rows, gate, row_of, a.with_shared ? T * k : -1, T, H, k, a.residual,
                        a.y, stream)))
    return st;
  if (a.update_bias && (st = moe_bias_update(a.bias, counts, N, T, k, a.gamma, stream))) return st;
  return MOE_OK;
}

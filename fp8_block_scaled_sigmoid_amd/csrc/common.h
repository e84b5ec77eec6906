// Shared device and host helpers of libmoe_fp8.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "moe_fp8.h"

#ifndef __HIP_DEVICE_COMPILE__
#include <cstring>
#endif

namespace moe {

// ---------------------------------------------------------------------------
// E4M3 ("fn", max 448) encoder: round to nearest, ties to the even code,
// saturating, sign kept.  gfx950's float -> OCP E4M3 conversion rounds to
// nearest even and keeps the sign; clamping to +-448 first gives the
// saturation (without it, magnitudes of 464 and above would become NaN).  This
// equals the format's definition on every finite float (checked exhaustively
// against a step-by-step software encoder on the device).
__device__ __forceinline__ float e4m3_clamp(float v) {
  return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
}
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(v), 0.0f, 0, false) & 0xFFu;
}
// four codes packed little-endian: a in bits 0-7, b 8-15, c 16-23, d 24-31
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), w, true);
  return (uint32_t)w;
}

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Quantisation multiplier and stored factor of a tile with absolute maximum
// amax: m = fl32(448 / amax), d = fl32(amax / 448); a zero tile, or one whose m
// overflows, gets m = 0 (all codes 0x00) and d = 1.
__device__ __forceinline__ void tile_scale(float amax, float& m, float& d) {
  m = 448.0f / amax;
  d = amax / 448.0f;
  if (!(amax > 0.0f) || !(m <= 3.402823466e38f)) {
    m = 0.0f;
    d = 1.0f;
  }
}

// Code of x * m with the zero-tile rule (m == 0 gives +0 -> 0x00).
__device__ __forceinline__ uint32_t quant_code(float x, float m) {
  return m == 0.0f ? 0u : e4m3_encode(x * m);
}

template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int ceil_div_dev(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe

// ---------------------------------------------------------------------------
// host side
namespace moe {

moe_status_t check_device();                  // MOE_ERR_DEVICE unless gfx950
moe_status_t hip_fail(hipError_t e);          // records e, returns MOE_ERR_HIP
moe_status_t launch_status();                 // hipGetLastError -> status
int cu_count();                               // compute units of the current device (0 on error)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Lets kernel `func` use `bytes` of dynamic LDS on the current device.  The
// attribute is set once per (launch site, device): `done` is the launch site's
// mask of devices already set (bit d for device d < 64; devices beyond 63 are
// set on every call).  Safe to call from several host threads at once.
moe_status_t allow_dynamic_lds(const void* func, int bytes, std::atomic<uint64_t>& done);

}  // namespace moe

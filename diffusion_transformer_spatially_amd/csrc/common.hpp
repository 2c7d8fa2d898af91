// Internal helpers shared by the gfx950 kernels and the host entry points (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "safe_attn.h"

namespace safe {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32 on raw 16-bit patterns.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  // Round to nearest even; NaN kept quiet.
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 16-byte loads that bypass the caches' retention (nontemporal): for inputs streamed once.
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float4* p) {
  const f32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_nt*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
  const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroup id remap so that consecutive logical tiles land on the same XCD (the hardware deals
// workgroup ids round-robin over the 8 XCDs, each with its own L2).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t x, uint32_t G) {
  const uint32_t G8 = G & ~7u;
  if (x >= G8) return x;
  return (x & 7u) * (G8 >> 3) + (x >> 3);
}

// Per-call kernel arguments of the attention kernels.
struct AttnArgs {
  const void* q;
  const void* k_img;
  const void* v_img;
  const void* k_txt;
  const void* v_txt;
  void* out;
  float* lse;
  float* xattn_out;
  float* lse_img_out;
  const int32_t* rows;  // nullptr for dense
  const void* mask;
  int32_t mask_dtype, mask_B, mask_H, mask_cols;
  const float* q_descale;  // fp8 Q / K: per-(b,h) dequantisation factors, nullptr = 1
  const float* k_descale;
  int32_t B, H, N, T, R;  // R = number of query rows computed per (b,h)
  float scale;            // natural-log logit scale
  int32_t tv[SAFE_MAX_BATCH];
};

}  // namespace safe

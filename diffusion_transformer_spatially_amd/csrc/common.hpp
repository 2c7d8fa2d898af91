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

__device__ __forceinline__ void store_nt(float4* p, float4 v) {
  const f32x4_nt w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4_nt*>(p));
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
  typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
  const u32x4_nt w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_nt*>(p));
}

// Streaming launches: a launch that moves more bytes than the 256 MB MALL (the last-level cache in front of
// HBM) cannot keep its data cache-resident, so its once-used inputs and its outputs go through nontemporal
// loads and stores (measured on MI355X with back-to-back launches over buffers larger than the MALL: row
// gather 103 -> 90 us, SW-CFG 52 -> 47 us, StepCache 49 -> 44 us, PCSP 129 -> 118 us, mask scan 122 -> 111 us);
// smaller launches keep plain accesses, so that data a previous kernel left in the MALL is used (with
// nontemporal accesses the cache-resident 28 MB SW-CFG took 6.8 instead of 4.5 us).
constexpr double kStreamBytes = 256.0 * 1024 * 1024;

template <bool NT, class T>
__device__ __forceinline__ T load_s(const T* p) {
  if constexpr (NT) return load_nt(p);
  else return *p;
}
template <bool NT, class T>
__device__ __forceinline__ void store_s(T* p, T v) {
  if constexpr (NT) store_nt(p, v);
  else *p = v;
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

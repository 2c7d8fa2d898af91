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
  int32_t B, H, N, T, R;  // R = number of query rows computed per (b,h)
  float scale;            // natural-log logit scale
  int32_t tv[SAFE_MAX_BATCH];
};

// Launchers (each returns a HIP error code; validation happens before they are called).
hipError_t launch_attn_mfma_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_generic(const AttnArgs& a, int dtype, hipStream_t s);
hipError_t launch_mask_check(const void* mask, int mask_dtype, int mB, int mH, int N, int cols, int T,
                             const int32_t* tv, int B, int32_t* flag, float* c_out, hipStream_t s);
hipError_t launch_pcsp_accumulate(const float* x, const float* lse_img, int H, int N, int T, int Tv, int c0, int c1,
                                  float* scores, int accumulate, hipStream_t s);
hipError_t launch_pcsp_partition(const float* scores, int N, int k, int32_t* S, int32_t* C, uint8_t* is_sens,
                                 float* s01, hipStream_t s);
hipError_t launch_swcfg(const float* eps, const float* sv, int C, int Hl, int Wl, int side, float g_ctx, float g_sens,
                        float* out, hipStream_t s);
hipError_t launch_affinity_accumulate(const float* x, const float* lse_img, int H, int N, int T, int Tv,
                                      const uint8_t* sel, float* scores, int accumulate, hipStream_t s);
hipError_t launch_stepcache(const float* eps_a, const float* eps_b, size_t n, float w, float* out, hipStream_t s);
hipError_t launch_rows_ffn(const uint16_t* x, const int32_t* rows, int k, int B, int N, int D, int F,
                           const uint16_t* w1, const float* b1, const uint16_t* w2, const float* b2, uint16_t* cache,
                           uint16_t* hidden, hipStream_t s);
hipError_t launch_rows_qkv(const uint16_t* x, const int32_t* rows, int k, int B, int N, int H, int d,
                           const uint16_t* wqkv, const float* bqkv, uint16_t* q, uint16_t* kc, uint16_t* vc,
                           hipStream_t s);
hipError_t launch_rows_copy(const void* src, void* dst, const int32_t* rows, int k, int B, int H, int N,
                            int row_bytes, bool scatter, hipStream_t s);

}  // namespace safe

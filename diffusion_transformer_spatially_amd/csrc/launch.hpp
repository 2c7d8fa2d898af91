// Launchers of the kernels, called by the C entry points in api.hip (not part of the ABI).
#pragma once
#include "common.hpp"

namespace safe {

// Launchers (each returns a HIP error code; validation happens before they are called).
hipError_t launch_attn_mfma_bf16(const AttnArgs& a, int d, hipStream_t s);
hipError_t launch_attn_mfma_fp8(const AttnArgs& a, int d, hipStream_t s);
hipError_t launch_attn_generic(const AttnArgs& a, int dtype, int d, hipStream_t s);
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

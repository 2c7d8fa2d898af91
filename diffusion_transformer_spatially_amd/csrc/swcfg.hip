// SW-CFG combine (SAFE-DiT technical summary, Methodology 4; AccelAes summary B.2, spatial CFG):
// gamma_i = g_ctx + (g_sens - g_ctx) s_i per token, out = eps_u + gamma (eps_c - eps_u) per latent
// pixel.  Elementwise and HBM-bound: 8 bytes read and 4 written per pixel, float4 vectors along x.
#include "common.hpp"

namespace safe {

__device__ __forceinline__ float guided(float ec, float eu, float g) { return fmaf(g, ec - eu, eu); }

__global__ __launch_bounds__(256) void k_swcfg_vec(const float4* __restrict__ ec4, const float4* __restrict__ eu4,
                                                   const float* __restrict__ sv, uint32_t Wl4, uint32_t Hl,
                                                   uint32_t side, uint32_t ph, uint32_t pw, float g_ctx, float g_d,
                                                   float4* __restrict__ out4, uint32_t total4) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < total4; e += stride) {
    const uint32_t x0 = (e % Wl4) * 4;
    const uint32_t y = (e / Wl4) % Hl;
    const uint32_t trow = (y / ph) * side;
    const float4 c = ec4[e];
    const float4 u = eu4[e];
    float4 o;
    o.x = guided(c.x, u.x, fmaf(g_d, sv[trow + (x0 + 0) / pw], g_ctx));
    o.y = guided(c.y, u.y, fmaf(g_d, sv[trow + (x0 + 1) / pw], g_ctx));
    o.z = guided(c.z, u.z, fmaf(g_d, sv[trow + (x0 + 2) / pw], g_ctx));
    o.w = guided(c.w, u.w, fmaf(g_d, sv[trow + (x0 + 3) / pw], g_ctx));
    out4[e] = o;
  }
}

__global__ __launch_bounds__(256) void k_swcfg_scalar(const float* __restrict__ ec, const float* __restrict__ eu,
                                                      const float* __restrict__ sv, uint32_t Wl, uint32_t Hl,
                                                      uint32_t side, uint32_t ph, uint32_t pw, float g_ctx, float g_d,
                                                      float* __restrict__ out, uint32_t total) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const uint32_t x = e % Wl;
    const uint32_t y = (e / Wl) % Hl;
    out[e] = guided(ec[e], eu[e], fmaf(g_d, sv[(y / ph) * side + x / pw], g_ctx));
  }
}

hipError_t launch_swcfg(const float* eps, const float* sv, int C, int Hl, int Wl, int side, float g_ctx, float g_sens,
                        float* out, hipStream_t s) {
  const uint32_t total = static_cast<uint32_t>(C) * Hl * Wl;
  const uint32_t ph = Hl / side, pw = Wl / side;
  const float g_d = g_sens - g_ctx;
  const bool vec = (Wl % 4 == 0) && ((reinterpret_cast<uintptr_t>(eps) | reinterpret_cast<uintptr_t>(out)) % 16 == 0);
  if (vec) {
    const uint32_t total4 = total / 4;
    uint32_t blocks = (total4 + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    k_swcfg_vec<<<blocks, 256, 0, s>>>(reinterpret_cast<const float4*>(eps), reinterpret_cast<const float4*>(eps + total),
                                        sv, Wl / 4, Hl, side, ph, pw, g_ctx, g_d, reinterpret_cast<float4*>(out), total4);
  } else {
    uint32_t blocks = (total + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    k_swcfg_scalar<<<blocks, 256, 0, s>>>(eps, eps + total, sv, Wl, Hl, side, ph, pw, g_ctx, g_d, out, total);
  }
  return hipGetLastError();
}

}  // namespace safe

// SW-CFG combine (SAFE-DiT technical summary, Methodology 4; AccelAes summary B.2, spatial CFG):
// gamma_i = g_ctx + (g_sens - g_ctx) s_i per token, out = eps_u + gamma (eps_c - eps_u) per latent
// pixel.  Elementwise and HBM-bound: 8 bytes read and 4 written per pixel, float4 vectors along x
// (nontemporal when the launch moves more than the MALL holds).
// The pixel -> token index arithmetic must stay cheaper than the memory traffic, so the vector path
// divides through float reciprocals (exactly, see fdiv) instead of 32-bit integer divisions.
#include "common.hpp"

namespace safe {

__device__ __forceinline__ float guided(float ec, float eu, float g) { return fmaf(g, ec - eu, eu); }

// gamma = g_ctx (1 - s) + g_sens s, the mix of the two scales: with s in [0, 1] and scales of one sign the two
// products never cancel, so gamma keeps fp32 relative accuracy even where it is small beside g_ctx (the
// form g_ctx + (g_sens - g_ctx) s rounds g_sens - g_ctx first, an absolute error of about one ulp of the larger
// scale), and s = 0 / s = 1 give g_ctx / g_sens exactly; equal scales give that scale exactly (global CFG).
__device__ __forceinline__ float gamma_of(float s, float g_ctx, float g_sens) {
  return g_ctx == g_sens ? g_ctx : fmaf(g_sens, s, g_ctx * (1.f - s));
}

// floor(a / b) for a < 2^24 without an integer divide: the float quotient is off by at most one, and
// one exact integer comparison each way fixes it.
struct FastDiv {
  uint32_t b;
  float inv;
};
__device__ __forceinline__ uint32_t fdiv(uint32_t a, FastDiv d) {
  uint32_t q = static_cast<uint32_t>(static_cast<float>(a) * d.inv);
  q -= (q * d.b > a) ? 1u : 0u;
  q += ((q + 1u) * d.b <= a) ? 1u : 0u;
  return q;
}

template <bool NT>
__global__ __launch_bounds__(256) void k_swcfg_vec(const float4* __restrict__ ec4, const float4* __restrict__ eu4,
                                                   const float* __restrict__ sv, FastDiv wl4, FastDiv hl,
                                                   uint32_t side, FastDiv ph, FastDiv pw, float g_ctx, float g_sens,
                                                   float4* __restrict__ out4, uint32_t total4) {
  const uint32_t e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= total4) return;
  const float4 c = load_s<NT>(ec4 + e);
  const float4 u = load_s<NT>(eu4 + e);
  const uint32_t row = fdiv(e, wl4);           // c * Hl + y
  const uint32_t x0 = (e - row * wl4.b) * 4;
  const uint32_t y = row - fdiv(row, hl) * hl.b;
  const uint32_t trow = fdiv(y, ph) * side;
  float4 o;
  if (pw.b >= 2) {
    // four consecutive pixels span at most two tokens: load the first and the last one's score
    const uint32_t tf = fdiv(x0, pw), tl = fdiv(x0 + 3, pw);
    const uint32_t split = (tf + 1) * pw.b;  // first pixel of the next token
    const float ga = gamma_of(sv[trow + tf], g_ctx, g_sens), gb = gamma_of(sv[trow + tl], g_ctx, g_sens);
    o.x = guided(c.x, u.x, ga);
    o.y = guided(c.y, u.y, x0 + 1 >= split ? gb : ga);
    o.z = guided(c.z, u.z, x0 + 2 >= split ? gb : ga);
    o.w = guided(c.w, u.w, gb);
  } else {
    o.x = guided(c.x, u.x, gamma_of(sv[trow + x0 + 0], g_ctx, g_sens));
    o.y = guided(c.y, u.y, gamma_of(sv[trow + x0 + 1], g_ctx, g_sens));
    o.z = guided(c.z, u.z, gamma_of(sv[trow + x0 + 2], g_ctx, g_sens));
    o.w = guided(c.w, u.w, gamma_of(sv[trow + x0 + 3], g_ctx, g_sens));
  }
  store_s<NT>(out4 + e, o);
}

__global__ __launch_bounds__(256) void k_swcfg_scalar(const float* __restrict__ ec, const float* __restrict__ eu,
                                                      const float* __restrict__ sv, uint32_t Wl, uint32_t Hl,
                                                      uint32_t side, uint32_t ph, uint32_t pw, float g_ctx, float g_sens,
                                                      float* __restrict__ out, uint32_t total) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const uint32_t x = e % Wl;
    const uint32_t y = (e / Wl) % Hl;
    out[e] = guided(ec[e], eu[e], gamma_of(sv[(y / ph) * side + x / pw], g_ctx, g_sens));
  }
}

hipError_t launch_swcfg(const float* eps, const float* sv, int C, int Hl, int Wl, int side, float g_ctx, float g_sens,
                        float* out, hipStream_t s) {
  const uint32_t total = static_cast<uint32_t>(C) * Hl * Wl;
  const uint32_t ph = Hl / side, pw = Wl / side;
  const bool vec = (Wl % 4 == 0) && ((reinterpret_cast<uintptr_t>(eps) | reinterpret_cast<uintptr_t>(out)) % 16 == 0);
  if (vec && total / 4 < (1u << 24)) {
    // one float4 per thread; the index arithmetic uses the float-reciprocal division (exact below 2^24)
    const uint32_t total4 = total / 4;
    auto fd = [](uint32_t b) { return FastDiv{b, 1.0f / static_cast<float>(b)}; };
    const bool nt = 12.0 * total > kStreamBytes;  // two predictions read, one written
    auto kern = nt ? k_swcfg_vec<true> : k_swcfg_vec<false>;
    kern<<<(total4 + 255) / 256, 256, 0, s>>>(
        reinterpret_cast<const float4*>(eps), reinterpret_cast<const float4*>(eps + total), sv, fd(Wl / 4), fd(Hl),
        side, fd(ph), fd(pw), g_ctx, g_sens, reinterpret_cast<float4*>(out), total4);
  } else {
    uint32_t blocks = (total + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    k_swcfg_scalar<<<blocks, 256, 0, s>>>(eps, eps + total, sv, Wl, Hl, side, ph, pw, g_ctx, g_sens, out, total);
  }
  return hipGetLastError();
}

}  // namespace safe

// StepCache (AccelAes technical summary, 2. Methodology B.3): between full steps the noise prediction is
// the line through the last two full predictions, out = eps_b + w (eps_b - eps_a).  Elementwise and
// HBM-bound: 8 bytes read and 4 written per element (nontemporal when the launch moves more than the MALL
// holds).  out may alias an input element for element, so
// the pointers are not restrict-qualified (each element is read before it is written, by one thread).
#include "common.hpp"

namespace safe {

__device__ __forceinline__ float extrap(float a, float b, float w) { return fmaf(w, b - a, b); }

// One float4 per thread; the thread just past the last full vector also takes the 1-3 trailing elements.
template <bool NT>
__global__ __launch_bounds__(256) void k_stepcache_vec(const float* a, const float* b,
                                                       float w, float* out, size_t n) {
  const size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t n4 = n / 4;
  if (e < n4) {
    const float4 va = load_s<NT>(reinterpret_cast<const float4*>(a) + e);
    const float4 vb = load_s<NT>(reinterpret_cast<const float4*>(b) + e);
    float4 o;
    o.x = extrap(va.x, vb.x, w);
    o.y = extrap(va.y, vb.y, w);
    o.z = extrap(va.z, vb.z, w);
    o.w = extrap(va.w, vb.w, w);
    store_s<NT>(reinterpret_cast<float4*>(out) + e, o);
  } else if (e == n4) {
    for (size_t i = 4 * n4; i < n; ++i) out[i] = extrap(a[i], b[i], w);
  }
}

// Any alignment: one element per thread.
__global__ __launch_bounds__(256) void k_stepcache_scalar(const float* a, const float* b,
                                                          float w, float* out, size_t n) {
  const size_t e = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e < n) out[e] = extrap(a[e], b[e], w);
}

hipError_t launch_stepcache(const float* eps_a, const float* eps_b, size_t n, float w, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const bool vec = ((reinterpret_cast<uintptr_t>(eps_a) | reinterpret_cast<uintptr_t>(eps_b) |
                     reinterpret_cast<uintptr_t>(out)) % 16) == 0;
  if (vec) {
    const size_t threads = n / 4 + 1;  // the extra thread takes the tail (if any)
    auto kern = 12.0 * n > kStreamBytes ? k_stepcache_vec<true> : k_stepcache_vec<false>;
    kern<<<static_cast<uint32_t>((threads + 255) / 256), 256, 0, s>>>(eps_a, eps_b, w, out, n);
  } else {
    k_stepcache_scalar<<<static_cast<uint32_t>((n + 255) / 256), 256, 0, s>>>(eps_a, eps_b, w, out, n);
  }
  return hipGetLastError();
}

}  // namespace safe

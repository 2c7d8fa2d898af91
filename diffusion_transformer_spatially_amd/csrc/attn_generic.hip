// General attention kernel on the vector ALUs: fp32 or bf16 storage (or fp8 E4M3 Q / K with bf16 V and
// output), dense or sensitive rows, optional kept additive mask (fp32 or bool), optional warmup emission.
// It serves the fp32 path and the bf16 / fp8 kept-mask calls the MFMA kernel does not take (an emission
// request, N or the mask row length not a multiple of 16, an unaligned mask, or an fp32 mask at head dim
// 128); all other bf16 and fp8 calls run on the MFMA kernel.  fp8 codes are decoded exactly to fp32 and the
// per-(b,h) dequantisation factors of Q and K scale the dot products, as the logit scale does.
//
// Semantics (SAFE-DiT technical summary, Methodology 1 and 3): one joint softmax per image query row
// over the image keys then the valid text keys (padded text slots never enter), logits scaled by
// `scale`, kept mask added; a fully masked row yields 0 and lse = -inf.
//
// Layout: D / 64 threads per query row, each holding 64 dims of q and of the output accumulators in
// registers (head dim 64: one thread per row, 256 rows per workgroup; head dim 128: two adjacent threads
// per row, 128 rows per workgroup, their partial dot products summed with one lane exchange); 32-key
// tiles of K and V are staged in LDS as fp32 and read as broadcasts.
#include "common.hpp"

namespace safe {

constexpr int kGenThreads = 256;
constexpr int kGenPart = 64;  // head dims per thread
constexpr int kGenTile = 32;

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
// OCP E4M3 (sign, 4 exponent bits of bias 7, 3 mantissa bits; no infinities, S.1111.111 is NaN): normal codes
// are (1 + m/8) 2^(e-7), placed directly in the fp32 exponent and mantissa fields; subnormals m 2^-9.
template <>
__device__ __forceinline__ float ld<uint8_t>(const uint8_t* p, size_t i) {
  const uint32_t c = p[i];
  const uint32_t sgn = (c & 0x80u) << 24, e = (c >> 3) & 0xfu, m = c & 7u;
  if ((c & 0x7fu) == 0x7fu) return __uint_as_float(sgn | 0x7fc00000u);
  if (e == 0) return __uint_as_float(sgn | __float_as_uint(static_cast<float>(m) * 0.001953125f));
  return __uint_as_float(sgn | ((e + 120u) << 23) | (m << 20));
}

template <typename T>
__device__ __forceinline__ void st(T* p, size_t i, float v);
template <>
__device__ __forceinline__ void st<float>(float* p, size_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16_rne(v); }

// T: storage of V and the output (and of Q / K unless TQ says otherwise); TQ: storage of Q and K
template <typename T, bool HAS_MASK, int D, typename TQ = T>
__global__ __launch_bounds__(kGenThreads) void k_attn_generic(AttnArgs a) {
  constexpr int kLpr = D / kGenPart;             // threads per query row
  constexpr int kRows = kGenThreads / kLpr;      // query rows per workgroup
  __shared__ float ks[kGenTile][D];
  __shared__ float vs[kGenTile][D];
  const int nqb = (a.R + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqb;
  const int qb = blockIdx.x - bh * nqb;
  const int b = bh / a.H, h = bh - b * a.H;
  const int part = static_cast<int>(threadIdx.x) % kLpr;  // which 64 dims of the row this thread holds
  const int c0 = part * kGenPart;
  const int r = qb * kRows + static_cast<int>(threadIdx.x) / kLpr;
  const bool active = r < a.R;
  int row = active ? (a.rows ? a.rows[r] : r) : 0;
  const bool valid_row = active && row >= 0 && row < a.N;
  if (!valid_row) row = 0;
  const int tv = a.tv[b];
  const TQ* Q = static_cast<const TQ*>(a.q) + static_cast<size_t>(bh) * a.N * D;
  const TQ* KI = static_cast<const TQ*>(a.k_img) + static_cast<size_t>(bh) * a.N * D;
  const T* VI = static_cast<const T*>(a.v_img) + static_cast<size_t>(bh) * a.N * D;
  const TQ* KT = static_cast<const TQ*>(a.k_txt) + static_cast<size_t>(bh) * a.T * D;
  const T* VT = static_cast<const T*>(a.v_txt) + static_cast<size_t>(bh) * a.T * D;
  // the logit scale in the units of the dot products (fp8 codes: times the (b,h) factors of Q and K)
  float scale = a.scale;
  if (a.q_descale != nullptr) scale *= a.q_descale[bh];
  if (a.k_descale != nullptr) scale *= a.k_descale[bh];

  float q[kGenPart], o[kGenPart];
#pragma unroll
  for (int c = 0; c < kGenPart; ++c) {
    q[c] = ld(Q, static_cast<size_t>(row) * D + c0 + c);
    o[c] = 0.f;
  }
  // mask row pointer (fp32 entries or bool bytes)
  const uint8_t* mrow = nullptr;
  if (HAS_MASK) {
    const int mb = a.mask_B == 1 ? 0 : b, mh = a.mask_H == 1 ? 0 : h;
    const int esz = a.mask_dtype == SAFE_DTYPE_BOOL ? 1 : 4;
    mrow = static_cast<const uint8_t*>(a.mask) +
           ((static_cast<size_t>(mb) * a.mask_H + mh) * a.N + row) * static_cast<size_t>(a.mask_cols) * esz;
  }
  const bool emit = (a.xattn_out != nullptr || a.lse_img_out != nullptr) && b == 0;
  float m = -INFINITY, l = 0.f;
  const int n_img_tiles = (a.N + kGenTile - 1) / kGenTile;
  const int n_txt_tiles = (tv + kGenTile - 1) / kGenTile;
  for (int t = 0; t < n_img_tiles + n_txt_tiles; ++t) {
    const bool txt = t >= n_img_tiles;
    const int j0 = txt ? (t - n_img_tiles) * kGenTile : t * kGenTile;
    const int nvalid = txt ? min(kGenTile, tv - j0) : min(kGenTile, a.N - j0);
    const TQ* Ksrc = txt ? KT : KI;
    const T* Vsrc = txt ? VT : VI;
    __syncthreads();
    for (int e = threadIdx.x; e < kGenTile * D; e += kGenThreads) {
      const int jj = e / D, c = e - jj * D;
      const bool ok = jj < nvalid;
      ks[jj][c] = ok ? ld(Ksrc, static_cast<size_t>(j0 + jj) * D + c) : 0.f;
      vs[jj][c] = ok ? ld(Vsrc, static_cast<size_t>(j0 + jj) * D + c) : 0.f;
    }
    __syncthreads();
    // logits of this tile, in log2 units, mask included
    float s[kGenTile];
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < kGenTile; ++jj) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < kGenPart; ++c) acc = fmaf(q[c], ks[jj][c0 + c], acc);
      if constexpr (kLpr == 2) acc += __shfl_xor(acc, 1);  // the other half of the row's dot product
      float z = acc * scale;  // natural-log logit
      if (HAS_MASK) {
        const int col = (txt ? a.N : 0) + j0 + jj;
        float mv = 0.f;
        if (jj < nvalid && (!txt || a.mask_cols != a.N)) {
          if (a.mask_dtype == SAFE_DTYPE_BOOL) mv = mrow[col] ? 0.f : -INFINITY;
          else mv = reinterpret_cast<const float*>(mrow)[col];
        }
        z += mv;
      }
      if (emit && txt && a.xattn_out != nullptr && valid_row && jj < nvalid && part == 0)
        a.xattn_out[(static_cast<size_t>(h) * a.N + row) * a.T + j0 + jj] = z;
      s[jj] = jj < nvalid ? z * kLog2e : -INFINITY;
      tmax = fmaxf(tmax, s[jj]);
    }
    const float mnew = fmaxf(m, tmax);
    if (mnew != -INFINITY) {
      const float alpha = exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int c = 0; c < kGenPart; ++c) o[c] *= alpha;
#pragma unroll
      for (int jj = 0; jj < kGenTile; ++jj) {
        const float p = exp2f(s[jj] - mnew);
        l += p;
#pragma unroll
        for (int c = 0; c < kGenPart; ++c) o[c] = fmaf(p, vs[jj][c0 + c], o[c]);
      }
      m = mnew;
    }
    if (emit && t == n_img_tiles - 1 && a.lse_img_out != nullptr && valid_row && part == 0)
      a.lse_img_out[static_cast<size_t>(h) * a.N + row] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
  if (!valid_row) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  T* O = static_cast<T*>(a.out) + static_cast<size_t>(bh) * a.N * D;
#pragma unroll
  for (int c = 0; c < kGenPart; ++c) st(O, static_cast<size_t>(row) * D + c0 + c, o[c] * inv);
  if (a.lse != nullptr && part == 0)
    a.lse[static_cast<size_t>(bh) * a.N + row] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <int D>
static void launch_generic(const AttnArgs& a, int dtype, hipStream_t s) {
  constexpr int kRows = kGenThreads / (D / kGenPart);
  const int nqb = (a.R + kRows - 1) / kRows;
  const uint32_t grid = static_cast<uint32_t>(a.B) * a.H * nqb;
  const bool mask = a.mask != nullptr;
  if (dtype == SAFE_DTYPE_F32) {
    if (mask) k_attn_generic<float, true, D><<<grid, kGenThreads, 0, s>>>(a);
    else k_attn_generic<float, false, D><<<grid, kGenThreads, 0, s>>>(a);
  } else if (dtype == SAFE_DTYPE_FP8_E4M3) {
    if (mask) k_attn_generic<uint16_t, true, D, uint8_t><<<grid, kGenThreads, 0, s>>>(a);
    else k_attn_generic<uint16_t, false, D, uint8_t><<<grid, kGenThreads, 0, s>>>(a);
  } else {
    if (mask) k_attn_generic<uint16_t, true, D><<<grid, kGenThreads, 0, s>>>(a);
    else k_attn_generic<uint16_t, false, D><<<grid, kGenThreads, 0, s>>>(a);
  }
}

hipError_t launch_attn_generic(const AttnArgs& a, int dtype, int d, hipStream_t s) {
  if (d == 128) launch_generic<128>(a, dtype, s);
  else launch_generic<64>(a, dtype, s);
  return hipGetLastError();
}

}  // namespace safe

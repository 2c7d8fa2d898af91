// Products of the sensitive-row update (SAFE-DiT technical summary, Methodology 3: only the rows of S are
// recomputed in a non-anchor step; AccelAes technical summary, Methodology B.2 SkipSparse: the FFN of the
// context tokens is skipped and its cached output reused):
//   Y[t, j] = epi( sum_c X[src(t), c] * W[j, c] + bias[j] ),   t < T = B * k tokens, j < Dout,
// with W in nn.Linear layout [Dout, Din], bf16 operands, fp32 accumulation, bf16 output.
//
// Shape of the work:
//  * D^T = W X^T on v_mfma_f32_32x32x16_bf16: output features are the M dimension, tokens the N
//    dimension, and both operands are K-contiguous rows (weight rows, token rows), so both come from
//    row-major LDS tiles with 16-byte reads; a fixed permutation of the weight rows fed to the
//    instruction makes output register r of lane half g hold feature 16 g + r, i.e. every lane ends with
//    16 consecutive features of one token: the epilogue (bias, GELU, bf16 pack) runs in registers and
//    stores 32 contiguous bytes per lane, wherever the token's row lives;
//  * wide products (D -> F, QKV): 256 features x 256 tokens per 8-wave workgroup (one per CU, two waves per
//    SIMD), each wave 128 x 64 (4 x 2 blocks of 32 x 32): 128 flop per byte loaded, 6 KB of LDS reads per
//    8 matrix instructions; narrow products (F -> D): 128 x 128 per 4-wave workgroup (enough workgroups to
//    fill the GPU); K streams through double-buffered LDS (two distinct objects per operand) filled by
//    direct global -> LDS copies, which are pinned ahead of the stage's matrix work, in stages of 64 on the
//    wide products and of 128 on the narrow ones (one 4-wave workgroup per CU with 128 KB of LDS: twice the
//    matrix work per barrier, enough to cover the next stage's copy); within a stage the operands of K step
//    ks + 1 are read while the matrix instructions of step ks run;
//  * LDS rows of 128 bytes (stages of 64) or 256 bytes (stages of 128), 16-byte chunks XOR-swizzled per
//    operand: weight rows are read 16 permuted rows at a time, token rows 16 consecutive rows at a time, and
//    each pattern has its own swizzle, so neither read conflicts;
//  * input rows: gathered through S from token-major hidden states [B, N, Din] (token t = b k + r reads
//    row S[r] of batch b), or packed [T, Din];
//  * output rows: packed [T, Dout], scattered to row S[r] of [B, N, Dout] (the FFN cache: context rows
//    untouched), or split into head-major Q / K / V [B, H, N, d] at row S[r] (16 consecutive features
//    never cross a head of d = 64 channels);
//  * the workgroup id is remapped so that the workgroups sharing one weight tile run on one XCD.
#include "common.hpp"

namespace safe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kKs = 64;                 // K elements per LDS stage: 128-byte rows of 8 chunks
constexpr int kJT = 128;                // output features per workgroup
constexpr int kTT = 128;                // tokens per workgroup
constexpr int kTileElems = 128 * kKs;   // one operand tile (128 rows) of one stage

// XOR swizzles of the 16-byte chunk index by row bits (128-byte rows; two rows per 256-byte bank window).
// Weight tiles are read 16 permuted rows at a time (rows 0-3, 16-19, 4-7, 20-23 of a 32-row block), token
// tiles 16 consecutive rows at a time; bits (1, 2, 4) spread the first pattern over all 16 bank groups and
// bits (1, 2, 3) the second, so neither read conflicts.
__device__ __forceinline__ int gswz_w(int row) { return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 4) & 1); }
__device__ __forceinline__ int gswz_x(int row) { return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1); }
__device__ __forceinline__ int goff_w(int row, int chunk) { return row * kKs + ((chunk ^ gswz_w(row)) << 3); }
__device__ __forceinline__ int goff_x(int row, int chunk) { return row * kKs + ((chunk ^ gswz_x(row)) << 3); }

// 256-byte rows (stages of 128 K elements, one row per bank window): weight reads (row bits 0, 1, 2, 4 vary
// across 16 lanes) and token reads (row bits 0-3) each need an injective 4-bit XOR of the 16 chunks.
__device__ __forceinline__ int gswz_w2(int r) { return ((r & 1) << 2) | (((r >> 1) & 1) << 3) | ((r >> 2) & 1) | (((r >> 4) & 1) << 1); }
__device__ __forceinline__ int gswz_x2(int r) { return ((r & 1) << 2) | (((r >> 1) & 1) << 3) | ((r >> 2) & 1) | (((r >> 3) & 1) << 1); }
__device__ __forceinline__ int goff_w2(int row, int chunk) { return row * 128 + ((chunk ^ gswz_w2(row)) << 3); }
__device__ __forceinline__ int goff_x2(int row, int chunk) { return row * 128 + ((chunk ^ gswz_x2(row)) << 3); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float gelu_tanh(float x) {
  return 0.5f * x * (1.f + tanhf(0.7978845608028654f * (x + 0.044715f * x * x * x)));
}

}  // namespace

struct RowsGemmArgs {
  const uint16_t* x;      // gathered: [B, N, Din]; packed: [T, Din]
  const int32_t* rows;    // [k], ascending row indices of S
  const uint16_t* w;      // [Dout, Din]
  const float* bias;      // [Dout] or null
  uint16_t* out;          // packed: [T, Dout]; scatter: [B, N, Dout]; heads: Q [B, H, N, d]
  uint16_t* out_k;        // heads: K
  uint16_t* out_v;        // heads: V
  int B, N, k, Din, Dout, H, d;
};

enum { kInPacked = 0, kInGather = 1 };
enum { kOutPacked = 0, kOutScatter = 1, kOutHeads = 2 };

// Epilogue of one lane: 16 consecutive features f0 .. f0+15 of token t (accumulators v), plus bias, GELU,
// packed to bf16 and stored as 32 contiguous bytes at the token's output row.
template <int OUT, bool GELU>
__device__ __forceinline__ void store16(const RowsGemmArgs& a, int t, int f0, const f32x16& acc) {
  const int T = a.B * a.k;
  if (t >= T) return;
  const int b = t / a.k, r = t - b * a.k;
  int row = 0;
  if (OUT != kOutPacked) {
    row = a.rows[r];
    if (row < 0 || row >= a.N) return;
  }
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = acc[i];
  if (a.bias != nullptr) {
    const float4* bp = reinterpret_cast<const float4*>(a.bias + f0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 bb = bp[q];
      v[4 * q + 0] += bb.x;
      v[4 * q + 1] += bb.y;
      v[4 * q + 2] += bb.z;
      v[4 * q + 3] += bb.w;
    }
  }
  if (GELU) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = gelu_tanh(v[i]);
  }
  uint4 lo, hi;
  lo.x = pack2(v[0], v[1]);
  lo.y = pack2(v[2], v[3]);
  lo.z = pack2(v[4], v[5]);
  lo.w = pack2(v[6], v[7]);
  hi.x = pack2(v[8], v[9]);
  hi.y = pack2(v[10], v[11]);
  hi.z = pack2(v[12], v[13]);
  hi.w = pack2(v[14], v[15]);
  uint16_t* dst;
  if (OUT == kOutPacked) {
    dst = a.out + static_cast<size_t>(t) * a.Dout + f0;
  } else if (OUT == kOutScatter) {
    dst = a.out + (static_cast<size_t>(b) * a.N + row) * a.Dout + f0;
  } else {
    const int D = a.H * a.d;
    const int which = f0 / D, hh = (f0 - which * D) / a.d, dd = f0 - which * D - hh * a.d;
    uint16_t* base = which == 0 ? a.out : which == 1 ? a.out_k : a.out_v;
    dst = base + ((static_cast<size_t>(b) * a.H + hh) * a.N + row) * a.d + dd;
  }
  reinterpret_cast<uint4*>(dst)[0] = lo;
  reinterpret_cast<uint4*>(dst)[1] = hi;
}

template <int IN, int OUT, bool GELU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_rows_gemm(RowsGemmArgs a) {
  constexpr int kK2 = 128;  // K elements per stage: 256-byte rows of 16 chunks
  __shared__ __attribute__((aligned(16))) uint16_t w_a[128 * kK2];
  __shared__ __attribute__((aligned(16))) uint16_t w_b[128 * kK2];
  __shared__ __attribute__((aligned(16))) uint16_t x_a[128 * kK2];
  __shared__ __attribute__((aligned(16))) uint16_t x_b[128 * kK2];

  const int T = a.B * a.k;
  const int nt = (T + kTT - 1) / kTT;
  const uint32_t G = static_cast<uint32_t>(nt) * static_cast<uint32_t>(a.Dout / kJT);
  const uint32_t lid = xcd_remap(blockIdx.x, G);
  const int jt = static_cast<int>(lid / nt), tt = static_cast<int>(lid - static_cast<uint32_t>(jt) * nt);
  const int j0 = jt * kJT, t0 = tt * kTT;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wj = wave & 1, wt = wave >> 1;
  const int qi = lane & 31;
  const int g = lane >> 5;
  const int kperm = 16 * ((qi >> 2) & 1) + 4 * (qi >> 3) + (qi & 3);

  // Copy sources of this lane: slot p = u * 256 + threadIdx.x of a 128-row tile holds row p / 8, chunk
  // (p % 8) ^ swizzle(row).  Token rows past T are clamped to the last token (loaded, never stored).
  const uint16_t* wsrc[8];
  const uint16_t* xsrc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int p = u * 256 + static_cast<int>(threadIdx.x);
    const int row = p >> 4;
    wsrc[u] = a.w + static_cast<size_t>(j0 + row) * a.Din + ((p & 15) ^ gswz_w2(row)) * 8;
    const int c = (p & 15) ^ gswz_x2(row);
    const int t = min(t0 + row, T - 1);
    size_t xr;
    if (IN == kInGather) {
      const int b = t / a.k, r = t - b * a.k;
      const int sr = a.rows[r];
      xr = static_cast<size_t>(b) * a.N + static_cast<size_t>((sr >= 0 && sr < a.N) ? sr : 0);
    } else {
      xr = static_cast<size_t>(t);
    }
    xsrc[u] = a.x + xr * a.Din + c * 8;
  }
  auto issue = [&](int s, uint16_t* wl, uint16_t* xl) {
    const int k0 = s * kK2;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int base = u * 256 + wave * 64;  // first slot of this wave instruction
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(wsrc[u] + k0),
                                       (__attribute__((address_space(3))) void*)(wl + base * 8), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(xsrc[u] + k0),
                                       (__attribute__((address_space(3))) void*)(xl + base * 8), 16, 0, 0);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[jb][tb][i] = 0.f;

  // operands of K step ks + 1 are read (into the other register set) before the matrix work of step ks
  auto compute = [&](const uint16_t* wl, const uint16_t* xl) {
    bf16x8 wa[2][2], xb[2][2];
    auto ld = [&](int ks, int slot) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) wa[slot][jb] = *reinterpret_cast<const bf16x8*>(wl + goff_w2(wj * 64 + jb * 32 + kperm, 2 * ks + g));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) xb[slot][tb] = *reinterpret_cast<const bf16x8*>(xl + goff_x2(wt * 64 + tb * 32 + qi, 2 * ks + g));
    };
    ld(0, 0);
#pragma unroll
    for (int ks = 0; ks < kK2 / 16; ++ks) {
      if (ks + 1 < kK2 / 16) ld(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[jb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[ks & 1][jb], xb[ks & 1][tb], acc[jb][tb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int ns = a.Din / kK2;
  issue(0, w_a, x_a);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int s = 0;
  for (; s + 1 < ns; s += 2) {
    issue(s + 1, w_b, x_b);
    __builtin_amdgcn_sched_barrier(0);  // keep the copies ahead of the compute
    compute(w_a, x_a);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (s + 2 < ns) issue(s + 2, w_a, x_a);
    __builtin_amdgcn_sched_barrier(0);
    compute(w_b, x_b);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (s < ns) compute(w_a, x_a);

  // ---- epilogue: lane (c + 32 g) holds token tb*32 + c, features jb*32 + 16 g + r (r = 0..15)
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
      store16<OUT, GELU>(a, t0 + wt * 64 + tb * 32 + qi, j0 + wj * 64 + jb * 32 + 16 * g, acc[jb][tb]);
}

// 256 features x 256 tokens per 8-wave workgroup (one per CU, two waves per SIMD): waves 2 (features) x 4
// (tokens), each 128 x 64 (4 x 2 blocks of 32 x 32), so every 16-element K step reads 6 KB of LDS per wave
// for 8 matrix instructions and the tile brings 128 flop per byte loaded (twice the 128 x 128 tile); K in
// stages of 64 through two 64 KB LDS buffers; one stage is about 2k cycles of matrix work per SIMD, long
// enough to cover the copy of the next.
template <int IN, int OUT, bool GELU>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_rows_gemm_big(RowsGemmArgs a) {
  constexpr int kJB = 256, kTB = 256, kElems = 256 * kKs;
  __shared__ __attribute__((aligned(16))) uint16_t w_a[kElems];
  __shared__ __attribute__((aligned(16))) uint16_t w_b[kElems];
  __shared__ __attribute__((aligned(16))) uint16_t x_a[kElems];
  __shared__ __attribute__((aligned(16))) uint16_t x_b[kElems];

  const int T = a.B * a.k;
  const int nt = (T + kTB - 1) / kTB;
  const uint32_t G = static_cast<uint32_t>(nt) * static_cast<uint32_t>(a.Dout / kJB);
  const uint32_t lid = xcd_remap(blockIdx.x, G);
  const int jt = static_cast<int>(lid / nt), tt = static_cast<int>(lid - static_cast<uint32_t>(jt) * nt);
  const int j0 = jt * kJB, t0 = tt * kTB;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wj = wave & 1, wt = wave >> 1;
  const int qi = lane & 31;
  const int g = lane >> 5;
  const int kperm = 16 * ((qi >> 2) & 1) + 4 * (qi >> 3) + (qi & 3);

  // copy sources: slot p = u * 512 + threadIdx.x of a 256-row tile holds row p / 8, chunk (p % 8) ^ swizzle(row)
  const uint16_t* wsrc[4];
  const uint16_t* xsrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = u * 512 + static_cast<int>(threadIdx.x);
    const int row = p >> 3;
    wsrc[u] = a.w + static_cast<size_t>(j0 + row) * a.Din + ((p & 7) ^ gswz_w(row)) * 8;
    const int c = (p & 7) ^ gswz_x(row);
    const int t = min(t0 + row, T - 1);
    size_t xr;
    if (IN == kInGather) {
      const int b = t / a.k, r = t - b * a.k;
      const int sr = a.rows[r];
      xr = static_cast<size_t>(b) * a.N + static_cast<size_t>((sr >= 0 && sr < a.N) ? sr : 0);
    } else {
      xr = static_cast<size_t>(t);
    }
    xsrc[u] = a.x + xr * a.Din + c * 8;
  }
  auto issue = [&](int s, uint16_t* wl, uint16_t* xl) {
    const int k0 = s * kKs;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int base = u * 512 + wave * 64;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(wsrc[u] + k0),
                                       (__attribute__((address_space(3))) void*)(wl + base * 8), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(xsrc[u] + k0),
                                       (__attribute__((address_space(3))) void*)(xl + base * 8), 16, 0, 0);
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[jb][tb][i] = 0.f;

  auto compute = [&](const uint16_t* wl, const uint16_t* xl) {
    bf16x8 wa[2][4], xb[2][2];
    auto ld = [&](int ks, int slot) {
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) wa[slot][jb] = *reinterpret_cast<const bf16x8*>(wl + goff_w(wj * 128 + jb * 32 + kperm, 2 * ks + g));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) xb[slot][tb] = *reinterpret_cast<const bf16x8*>(xl + goff_x(wt * 64 + tb * 32 + qi, 2 * ks + g));
    };
    ld(0, 0);
#pragma unroll
    for (int ks = 0; ks < kKs / 16; ++ks) {
      if (ks + 1 < kKs / 16) ld(ks + 1, (ks + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[jb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[ks & 1][jb], xb[ks & 1][tb], acc[jb][tb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int ns = a.Din / kKs;
  issue(0, w_a, x_a);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int s = 0;
  for (; s + 1 < ns; s += 2) {
    issue(s + 1, w_b, x_b);
    __builtin_amdgcn_sched_barrier(0);  // keep the copies ahead of the compute
    compute(w_a, x_a);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (s + 2 < ns) issue(s + 2, w_a, x_a);
    __builtin_amdgcn_sched_barrier(0);
    compute(w_b, x_b);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (s < ns) compute(w_a, x_a);

#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      store16<OUT, GELU>(a, t0 + wt * 64 + tb * 32 + qi, j0 + wj * 128 + jb * 32 + 16 * g, acc[jb][tb]);
}

template <int IN, int OUT, bool GELU>
static hipError_t launch_gemm(const RowsGemmArgs& a, hipStream_t s) {
  const int T = a.B * a.k;
  if (a.Dout % 256 == 0 && a.Dout >= 2048) {
    // wide products (the FFN's D -> F, QKV): 256 x 256 tiles still give at least 8 tiles across features
    const uint32_t grid = static_cast<uint32_t>((T + 255) / 256) * static_cast<uint32_t>(a.Dout / 256);
    k_rows_gemm_big<IN, OUT, GELU><<<grid, 512, 0, s>>>(a);
    return hipGetLastError();
  }
  const uint32_t grid = static_cast<uint32_t>((T + kTT - 1) / kTT) * static_cast<uint32_t>(a.Dout / kJT);
  k_rows_gemm<IN, OUT, GELU><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_rows_ffn(const uint16_t* x, const int32_t* rows, int k, int B, int N, int D, int F,
                           const uint16_t* w1, const float* b1, const uint16_t* w2, const float* b2, uint16_t* cache,
                           uint16_t* hidden, hipStream_t s) {
  if (B * k == 0) return hipSuccess;
  RowsGemmArgs a1{x, rows, w1, b1, hidden, nullptr, nullptr, B, N, k, D, F, 0, 0};
  hipError_t e = launch_gemm<kInGather, kOutPacked, true>(a1, s);
  if (e != hipSuccess) return e;
  RowsGemmArgs a2{hidden, rows, w2, b2, cache, nullptr, nullptr, B, N, k, F, D, 0, 0};
  return launch_gemm<kInPacked, kOutScatter, false>(a2, s);
}

hipError_t launch_rows_qkv(const uint16_t* x, const int32_t* rows, int k, int B, int N, int H, int d,
                           const uint16_t* wqkv, const float* bqkv, uint16_t* q, uint16_t* kc, uint16_t* vc,
                           hipStream_t s) {
  if (B * k == 0) return hipSuccess;
  RowsGemmArgs a{x, rows, wqkv, bqkv, q, kc, vc, B, N, k, H * d, 3 * H * d, H, d};
  return launch_gemm<kInGather, kOutHeads, false>(a, s);
}

}  // namespace safe

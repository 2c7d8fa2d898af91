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
//  * wide products (D -> F, QKV): 256 (or 192) features x 256 tokens per 8-wave workgroup (one per CU, two
//    waves per SIMD), each wave 128 x 64 (4 x 2 blocks of 32 x 32): 128 flop per byte loaded, 6 KB of LDS
//    reads per 8 matrix instructions; 192 where 256-feature tiles would leave many CUs idle; K streams
//    through a ring of four 32-element LDS stages filled by direct global -> LDS copies three stages ahead
//    (the schedule is described at the kernel);
//  * narrow products (F -> D): 128 x 128 per 4-wave workgroup (enough workgroups to fill the GPU), K in
//    double-buffered stages of 128 (two distinct LDS objects per operand, one 4-wave workgroup per CU with
//    128 KB of LDS), the copies pinned ahead of the stage's matrix work, the operands of K step ks + 1 read
//    while the matrix instructions of step ks run;
//  * LDS rows of 64 bytes (ring stages of 32) or 256 bytes (stages of 128), 16-byte chunks XOR-swizzled per
//    operand: weight rows are read 16 permuted rows at a time, token rows 16 consecutive rows at a time, and
//    each pattern has its own swizzle, so neither read conflicts;
//  * input rows: gathered through S from token-major hidden states [B, N, Din] (token t = b k + r reads
//    row S[r] of batch b), or packed [T, Din];
//  * output rows: packed [T, Dout], scattered to row S[r] of [B, N, Dout] (the FFN cache: context rows
//    untouched), or split into head-major Q / K / V [B, H, N, d] at row S[r] (16 consecutive features
//    never cross a head of d = 64 channels);
//  * the workgroup id is remapped so that consecutive tiles run on one XCD: on the wide products the tiles
//    of one weight tile, on the narrow product (K four times longer, 1.5 MB per operand tile) a block of
//    about five token tiles by six feature tiles, so that its L2 holds the operands of that block only.
#include <type_traits>

#include "common.hpp"

namespace safe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kJT = 128;                // output features per workgroup of the narrow product
constexpr int kTT = 128;                // tokens per workgroup of the narrow product

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

// tanh-approximated GELU, 0.5 x (1 + tanh(u)) with u = sqrt(2/pi) (x + 0.044715 x^3), evaluated through the
// identity 1 + tanh(u) = 2 / (1 + e^(-2u)): x / (1 + 2^(x (a + b x^2))) with a = -2 sqrt(2/pi) log2(e),
// b = 0.044715 a.  One exp2 and one reciprocal per value (the hardware's, each within about one ulp), so the
// relative error stays near 1e-6, far below the bf16 rounding of the output; for very negative x the
// exponential overflows to +inf and the value goes to -0, for large x it goes to 0 and the value to x.  About a
// fifth of the vector instructions of a library tanh, which made the epilogue of the D -> F product cost as
// much as 5 us of its 57.
__device__ __forceinline__ float gelu_tanh(float x) {
  constexpr float a = -2.f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float b = 0.044715f * a;
  const float e = __builtin_amdgcn_exp2f(x * __builtin_fmaf(x * x, b, a));
  return x * __builtin_amdgcn_rcpf(1.f + e);
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

// Bias of the 16 consecutive features f0 .. f0 + 15 (zero without a bias).  The epilogues load the bias of
// all their feature blocks before the first store: stores count in the same vector-memory counter as loads,
// so a bias load issued after a store would wait for that store too, and the eight blocks of a wave would
// chain eight load-and-store round trips (about 5k shader cycles per workgroup).
__device__ __forceinline__ void load_bias16(const RowsGemmArgs& a, int f0, float4 (&bb)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    bb[q] = a.bias != nullptr ? reinterpret_cast<const float4*>(a.bias + f0)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// Epilogue of one lane: 16 consecutive features f0 .. f0+15 of token t (accumulators v), plus bias, GELU,
// packed to bf16 and stored as 32 contiguous bytes at the token's output row.
template <int OUT, bool GELU>
__device__ __forceinline__ void store16(const RowsGemmArgs& a, int t, int f0, const f32x16& acc, const float4 (&bb)[4]) {
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
  for (int q = 0; q < 4; ++q) {
    v[4 * q + 0] = acc[4 * q + 0] + bb[q].x;
    v[4 * q + 1] = acc[4 * q + 1] + bb[q].y;
    v[4 * q + 2] = acc[4 * q + 2] + bb[q].z;
    v[4 * q + 3] = acc[4 * q + 3] + bb[q].w;
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

// Launch-order index -> (token tile, feature tile) of the narrow product: token tiles in groups of kGroupT, and
// inside a group the token tile varies fastest, so the consecutive indices that run on one XCD cover a block of
// a few token tiles by a few feature tiles (5 x 6 of the 20 x 12 tiles at the 1024^2 shapes) and its L2 holds the
// input rows and weight rows of that block only.
constexpr int kGroupT = 5;
__device__ __forceinline__ void grouped_tile(uint32_t lid, int nt, int nj, int& tt, int& jt) {
  const int per = kGroupT * nj;
  const int grp = static_cast<int>(lid) / per;
  const int within = static_cast<int>(lid) - grp * per;
  const int gt = min(kGroupT, nt - grp * kGroupT);
  tt = grp * kGroupT + within % gt;
  jt = within / gt;
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
  int tt, jt;
  grouped_tile(lid, nt, a.Dout / kJT, tt, jt);
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
  float4 bias[2][4];
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) load_bias16(a, j0 + wj * 64 + jb * 32 + 16 * g, bias[jb]);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
      store16<OUT, GELU>(a, t0 + wt * 64 + tb * 32 + qi, j0 + wj * 64 + jb * 32 + 16 * g, acc[jb][tb], bias[jb]);
}

// 64-byte LDS rows (stages of 32 K elements, four rows per 256-byte bank window).  Weight reads take 16
// permuted rows at a time (rows 0-3, 16-19, 4-7, 20-23 of a 32-row block, or 8-11, 24-27, 12-15, 28-31),
// token reads 16 consecutive rows; rows that share a bank-window offset (row % 4) differ in row bits (2, 4) in
// the first pattern and (2, 3) in the second, so XOR-ing the 16-byte chunk index with those two bits puts the
// 16 reads of either pattern in distinct bank groups.
__device__ __forceinline__ int rswz_w(int r) { return ((r >> 2) & 1) | (((r >> 4) & 1) << 1); }
__device__ __forceinline__ int rswz_x(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int roff_w(int row, int c) { return row * 32 + ((c ^ rswz_w(row)) << 3); }
__device__ __forceinline__ int roff_x(int row, int c) { return row * 32 + ((c ^ rswz_x(row)) << 3); }

// Wait until at most N of this wave's vector-memory operations are outstanding (expcnt / lgkmcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// JB features (256 or 192) x 256 tokens per 8-wave workgroup (one per CU, two waves per SIMD): waves 2
// (features) x 4 (tokens), each JB / 2 x 64 (JB / 64 x 2 blocks of 32 x 32), so at JB = 256 every 16-element
// K step reads 6 KB of LDS per wave for 8 matrix instructions and the tile brings 128 flop per byte loaded.
// JB = 192 serves products whose 256-feature tiles would leave a large part of the GPU idle (QKV at the
// 1024^2 shapes: 180 tiles of 256 on 256 CUs, 240 of 192).
//
// K streams through a ring of four LDS stages of 32 elements (four distinct objects per operand, so the
// compiler sees that a copy in flight into one does not alias the reads of another).  The copies of a stage
// are issued three stages before it is multiplied (96 K elements ahead, against 64 for two buffers of 64
// elements), and the launch waits for half as many bytes before its first matrix instruction.  Stage s runs in
// two halves of 2 JB / 64 matrix instructions per wave (8 at JB = 256, 6 at 192):
//   * first half: the first K step (operands read during the previous stage), with the reads of the second K
//     step issued after the first half of its instructions;
//   * then this wave's reads of the buffer are waited for and its copies of stage s + 1 (vector-memory count,
//     not a drain of every copy in flight), two instructions of the second half are queued, and the
//     workgroup meets at a bare s_barrier (a fence-carrying __syncthreads would wait for every copy);
//   * second half: the reads of the first K step of stage s + 1 and the copies of stage s + 4 into the buffer
//     just released, interleaved with the remaining instructions.
// Measured on the gathered D -> F product at the 1024^2 shapes (2458 x 1536 -> 6144): 71k against 93k
// shader cycles per workgroup for the two-buffer form with stages of 64, bitwise the same outputs.
template <int IN, int OUT, bool GELU, int JB = 256>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void k_rows_gemm_big(RowsGemmArgs a) {
  static_assert(JB == 256 || JB == 192, "feature tile");
  constexpr int kJW = JB / 64;                 // 32-feature blocks per wave
  constexpr int kWS = JB * 4, kXS = 256 * 4;   // 16-byte slots of one stage's weight / token tile
  constexpr int kWU = (kWS + 511) / 512;       // weight copies per thread and stage (the last partial at 192)
  constexpr bool kWFull = kWU * 512 == kWS;
  constexpr int kCopies = kWU - (kWFull ? 0 : 1) + kXS / 512;  // copies per stage that every wave issues
  __shared__ __attribute__((aligned(16))) uint16_t w0[JB * 32], w1[JB * 32], w2[JB * 32], w3[JB * 32];
  __shared__ __attribute__((aligned(16))) uint16_t x0[256 * 32], x1[256 * 32], x2[256 * 32], x3[256 * 32];

  const int T = a.B * a.k;
  const int nt = (T + 255) / 256;
  const uint32_t G = static_cast<uint32_t>(nt) * static_cast<uint32_t>(a.Dout / JB);
  const uint32_t lid = xcd_remap(blockIdx.x, G);
  const int jt = static_cast<int>(lid / nt), tt = static_cast<int>(lid - static_cast<uint32_t>(jt) * nt);
  const int j0 = jt * JB, t0 = tt * 256;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wj = wave & 1, wt = wave >> 1;
  const int qi = lane & 31;
  const int g = lane >> 5;
  const int kperm = 16 * ((qi >> 2) & 1) + 4 * (qi >> 3) + (qi & 3);

  // copy sources: slot p = u * 512 + threadIdx.x of a stage's tile holds row p / 4, chunk (p % 4) ^ swizzle;
  // token rows past T are clamped to the last token (loaded, never stored)
  const uint16_t* wsrc[kWU];
  const uint16_t* xsrc[kXS / 512];
#pragma unroll
  for (int u = 0; u < kWU; ++u) {
    const int p = min(u * 512 + static_cast<int>(threadIdx.x), kWS - 1);
    const int row = p >> 2;
    wsrc[u] = a.w + static_cast<size_t>(j0 + row) * a.Din + ((p & 3) ^ rswz_w(row)) * 8;
  }
#pragma unroll
  for (int u = 0; u < kXS / 512; ++u) {
    const int p = u * 512 + static_cast<int>(threadIdx.x);
    const int row = p >> 2;
    const int t = min(t0 + row, T - 1);
    size_t xr;
    if (IN == kInGather) {
      const int b = t / a.k, r = t - b * a.k;
      const int sr = a.rows[r];
      xr = static_cast<size_t>(b) * a.N + static_cast<size_t>((sr >= 0 && sr < a.N) ? sr : 0);
    } else {
      xr = static_cast<size_t>(t);
    }
    xsrc[u] = a.x + xr * a.Din + ((p & 3) ^ rswz_x(row)) * 8;
  }
  const bool w_tail = (kWU - 1) * 512 + wave * 64 < kWS;  // this wave copies a slot of the last weight row group
  auto issue = [&](int s, uint16_t* wl, uint16_t* xl) {
    const int k0 = s * 32;
#pragma unroll
    for (int u = 0; u < kWU; ++u) {
      const int base = u * 512 + wave * 64;
      if (u < kWU - 1 || kWFull || w_tail)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(wsrc[u] + k0),
                                         (__attribute__((address_space(3))) void*)(wl + base * 8), 16, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kXS / 512; ++u) {
      const int base = u * 512 + wave * 64;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(xsrc[u] + k0),
                                       (__attribute__((address_space(3))) void*)(xl + base * 8), 16, 0, 0);
    }
  };

  f32x16 acc[kJW][2];
#pragma unroll
  for (int jb = 0; jb < kJW; ++jb)
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[jb][tb][i] = 0.f;

  // operands of the first (wa0, xb0) and second (wa1, xb1) 16-element K step of a stage
  bf16x8 wa0[kJW], xb0[2], wa1[kJW], xb1[2];
  auto read0 = [&](const uint16_t* wl, const uint16_t* xl) {
#pragma unroll
    for (int jb = 0; jb < kJW; ++jb) wa0[jb] = *reinterpret_cast<const bf16x8*>(wl + roff_w(wj * (JB / 2) + jb * 32 + kperm, g));
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) xb0[tb] = *reinterpret_cast<const bf16x8*>(xl + roff_x(wt * 64 + tb * 32 + qi, g));
  };
  auto read1 = [&](const uint16_t* wl, const uint16_t* xl) {
#pragma unroll
    for (int jb = 0; jb < kJW; ++jb) wa1[jb] = *reinterpret_cast<const bf16x8*>(wl + roff_w(wj * (JB / 2) + jb * 32 + kperm, 2 + g));
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) xb1[tb] = *reinterpret_cast<const bf16x8*>(xl + roff_x(wt * 64 + tb * 32 + qi, 2 + g));
  };
  auto mma0 = [&](int j_lo, int j_hi) {
#pragma unroll
    for (int jb = 0; jb < kJW; ++jb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        if (jb >= j_lo && jb < j_hi) acc[jb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa0[jb], xb0[tb], acc[jb][tb], 0, 0, 0);
  };
  auto mma1 = [&](int j_lo, int j_hi) {
#pragma unroll
    for (int jb = 0; jb < kJW; ++jb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        if (jb >= j_lo && jb < j_hi) acc[jb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa1[jb], xb1[tb], acc[jb][tb], 0, 0, 0);
  };
  auto barrier = [] { asm volatile("s_barrier" ::: "memory"); };
  using C2 = std::integral_constant<int, 2>;
  using C1 = std::integral_constant<int, 1>;
  using C0 = std::integral_constant<int, 0>;

  // stage s (buffer wc, xc); the next stage's buffer is wn, xn; AF stages of copies may stay in flight after
  // those of stage s + 1; copy: issue the copies of stage s4 = s + 4 into the buffer of s
  auto step = [&](auto af, bool copy, uint16_t* wc, uint16_t* xc, const uint16_t* wn, const uint16_t* xn, int s4) {
    constexpr int AF = decltype(af)::value;
    mma0(0, kJW / 2);
    __builtin_amdgcn_sched_barrier(0);
    read1(wc, xc);
    __builtin_amdgcn_sched_barrier(0);
    mma0(kJW / 2, kJW);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of the buffer have returned
    wait_vmcnt<AF * kCopies>();          // and its copies of stage s + 1 have landed
    __builtin_amdgcn_sched_barrier(0);
    mma1(0, 1);  // two matrix instructions queued while the waves meet at the barrier
    __builtin_amdgcn_sched_barrier(0);
    barrier();
    if (copy) issue(s4, wc, xc);
    read0(wn, xn);
    mma1(1, kJW);
    // the reads of the next stage first (its first matrix instructions wait for them), in threes between
    // matrix instructions, then one copy after each of the following ones
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
    for (int i = 0; i < 2 * kJW - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const int ns = a.Din / 32;  // Din is a multiple of 128: ns is a multiple of 4, at least 4
  issue(0, w0, x0);
  issue(1, w1, x1);
  issue(2, w2, x2);
  wait_vmcnt<2 * kCopies>();
  barrier();
  issue(3, w3, x3);
  read0(w0, x0);
  int s = 0;
  for (; s + 4 < ns; s += 4) {
    step(C2{}, true, w0, x0, w1, x1, s + 4);
    step(C2{}, true, w1, x1, w2, x2, s + 5);
    step(C2{}, true, w2, x2, w3, x3, s + 6);
    step(C2{}, true, w3, x3, w0, x0, s + 7);
  }
  // the last four stages issue no copies; stage ns - 4 waits for ns - 3 with ns - 2 and ns - 1 in flight, ...
  step(C2{}, false, w0, x0, w1, x1, 0);
  step(C1{}, false, w1, x1, w2, x2, 0);
  step(C0{}, false, w2, x2, w3, x3, 0);
  read1(w3, x3);
  mma0(0, kJW);
  mma1(0, kJW);

  // ---- epilogue: lane (c + 32 g) holds token tb*32 + c, features jb*32 + 16 g + r (r = 0..15)
  float4 bias[kJW][4];
#pragma unroll
  for (int jb = 0; jb < kJW; ++jb) load_bias16(a, j0 + wj * (JB / 2) + jb * 32 + 16 * g, bias[jb]);
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int jb = 0; jb < kJW; ++jb)
      store16<OUT, GELU>(a, t0 + wt * 64 + tb * 32 + qi, j0 + wj * (JB / 2) + jb * 32 + 16 * g, acc[jb][tb], bias[jb]);
}

template <int IN, int OUT, bool GELU>
static hipError_t launch_gemm(const RowsGemmArgs& a, hipStream_t s) {
  const int T = a.B * a.k;
  if (a.Dout >= 2048 && (a.Dout % 256 == 0 || a.Dout % 192 == 0)) {
    // wide products (the FFN's D -> F, QKV): 256 or 192 features x 256 tokens, whichever finishes its
    // rounds of one workgroup per CU sooner (a workgroup's time taken as its feature count, 5% more per
    // feature at 192 for the smaller flop per byte): QKV at the 1024^2 shapes takes 192 (one round of 240
    // tiles against one of 180), the FFN's D -> F 256 (240 tiles against two rounds of 320)
    const int tt = (T + 255) / 256;
    auto cost = [&](int jb) {
      if (a.Dout % jb != 0) return 1e30;
      const int rounds = (tt * (a.Dout / jb) + 255) / 256;
      return static_cast<double>(rounds) * jb * (jb == 192 ? 1.05 : 1.0);
    };
    if (cost(192) < cost(256)) {
      k_rows_gemm_big<IN, OUT, GELU, 192><<<static_cast<uint32_t>(tt * (a.Dout / 192)), 512, 0, s>>>(a);
    } else {
      k_rows_gemm_big<IN, OUT, GELU, 256><<<static_cast<uint32_t>(tt * (a.Dout / 256)), 512, 0, s>>>(a);
    }
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

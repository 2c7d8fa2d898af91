// PCSP (SAFE-DiT technical summary, Methodology 2): per image token, the attention mass the joint
// softmax row puts on the text content slots, summed over heads; then the exact top-|S| partition.
#include "common.hpp"

namespace safe {

// ---------------------------------------------------------------------------------------------
// Aggregation.  One 16-lane group owns one (head, token) row at a time: it reads the row's valid
// text logits with float4 loads, reduces max / sum-exp / content mass with xor shuffles inside the
// group, and leaves one fp32 contribution in LDS.  A workgroup covers kRows tokens x all heads;
// contributions are then summed over heads in index order, so the result is deterministic.
// HBM-bound: each valid logit is read once.
constexpr int kPcspThreads = 256;
constexpr int kPcspGroups = kPcspThreads / 16;
constexpr int kPcspRows = 4;

__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 16));
  return v;
}
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, 16);
  return v;
}

template <bool VEC>
__global__ __launch_bounds__(kPcspThreads) void k_pcsp_accumulate(const float* __restrict__ x,
                                                                  const float* __restrict__ lse_img, int H, int N,
                                                                  int T, int Tv, int c0, int c1,
                                                                  float* __restrict__ scores, int accumulate,
                                                                  int H_alloc) {
  extern __shared__ float part[];  // [kPcspRows][H]
  const int g = threadIdx.x >> 4;
  const int lane = threadIdx.x & 15;
  const int i0 = blockIdx.x * kPcspRows;
  const int pairs = kPcspRows * H;
  for (int p = g; p < pairs; p += kPcspGroups) {
    const int r = p / H;
    const int h = p - r * H;
    const int i = i0 + r;
    float contrib = 0.f;
    if (i < N) {
      const float* row = x + (static_cast<size_t>(h) * N + i) * T;
      // pass 1: log-sum-exp over the valid slots (lane-local online form, then group combine)
      float m = -INFINITY, sum = 0.f;
      if (VEC) {
        for (int t = lane * 4; t < Tv; t += 64) {
          const float4 v = *reinterpret_cast<const float4*>(row + t);
          const float a0 = v.x, a1 = (t + 1 < Tv) ? v.y : -INFINITY, a2 = (t + 2 < Tv) ? v.z : -INFINITY,
                      a3 = (t + 3 < Tv) ? v.w : -INFINITY;
          const float mn = fmaxf(fmaxf(m, a0), fmaxf(fmaxf(a1, a2), a3));
          if (mn != -INFINITY) {
            sum = sum * expf(m - mn) + expf(a0 - mn) + expf(a1 - mn) + expf(a2 - mn) + expf(a3 - mn);
            m = mn;
          }
        }
      } else {
        for (int t = lane; t < Tv; t += 16) {
          const float a = row[t];
          const float mn = fmaxf(m, a);
          if (mn != -INFINITY) {
            sum = sum * expf(m - mn) + expf(a - mn);
            m = mn;
          }
        }
      }
      const float gm = group16_max(m);
      const float s = group16_sum(m == -INFINITY ? 0.f : sum * expf(m - gm));
      float lse = (s > 0.f) ? gm + logf(s) : -INFINITY;
      if (lse_img != nullptr) {
        const float li = lse_img[static_cast<size_t>(h) * N + i];
        const float hi = fmaxf(li, lse), lo = fminf(li, lse);
        lse = (hi == -INFINITY) ? -INFINITY : hi + log1pf(expf(lo - hi));
      }
      // pass 2: mass on the content slots [c0, c1)
      float c = 0.f;
      for (int t = c0 + lane; t < c1; t += 16) c += expf(row[t] - lse);
      contrib = group16_sum(c);
    }
    if (lane == 0) part[r * H_alloc + h] = contrib;
  }
  __syncthreads();
  if (threadIdx.x < kPcspRows) {
    const int i = i0 + threadIdx.x;
    if (i < N) {
      float a = 0.f;
      for (int h = 0; h < H; ++h) a += part[threadIdx.x * H_alloc + h];
      scores[i] = accumulate ? scores[i] + a : a;
    }
  }
}

hipError_t launch_pcsp_accumulate(const float* x, const float* lse_img, int H, int N, int T, int Tv, int c0, int c1,
                                  float* scores, int accumulate, hipStream_t s) {
  const int blocks = (N + kPcspRows - 1) / kPcspRows;
  const size_t lds = sizeof(float) * kPcspRows * H;
  const bool vec = (T % 4 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0);
  if (vec)
    k_pcsp_accumulate<true><<<blocks, kPcspThreads, lds, s>>>(x, lse_img, H, N, T, Tv, c0, c1, scores, accumulate, H);
  else
    k_pcsp_accumulate<false><<<blocks, kPcspThreads, lds, s>>>(x, lse_img, H, N, T, Tv, c0, c1, scores, accumulate, H);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Partition: one workgroup of 1024 threads.  Scores map to order-preserving uint32 keys (NaN -> 0,
// below every number; -0 -> +0).  An MSB-first 8-bit radix select finds the k-th largest key K*;
// S = {key > K*} plus the lowest-index (k - #greater) entries equal to K*.  Thread t owns the
// contiguous index chunk [t*E, (t+1)*E), so two block-wide exclusive scans give each index its
// rank among the equal keys and its slot in S (or C) in ascending index order.
constexpr int kPartThreads = 1024;
constexpr int kPartWaves = kPartThreads / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) == 0u) b = 0u;  // -0 ranks with +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Block-wide exclusive scan of one uint32 per thread; also returns the total.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wave_tot[w] = inc;
  __syncthreads();
  if (w == 0) {
    uint32_t t = lane < kPartWaves ? wave_tot[lane] : 0u;
    uint32_t ti = t;
#pragma unroll
    for (int o = 1; o < kPartWaves; o <<= 1) {
      const uint32_t y = __shfl_up(ti, o, 64);
      if (lane >= o) ti += y;
    }
    if (lane < kPartWaves) wave_tot[kPartWaves + lane] = ti - t;  // exclusive wave offsets
    if (lane == kPartWaves - 1) wave_tot[2 * kPartWaves] = ti;
  }
  __syncthreads();
  const uint32_t r = wave_tot[kPartWaves + w] + inc - v;
  *total = wave_tot[2 * kPartWaves];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPartThreads) void k_partition(const float* __restrict__ scores, int N, int k,
                                                            int32_t* __restrict__ S, int32_t* __restrict__ C,
                                                            uint8_t* __restrict__ is_sens, float* __restrict__ s01) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[2 * kPartWaves + 1];
  __shared__ uint32_t sel_digit, sel_above;
  __shared__ float red_lo[kPartWaves], red_hi[kPartWaves];
  const int tid = threadIdx.x;
  const int E = (N + kPartThreads - 1) / kPartThreads;
  const int beg = min(N, tid * E), end = min(N, beg + E);

  // ---- radix select of the k-th largest key (skipped when k == 0)
  uint32_t prefix = 0, pmask = 0, remaining = static_cast<uint32_t>(k);
  if (k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int j = tid; j < 256; j += kPartThreads) hist[j] = 0;
      __syncthreads();
      for (int i = beg; i < end; ++i) {
        const uint32_t key = order_key(scores[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t above = 0;
        int dsel = 0;
        for (int dgt = 255; dgt >= 0; --dgt) {
          if (above + hist[dgt] >= remaining) { dsel = dgt; break; }
          above += hist[dgt];
        }
        sel_digit = static_cast<uint32_t>(dsel);
        sel_above = above;
      }
      __syncthreads();
      remaining -= sel_above;
      prefix |= sel_digit << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
  }
  const uint32_t kstar = prefix;
  const uint32_t need = (k > 0) ? remaining : 0u;  // how many keys equal to K* are taken

  // ---- rank among equal keys, in index order
  uint32_t neq = 0;
  if (k > 0)
    for (int i = beg; i < end; ++i) neq += (order_key(scores[i]) == kstar) ? 1u : 0u;
  uint32_t tot;
  const uint32_t eq_base = block_exclusive_scan(neq, wave_tot, &tot);

  // ---- selection flags and their count per chunk
  uint32_t nsel = 0;
  {
    uint32_t er = eq_base;
    for (int i = beg; i < end; ++i) {
      const uint32_t key = order_key(scores[i]);
      bool sel = false;
      if (k > 0) {
        if (key > kstar) sel = true;
        else if (key == kstar) { sel = er < need; ++er; }
      }
      nsel += sel ? 1u : 0u;
    }
  }
  const uint32_t s_base = block_exclusive_scan(nsel, wave_tot, &tot);

  // ---- min / max over non-NaN scores for s01
  float lo = INFINITY, hi = -INFINITY;
  if (s01 != nullptr) {
    for (int i = beg; i < end; ++i) { const float a = scores[i]; lo = fminf(lo, a); hi = fmaxf(hi, a); }
    for (int o = 32; o >= 1; o >>= 1) { lo = fminf(lo, __shfl_xor(lo, o, 64)); hi = fmaxf(hi, __shfl_xor(hi, o, 64)); }
    if ((tid & 63) == 0) { red_lo[tid >> 6] = lo; red_hi[tid >> 6] = hi; }
    __syncthreads();
    lo = red_lo[0]; hi = red_hi[0];
    for (int w = 1; w < kPartWaves; ++w) { lo = fminf(lo, red_lo[w]); hi = fmaxf(hi, red_hi[w]); }
  }
  const bool all_nan = !(lo <= hi);

  // ---- write S, C, is_sens, s01
  uint32_t er = eq_base, sp = s_base;
  for (int i = beg; i < end; ++i) {
    const float a = scores[i];
    const uint32_t key = order_key(a);
    bool sel = false;
    if (k > 0) {
      if (key > kstar) sel = true;
      else if (key == kstar) { sel = er < need; ++er; }
    }
    if (sel) S[sp++] = i;
    else C[static_cast<uint32_t>(i) - sp] = i;
    is_sens[i] = sel ? 1 : 0;
    if (s01 != nullptr) {
      float v;
      if (a != a || all_nan) v = NAN;
      else if (hi > lo) v = (a - lo) / (hi - lo);
      else v = 0.f;
      s01[i] = v;
    }
  }
}

hipError_t launch_pcsp_partition(const float* scores, int N, int k, int32_t* S, int32_t* C, uint8_t* is_sens,
                                 float* s01, hipStream_t s) {
  k_partition<<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  return hipGetLastError();
}

}  // namespace safe

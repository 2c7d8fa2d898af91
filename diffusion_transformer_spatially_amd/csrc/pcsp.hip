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

// All-reduce inside each 16-lane row of the wave through DPP lane permutations (no LDS round trip):
// swap neighbours, swap pairs, mirror within each half-row of 8, mirror the row.  Every lane ends with
// the same value (each step combines two equal-shaped partial results, and + and max commute).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
__device__ __forceinline__ float group16_max(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
  return fmaxf(v, dpp_mov<kDppMirror>(v));
}
__device__ __forceinline__ float group16_sum(float v) {
  v += dpp_mov<kDppXor1>(v);
  v += dpp_mov<kDppXor2>(v);
  v += dpp_mov<kDppHalfMirror>(v);
  return v + dpp_mov<kDppMirror>(v);
}

// SEL: the content slots are the valid slots t with sel[t] != 0 (the AesMask affinity) instead of the
// range [c0, c1) (the PCSP score).
template <bool VEC, bool SEL>
__global__ __launch_bounds__(kPcspThreads) void k_pcsp_accumulate(const float* __restrict__ x,
                                                                  const float* __restrict__ lse_img, int H, int N,
                                                                  int T, int Tv, int c0, int c1,
                                                                  const uint8_t* __restrict__ sel,
                                                                  float* __restrict__ scores, int accumulate,
                                                                  int H_alloc) {
  extern __shared__ float part[];  // [kPcspRows][H]
  const int g = threadIdx.x >> 4;
  const int lane = threadIdx.x & 15;
  // token blocks that share lse_img cache lines (32 tokens per 128-byte line) run on one XCD and its L2
  const int i0 = static_cast<int>(xcd_remap(blockIdx.x, gridDim.x)) * kPcspRows;
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
      // pass 2: mass on the content slots
      float c = 0.f;
      if (SEL) {
        for (int t = lane; t < Tv; t += 16)
          if (sel[t] != 0) c += expf(row[t] - lse);
      } else {
        for (int t = c0 + lane; t < c1; t += 16) c += expf(row[t] - lse);
      }
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

// Batched form for Tv <= 64*TV4 with float4 rows: each 16-lane group issues the loads of JB (head,
// token) rows at once, with their image log-sum-exp values, and then reduces them from registers, so
// HBM latency is paid once per batch instead of once per row.  The logits are read once: nontemporal loads
// when the launch streams more than the MALL holds (NT).  The loads are unconditional (addresses
// of padded slots and of pairs past the end are clamped to valid memory and their values discarded
// afterwards), so no load sits under divergent control flow and the waits stay exact.
template <int TV4, bool SEL, bool NT>
__global__ __launch_bounds__(kPcspThreads) void k_pcsp_accumulate_b(const float* __restrict__ x,
                                                                   const float* __restrict__ lse_img, int H, int N,
                                                                   int T, int Tv, int c0, int c1,
                                                                   const uint8_t* __restrict__ sel,
                                                                   float* __restrict__ scores, int accumulate) {
  constexpr int JB = 6;  // 16 groups x 6 rows: the 4 tokens x 24 heads of a workgroup in one round of loads
  extern __shared__ float part[];  // [kPcspRows][H]
  const int g = threadIdx.x >> 4;
  const int lane = threadIdx.x & 15;
  // SEL: a lane's slots are the same in every row, so its selection bytes (4 per float4 of slots; the
  // host passes sel 4-byte aligned with T a multiple of 4) are loaded once
  uint32_t selw[TV4];
#pragma unroll
  for (int c = 0; c < TV4; ++c)
    selw[c] = (SEL && lane * 4 + 64 * c < Tv) ? reinterpret_cast<const uint32_t*>(sel)[lane + 16 * c] : 0u;
  // token blocks that share lse_img cache lines (32 tokens per 128-byte line) run on one XCD and its L2
  const int i0 = static_cast<int>(xcd_remap(blockIdx.x, gridDim.x)) * kPcspRows;
  const int pairs = kPcspRows * H;
  for (int pb = g; pb < pairs; pb += kPcspGroups * JB) {
    float4 v[JB][TV4];
    float li[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int p = pb + kPcspGroups * jj;
      const int r = p / H, h = p - r * H, i = i0 + r;
      const bool ok = p < pairs && i < N;
      const size_t ri = ok ? static_cast<size_t>(h) * N + i : 0;
      const float* row = x + ri * T;
#pragma unroll
      for (int c = 0; c < TV4; ++c) {
        const int t = lane * 4 + 64 * c;
        v[jj][c] = load_s<NT>(reinterpret_cast<const float4*>(row + (t < Tv ? t : 0)));
      }
      li[jj] = lse_img != nullptr ? lse_img[ri] : 0.f;
    }
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int p = pb + kPcspGroups * jj;
      const int r = p / H, h = p - r * H, i = i0 + r;
      const bool ok = p < pairs && i < N;
      float e[TV4 * 4];
#pragma unroll
      for (int c = 0; c < TV4; ++c) {
        const int t = lane * 4 + 64 * c;
        e[4 * c + 0] = (t + 0 < Tv) ? v[jj][c].x : -INFINITY;
        e[4 * c + 1] = (t + 1 < Tv) ? v[jj][c].y : -INFINITY;
        e[4 * c + 2] = (t + 2 < Tv) ? v[jj][c].z : -INFINITY;
        e[4 * c + 3] = (t + 3 < Tv) ? v[jj][c].w : -INFINITY;
      }
      // One exponential per logit: with gm the row's text max (0 when there is no valid text slot),
      //   mass = sum_content e^(x-gm) / (sum_valid e^(x-gm) + e^(lse_img-gm)),
      // which equals sum_content exp(x - LSE) for LSE = log(exp(lse_img) + sum_valid exp(x)).
      float m = -INFINITY;
#pragma unroll
      for (int q = 0; q < TV4 * 4; ++q) m = fmaxf(m, e[q]);
      const float gm = group16_max(m);
      const float gmu = gm == -INFINITY ? 0.f : gm;
      const float gml = gmu * kLog2e;
      float sum = 0.f, cs = 0.f;
#pragma unroll
      for (int c = 0; c < TV4; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = lane * 4 + 64 * c + q;
          const float ev = __builtin_amdgcn_exp2f(fmaf(e[4 * c + q], kLog2e, -gml));
          sum += ev;
          const bool content = SEL ? ((selw[c] >> (8 * q)) & 0xffu) != 0u : (t >= c0 && t < c1);
          cs += content ? ev : 0.f;
        }
      sum = group16_sum(sum);
      cs = group16_sum(cs);
      float den = sum;
      if (lse_img != nullptr) den += __builtin_amdgcn_exp2f((li[jj] - gmu) * kLog2e);
      const float contrib = den > 0.f ? cs / den : 0.f;
      if (ok && lane == 0) part[r * H + h] = contrib;
    }
  }
  __syncthreads();
  if (threadIdx.x < kPcspRows) {
    const int i = i0 + threadIdx.x;
    if (i < N) {
      float acc = 0.f;
      for (int h = 0; h < H; ++h) acc += part[threadIdx.x * H + h];
      scores[i] = accumulate ? scores[i] + acc : acc;
    }
  }
}

template <bool SEL>
static void pcsp_launch(const float* x, const float* lse_img, int H, int N, int T, int Tv, int c0, int c1,
                        const uint8_t* sel, float* scores, int accumulate, hipStream_t s) {
  const int blocks = (N + kPcspRows - 1) / kPcspRows;
  const size_t lds = sizeof(float) * kPcspRows * H;
  const bool vec = (T % 4 == 0) && (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                   (!SEL || reinterpret_cast<uintptr_t>(sel) % 4 == 0);
  if (vec && Tv <= 256) {
    const int tv4 = Tv <= 64 ? 1 : Tv <= 128 ? 2 : Tv <= 192 ? 3 : 4;
    const bool nt = 4.0 * H * N * Tv > kStreamBytes;
#define PCSP_B(TV, NTV) k_pcsp_accumulate_b<TV, SEL, NTV><<<blocks, kPcspThreads, lds, s>>>(x, lse_img, H, N, T, Tv, c0, c1, sel, scores, accumulate)
    switch (tv4 * 2 + (nt ? 1 : 0)) {
      case 2: PCSP_B(1, false); break;
      case 3: PCSP_B(1, true); break;
      case 4: PCSP_B(2, false); break;
      case 5: PCSP_B(2, true); break;
      case 6: PCSP_B(3, false); break;
      case 7: PCSP_B(3, true); break;
      case 8: PCSP_B(4, false); break;
      default: PCSP_B(4, true); break;
    }
#undef PCSP_B
  } else if (T % 4 == 0 && reinterpret_cast<uintptr_t>(x) % 16 == 0)
    k_pcsp_accumulate<true, SEL><<<blocks, kPcspThreads, lds, s>>>(x, lse_img, H, N, T, Tv, c0, c1, sel, scores, accumulate, H);
  else
    k_pcsp_accumulate<false, SEL><<<blocks, kPcspThreads, lds, s>>>(x, lse_img, H, N, T, Tv, c0, c1, sel, scores, accumulate, H);
}

hipError_t launch_pcsp_accumulate(const float* x, const float* lse_img, int H, int N, int T, int Tv, int c0, int c1,
                                  float* scores, int accumulate, hipStream_t s) {
  pcsp_launch<false>(x, lse_img, H, N, T, Tv, c0, c1, nullptr, scores, accumulate, s);
  return hipGetLastError();
}

hipError_t launch_affinity_accumulate(const float* x, const float* lse_img, int H, int N, int T, int Tv,
                                      const uint8_t* sel, float* scores, int accumulate, hipStream_t s) {
  pcsp_launch<true>(x, lse_img, H, N, T, Tv, 0, 0, sel, scores, accumulate, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Partition: one workgroup of 1024 threads.  Scores map to order-preserving uint32 keys (NaN -> 0,
// below every number; -0 -> +0).  An MSB-first 8-bit radix select finds the k-th largest key K*
// (coalesced strided passes, LDS histogram, the digit found by one wave with a prefix scan over the
// 256 bins); S = {key > K*} plus the lowest-index (k - #greater) entries equal to K*.  The output is
// then written in rounds of 1024 consecutive indices: ballot/popcount block scans give each index its
// rank among the equal keys and its slot in S (or C), in ascending index order.
constexpr int kPartThreads = 1024;
constexpr int kPartWaves = kPartThreads / 64;

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7fffffffu) == 0u) b = 0u;  // -0 ranks with +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Whole-wave all-reduce without LDS: the four DPP steps of each 16-lane row (as group16_* above), then
// the row-pair and half-wave exchanges of v_permlane16_swap / v_permlane32_swap, combining what each lane
// holds with what its partner row holds.  Every lane ends with the result.  (A __shfl_xor ladder is six
// dependent ds_bpermute round trips per value.)
template <typename Op>
__device__ __forceinline__ uint32_t wave_allreduce(uint32_t v, Op op) {
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), kDppXor1, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), kDppXor2, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), kDppHalfMirror, 0xf, 0xf, false)));
  v = op(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), kDppMirror, 0xf, 0xf, false)));
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) { return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a & b; }); }
__device__ __forceinline__ uint32_t wave_or(uint32_t v) { return wave_allreduce(v, [](uint32_t a, uint32_t b) { return a | b; }); }
__device__ __forceinline__ float wave_fmin(float v) {
  return __uint_as_float(wave_allreduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_fmax(float v) {
  return __uint_as_float(wave_allreduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

// Inclusive sum over lanes 0 .. L of the wave without LDS: row shifts by 1, 2, 4 and 8 (lanes past the row
// start add 0) give each 16-lane row its own scan; then the last lane of rows 0 and 2 is broadcast into rows 1
// and 3, and the last lane of row 1 (by then the total of rows 0 and 1) into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr + 1, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr + 2, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr + 4, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowShr + 8, 0xf, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowBcast15, 0xa, 0xf, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), kRowBcast31, 0xc, 0xf, false));
  return v;
}

// Exclusive block prefix count of a per-thread flag and the block total.  wcnt: [kPartWaves] LDS slots
// used by this call only (alternate two sets between consecutive calls so one barrier suffices).
__device__ __forceinline__ uint32_t block_flag_scan(bool flag, uint32_t* wcnt, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned long long b = __ballot(flag ? 1 : 0);
  const uint32_t wexcl = static_cast<uint32_t>(__popcll(b & ((1ull << lane) - 1ull)));
  if (lane == 0) wcnt[w] = static_cast<uint32_t>(__popcll(b));
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int j = 0; j < kPartWaves; ++j) {
    const uint32_t c = wcnt[j];
    before += (j < w) ? c : 0u;
    tot += c;
  }
  *total = tot;
  return before + wexcl;
}

__global__ __launch_bounds__(kPartThreads) void k_partition(const float* __restrict__ scores, int N, int k,
                                                            int32_t* __restrict__ S, int32_t* __restrict__ C,
                                                            uint8_t* __restrict__ is_sens, float* __restrict__ s01) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wcnt[4][kPartWaves];
  __shared__ uint32_t sel_digit, sel_above;
  __shared__ float red_lo[kPartWaves], red_hi[kPartWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // ---- min / max over non-NaN scores for s01
  float lo = INFINITY, hi = -INFINITY;
  if (s01 != nullptr) {
    for (int i = tid; i < N; i += kPartThreads) { const float a = scores[i]; lo = fminf(lo, a); hi = fmaxf(hi, a); }
    lo = wave_fmin(lo);
    hi = wave_fmax(hi);
    if (lane == 0) { red_lo[w] = lo; red_hi[w] = hi; }
    __syncthreads();
    lo = red_lo[0]; hi = red_hi[0];
    for (int j = 1; j < kPartWaves; ++j) { lo = fminf(lo, red_lo[j]); hi = fmaxf(hi, red_hi[j]); }
  }
  const bool all_nan = !(lo <= hi);

  // ---- radix select of the k-th largest key (skipped when k == 0)
  uint32_t prefix = 0, pmask = 0, remaining = static_cast<uint32_t>(k);
  if (k > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < N; i += kPartThreads) {
        const uint32_t key = order_key(scores[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (w == 0) {
        // lane l owns bins 255-4l .. 252-4l (descending); find where the running count from the top
        // first reaches `remaining`
        uint32_t c[4], loc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; loc += c[j]; }
        const uint32_t inc = wave_inclusive_sum(loc);
        const uint32_t exc = inc - loc;
        if (exc < remaining && remaining <= inc) {
          uint32_t acc = exc;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (acc + c[j] >= remaining) { sel_digit = 255u - 4u * lane - j; sel_above = acc; break; }
            acc += c[j];
          }
        }
      }
      __syncthreads();
      remaining -= sel_above;
      prefix |= sel_digit << shift;
      pmask |= 255u << shift;
    }
  }
  const uint32_t kstar = prefix;
  const uint32_t need = (k > 0) ? remaining : 0u;  // how many keys equal to K* are taken

  // ---- output in rounds of 1024 consecutive indices
  uint32_t run_eq = 0, run_s = 0;
  int set = 0;
  for (int base = 0; base < N; base += kPartThreads) {
    const int i = base + tid;
    const bool valid = i < N;
    const float a = valid ? scores[i] : 0.f;
    const uint32_t key = order_key(a);
    const bool eq = valid && k > 0 && key == kstar;
    const bool gt = valid && k > 0 && key > kstar;
    uint32_t eq_tot, s_tot;
    const uint32_t eq_rank = run_eq + block_flag_scan(eq, wcnt[set], &eq_tot);
    const bool sel = gt || (eq && eq_rank < need);
    const uint32_t s_pos = run_s + block_flag_scan(sel, wcnt[set + 1], &s_tot);
    set ^= 2;
    if (valid) {
      if (sel) S[s_pos] = i;
      else C[static_cast<uint32_t>(i) - s_pos] = i;
      is_sens[i] = sel ? 1 : 0;
      if (s01 != nullptr) {
        float v;
        if (a != a || all_nan) v = NAN;
        else if (hi > lo) v = (a - lo) / (hi - lo);
        else v = 0.f;
        s01[i] = v;
      }
    }
    run_eq += eq_tot;
    run_s += s_tot;
  }
}

// Register-resident form for N <= 1024 * IPT.  Wave w owns the CH = 64 * IPT consecutive indices
// [w * CH, (w + 1) * CH); lane l holds item j at index w * CH + 64 j + l, so every load is coalesced
// and, for each j, the wave's 64 lanes cover 64 consecutive indices.  The keys are loaded once and stay
// in registers for every pass.  The radix select runs on the offsets key - kmin of the valid keys (block
// min / max; subtracting kmin keeps the order and the ties), from the highest bit of kmax - kmin down, in
// the fewest passes of at most 9 bits: the leading bits that every key shares cost no pass, and the first
// digit cuts the keys' actual range into up to 512 bins.  (On the keys themselves, the first digit of
// scores spanning a few binades is mostly exponent bits, which piles the keys onto two or three bins, and
// LDS atomics of a wave on one address run one lane at a time: that pass took six times as long as the
// next.)  Wave reductions use DPP and the lane-swap instructions, not LDS.  The output walks each wave's items in
// index order with ballots (rank among the wave's earlier lanes by mbcnt, running totals in scalars); one
// block scan of the per-wave totals gives each wave its base.  Slots past N hold key 0 (the NaN key): they
// are left out of the counts, and in the output they are the highest indices, so they never reach S
// (k <= N); the stores skip them.
__device__ __forceinline__ float key_value(uint32_t key) {
  if (key == 0u) return NAN;
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Number of set bits of a wave ballot in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(unsigned long long b) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u));
}

template <int IPT, int NT = kPartThreads, int DB = 9>
__global__ __launch_bounds__(NT) void k_partition_reg(const float* __restrict__ scores, int N, int k,
                                                                int32_t* __restrict__ S, int32_t* __restrict__ C,
                                                                uint8_t* __restrict__ is_sens,
                                                                float* __restrict__ s01) {
  // pass p counts into hist[p & 1] (digits of up to DB bits); the other is cleared meanwhile
  constexpr int kBins = 1 << DB, kBinsPerLane = kBins / 64;
  static_assert(kBinsPerLane % 4 == 0, "whole 16-byte reads of the bins");
  __shared__ __attribute__((aligned(16))) uint32_t hist[2][kBins];
  constexpr int kW = NT / 64;  // waves
  __shared__ uint32_t wred[4][kW];  // per-wave min / max
  __shared__ uint32_t wcnt[2][kW];  // per-wave output counts
  __shared__ uint32_t sel_digit, sel_above, sel_count;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int base = w * 64 * IPT + lane;  // index of item j: base + 64 j

  uint32_t key[IPT];
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  float lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = base + 64 * j;
    const float a = i < N ? scores[i] : NAN;
    key[j] = order_key(a);
    kmin = min(kmin, i < N ? key[j] : 0xffffffffu);
    kmax = max(kmax, i < N ? key[j] : 0u);
    lo = fminf(lo, a);
    hi = fmaxf(hi, a);
  }
  kmin = wave_allreduce(kmin, [](uint32_t x, uint32_t y) { return min(x, y); });
  kmax = wave_allreduce(kmax, [](uint32_t x, uint32_t y) { return max(x, y); });
  lo = wave_fmin(lo);
  hi = wave_fmax(hi);
  if (lane == 0) {
    wred[0][w] = kmin;
    wred[1][w] = kmax;
    wred[2][w] = __float_as_uint(lo);
    wred[3][w] = __float_as_uint(hi);
  }
  for (int t = tid; t < 2 * kBins; t += NT) hist[t / kBins][t % kBins] = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kW; ++j) {
    kmin = min(kmin, wred[0][j]);
    kmax = max(kmax, wred[1][j]);
    lo = fminf(lo, __uint_as_float(wred[2][j]));
    hi = fmaxf(hi, __uint_as_float(wred[3][j]));
  }
  const bool all_nan = !(lo <= hi);
  // offsets from here on; slots past N get 0 (never above K*, and the last in index order among equal ones)
#pragma unroll
  for (int j = 0; j < IPT; ++j) key[j] = base + 64 * j < N ? key[j] - kmin : 0u;

  // ---- radix select of the k-th largest offset key - kmin of the valid keys, over the fewest passes of at
  // most DB bits that cover kmax - kmin, of near-equal widths (25 bits: 9 + 8 + 8; with 8-bit digits, four
  // passes took 1k clocks more at N = 4096)
  uint32_t prefix = 0, remaining = static_cast<uint32_t>(k);
  uint32_t total_eq = static_cast<uint32_t>(N);  // valid keys equal to K* (all of them when all are equal)
  if (k > 0) {
    const uint32_t span = kmax - kmin;  // every valid offset lies in [0, span]
    const int nbits = span != 0u ? 32 - __clz(span) : 0;
    const int npass = (nbits + DB - 1) / DB;
    uint32_t pmask = nbits == 32 ? 0u : ~((1u << nbits) - 1u);  // bits already decided (zero in every offset)
    int hb = nbits - 1;
    for (int pass = 0; pass < npass; ++pass) {
      const int width = (hb + npass - pass) / (npass - pass);  // ceil(bits left / passes left) <= DB
      const int lob = hb + 1 - width;
      const uint32_t dmask = (1u << width) - 1u;
      uint32_t* const h = hist[pass & 1];
#pragma unroll
      for (int j = 0; j < IPT; ++j)
        if (base + 64 * j < N && (key[j] & pmask) == prefix) atomicAdd(&h[(key[j] >> lob) & dmask], 1u);
      __syncthreads();
      if (w != 0)  // the next pass's bins (last read two passes ago), while wave 0 scans this pass's
        for (int t = tid - 64; t < kBins; t += NT - 64) hist[(pass + 1) & 1][t] = 0;
      if (w == 0) {
        // lane l owns the kBinsPerLane bins below kBins - kBinsPerLane * l (descending; bins past dmask stay
        // 0); find where the running count from the top first reaches `remaining`
        const uint4* hp = reinterpret_cast<const uint4*>(h + kBins - kBinsPerLane * (lane + 1));
        uint32_t c[kBinsPerLane];
#pragma unroll
        for (int u = 0; u < kBinsPerLane / 4; ++u) {
          const uint4 v = hp[u];
          const int q = kBinsPerLane - 1 - 4 * u;  // c[q] = the highest bin of this read
          c[q] = v.x;
          c[q - 1] = v.y;
          c[q - 2] = v.z;
          c[q - 3] = v.w;
        }
        uint32_t loc = 0;
#pragma unroll
        for (int q = 0; q < kBinsPerLane; ++q) loc += c[q];
        const uint32_t inc = wave_inclusive_sum(loc);
        const uint32_t exc = inc - loc;
        if (exc < remaining && remaining <= inc) {
          uint32_t acc = exc;
#pragma unroll
          for (int q = 0; q < kBinsPerLane; ++q) {
            if (acc + c[q] >= remaining) {
              sel_digit = kBins - 1u - kBinsPerLane * lane - q;
              sel_above = acc;
              sel_count = c[q];
              break;
            }
            acc += c[q];
          }
        }
      }
      __syncthreads();
      remaining -= sel_above;
      prefix |= sel_digit << lob;
      pmask |= dmask << lob;
      hb = lob - 1;
      total_eq = sel_count;  // after the last pass: the keys whose offset is K*
    }
  }
  const uint32_t kstar = prefix;  // the k-th largest offset
  const uint32_t need = (k > 0) ? remaining : 0u;  // how many keys equal to K* are taken

  // ---- output.  When every key equal to K* is taken (always without ties at the boundary), S is the set of
  // offsets >= K*; otherwise the equal keys are taken in index order, which needs each wave's count of them
  // first.  Slots past N are never selected (and come last among equal keys).
  const bool all_eq_taken = need == total_eq;
  auto selected = [&](int j, unsigned long long be, uint32_t run) -> bool {
    if (k <= 0) return false;
    if (all_eq_taken) return base + 64 * j < N && key[j] >= kstar;
    const bool eq = (be >> lane) & 1ull;
    return key[j] > kstar || (eq && run + lanes_below(be) < need);
  };
  // Pass 1 (ties only): each wave's count of keys equal to K*; block scan -> the wave's base rank.
  uint32_t eq_run = 0;
  if (k > 0 && !all_eq_taken) {
    uint32_t w_eq = 0;
#pragma unroll
    for (int j = 0; j < IPT; ++j) w_eq += static_cast<uint32_t>(__popcll(__ballot(key[j] == kstar)));
    if (lane == 0) wcnt[0][w] = w_eq;
    __syncthreads();
    for (int j = 0; j < w; ++j) eq_run += wcnt[0][j];
  }
  // Pass 2: each wave's count of selected keys; block scan -> the wave's base slot in S.
  uint32_t w_sel = 0;
  {
    uint32_t run = eq_run;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const unsigned long long be = __ballot(k > 0 && key[j] == kstar);
      w_sel += static_cast<uint32_t>(__popcll(__ballot(selected(j, be, run))));
      run += static_cast<uint32_t>(__popcll(be));
    }
  }
  if (lane == 0) wcnt[1][w] = w_sel;
  __syncthreads();
  uint32_t s_run = 0;
  for (int j = 0; j < w; ++j) s_run += wcnt[1][j];
  // Pass 3: write S, C, is_sens and s01 in index order.  The bound goes through an empty asm so that
  // the compiler does not keep the IPT lane masks of the load loop alive until here (they spill).
  int n_end = N;
  asm volatile("" : "+s"(n_end));
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    const int i = base + 64 * j;
    const unsigned long long be = __ballot(k > 0 && key[j] == kstar);
    const bool sel = selected(j, be, eq_run);
    const unsigned long long bs = __ballot(sel);
    const uint32_t s_pos = s_run + lanes_below(bs);
    if (i < n_end) {
      if (sel) S[s_pos] = i;
      else C[static_cast<uint32_t>(i) - s_pos] = i;
      is_sens[i] = sel ? 1 : 0;
      if (s01 != nullptr) {
        const float a = key_value(key[j] + kmin);
        float v;
        if (a != a || all_nan) v = NAN;
        else if (hi > lo) v = (a - lo) / (hi - lo);
        else v = 0.f;
        s01[i] = v;
      }
    }
    eq_run += static_cast<uint32_t>(__popcll(be));
    s_run += static_cast<uint32_t>(__popcll(bs));
  }
}

hipError_t launch_pcsp_partition(const float* scores, int N, int k, int32_t* S, int32_t* C, uint8_t* is_sens,
                                 float* s01, hipStream_t s) {
  const int ipt = (N + kPartThreads - 1) / kPartThreads;
  if (ipt <= 1) k_partition_reg<1><<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  else if (ipt <= 2) k_partition_reg<2><<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  else if (ipt <= 4) k_partition_reg<4><<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  else if (ipt <= 8) k_partition_reg<8><<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  else if (ipt <= 16) k_partition_reg<16><<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  else if (ipt <= 32) k_partition_reg<32><<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  else if (ipt <= 40) k_partition_reg<40><<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  else k_partition<<<1, kPartThreads, 0, s>>>(scores, N, k, S, C, is_sens, s01);
  return hipGetLastError();
}

}  // namespace safe

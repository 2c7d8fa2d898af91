// Exact mask-elision check (SAFE-DiT technical summary, Methodology 1): is every row of an additive
// mask one finite constant over the keys that row attends to?  Every entry is compared with the row's
// first entry with IEEE == (no arithmetic, no tolerance), streaming the rows with aligned 16-byte
// loads.  HBM-bound.  Without a c_out request (k_mask_scan) each workgroup covers several rows with
// all their loads in flight and reduces its verdict once, and a failed row lets the other workgroups
// stop early (the verdict only ever moves from 1 to 0, so it stays deterministic).  With c_out
// (k_mask_check) one workgroup per row also reports the row's constant.
#include "common.hpp"

#include <algorithm>

namespace safe {

constexpr int kMaskThreads = 256;

__device__ __forceinline__ float mask_value(const uint8_t* p, int dtype) {
  if (dtype == SAFE_DTYPE_BOOL) return *p ? 0.f : -INFINITY;
  return *reinterpret_cast<const float*>(p);
}

__global__ void k_flag_init(int32_t* flag) { *flag = 1; }

__global__ __launch_bounds__(kMaskThreads) void k_mask_check(const uint8_t* __restrict__ mask, int dtype, int esize,
                                                             int cols, int ncheck, int zero_required, int32_t* flag,
                                                             float* __restrict__ c_out, int early) {
  const uint32_t row = blockIdx.x;
  if (early && __atomic_load_n(flag, __ATOMIC_RELAXED) == 0) return;
  const uint8_t* base = mask + static_cast<size_t>(row) * cols * esize;
  const float first = mask_value(base, dtype);
  bool ok = isfinite(first) && !(zero_required && first != 0.f);
  // Aligned 16-byte blocks covering [base, base + ncheck * esize).
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(base);
  const uintptr_t lo = b0 & ~static_cast<uintptr_t>(15);
  const uintptr_t hi = b0 + static_cast<uintptr_t>(ncheck) * esize;
  const size_t nblk = (hi - lo + 15) / 16;
  for (size_t blk = threadIdx.x; ok && blk < nblk; blk += kMaskThreads) {
    const uintptr_t a = lo + blk * 16;
    const uint4 v = *reinterpret_cast<const uint4*>(a);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if (dtype == SAFE_DTYPE_BOOL) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uintptr_t ea = a + j;
        if (ea < b0 || ea >= hi) continue;
        const float m = ((w[j >> 2] >> (8 * (j & 3))) & 0xffu) ? 0.f : -INFINITY;
        ok = ok && (m == first);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uintptr_t ea = a + 4 * j;
        if (ea < b0 || ea >= hi) continue;
        ok = ok && (__uint_as_float(w[j]) == first);
      }
    }
  }
  const int all_ok = __syncthreads_and(ok ? 1 : 0);
  if (threadIdx.x == 0) {
    if (!all_ok) __atomic_store_n(flag, 0, __ATOMIC_RELAXED);
    if (c_out != nullptr) c_out[row] = all_ok ? first : NAN;
  }
}


// A byte of w is zero iff the corresponding byte of the result has its top bit set.
__device__ __forceinline__ uint32_t zero_bytes(uint32_t w) { return (w - 0x01010101u) & ~w & 0x80808080u; }

// Word of byte-validity for the 4 bytes at address wa against the span [b0, hi): 0xff per valid byte.
__device__ __forceinline__ uint32_t valid_bytes(uintptr_t wa, uintptr_t b0, uintptr_t hi) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m |= (wa + j >= b0 && wa + j < hi) ? (0xffu << (8 * j)) : 0u;
  return m;
}

// Is the 16-byte block at a (16-aligned) consistent with a row constant?  Bool rows can only be
// constant and finite if their first byte is nonzero (attend, value 0), so the block must hold no
// zero byte inside the span; fp32 rows compare every word inside the span with the first value.
__device__ __forceinline__ bool block_ok(uint4 v, uintptr_t a, uintptr_t b0, uintptr_t hi, int dtype, float first) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const bool interior = a >= b0 && a + 16 <= hi;
  bool ok = true;
  if (dtype == SAFE_DTYPE_BOOL) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t vb = interior ? 0xffffffffu : valid_bytes(a + 4 * j, b0, hi);
      ok = ok && zero_bytes(w[j] | ~vb) == 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uintptr_t ea = a + 4 * j;
      const bool in = interior || (ea >= b0 && ea < hi);
      ok = ok && (!in || __uint_as_float(w[j]) == first);
    }
  }
  return ok;
}

constexpr int kScanRows = 4;

__global__ __launch_bounds__(kMaskThreads) void k_mask_scan(const uint8_t* __restrict__ mask, int dtype, int esize,
                                                            int cols, int nrows, int ncheck, int zero_required,
                                                            int32_t* flag) {
  bool ok = true;
  for (int r0 = blockIdx.x * kScanRows; r0 < nrows; r0 += gridDim.x * kScanRows) {
    if (__atomic_load_n(flag, __ATOMIC_RELAXED) == 0) return;
#pragma unroll
    for (int rr = 0; rr < kScanRows; ++rr) {
      const int row = r0 + rr;
      if (row >= nrows) break;
      const uint8_t* base = mask + static_cast<size_t>(row) * cols * esize;
      const float first = mask_value(base, dtype);
      ok = ok && isfinite(first) && !(zero_required && first != 0.f);
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(base);
      const uintptr_t lo = b0 & ~static_cast<uintptr_t>(15);
      const uintptr_t hi = b0 + static_cast<uintptr_t>(ncheck) * esize;
      const uint32_t nblk = static_cast<uint32_t>((hi - lo + 15) / 16);
      for (uint32_t blk = threadIdx.x; blk < nblk; blk += kMaskThreads) {
        const uintptr_t a = lo + static_cast<uintptr_t>(blk) * 16;
        ok = block_ok(*reinterpret_cast<const uint4*>(a), a, b0, hi, dtype, first) && ok;
      }
    }
  }
  const int all_ok = __syncthreads_and(ok ? 1 : 0);
  if (threadIdx.x == 0 && !all_ok) __atomic_store_n(flag, 0, __ATOMIC_RELAXED);
}

hipError_t launch_mask_check(const void* mask, int mask_dtype, int mB, int mH, int N, int cols, int T,
                             const int32_t* tv, int B, int32_t* flag, float* c_out, hipStream_t s) {
  // Valid text span per slice: the batch entries using slice mb are {mb} when mB == B, else all of
  // them (nested prefixes, so the longest one decides).  One launch per batch slice.
  int tmax_all = 0;
  for (int b = 0; b < B; ++b) tmax_all = tv[b] > tmax_all ? tv[b] : tmax_all;
  const int esize = mask_dtype == SAFE_DTYPE_BOOL ? 1 : 4;
  const bool full = cols == N + T;
  auto ncheck_of = [&](int tspan) { return full ? N + tspan : N; };
  auto zero_of = [&](int tspan) { return (!full && tspan > 0) ? 1 : 0; };
  k_flag_init<<<1, 1, 0, s>>>(flag);
  const int early = c_out == nullptr ? 1 : 0;
  if (c_out == nullptr) {
    const size_t slice_bytes = static_cast<size_t>(mH) * N * cols * esize;
    const int nrows = mH * N;
    const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>((nrows + kScanRows - 1) / kScanRows, 2048));
    for (int b = 0; b < mB; ++b) {
      const int tspan = mB == 1 ? tmax_all : tv[b];
      k_mask_scan<<<grid, kMaskThreads, 0, s>>>(static_cast<const uint8_t*>(mask) + b * slice_bytes, mask_dtype,
                                                esize, cols, nrows, ncheck_of(tspan), zero_of(tspan), flag);
    }
  } else if (mB == 1) {
    const int nc = ncheck_of(tmax_all), z = zero_of(tmax_all);
    k_mask_check<<<static_cast<uint32_t>(mH) * N, kMaskThreads, 0, s>>>(
        static_cast<const uint8_t*>(mask), mask_dtype, esize, cols, nc, z, flag, c_out, early);
  } else {
    const size_t slice_bytes = static_cast<size_t>(mH) * N * cols * esize;
    for (int b = 0; b < mB; ++b) {
      const int nc = ncheck_of(tv[b]), z = zero_of(tv[b]);
      k_mask_check<<<static_cast<uint32_t>(mH) * N, kMaskThreads, 0, s>>>(
          static_cast<const uint8_t*>(mask) + b * slice_bytes, mask_dtype, esize, cols, nc, z, flag,
          c_out ? c_out + static_cast<size_t>(b) * mH * N : nullptr, early);
    }
  }
  return hipGetLastError();
}

}  // namespace safe

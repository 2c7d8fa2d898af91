// Exact mask-elision check (SAFE-DiT technical summary, Methodology 1): is every row of an additive
// mask one finite constant over the keys that row attends to?  Every entry is compared with the row's
// first entry with IEEE == (no arithmetic, no tolerance), streaming the rows with aligned 16-byte
// loads.  HBM-bound.  Without a c_out request (k_mask_scan) each workgroup covers several rows with
// all their loads in flight and reduces its verdict once, and a failed row lets the other workgroups
// stop early (the verdict only ever moves from 1 to 0, so it stays deterministic).  With c_out
// (k_mask_check) one workgroup per row also reports the row's constant.
#include "common.hpp"
#include "mask_span.hpp"

#include <algorithm>

namespace safe {

constexpr int kMaskThreads = 256;

__device__ __forceinline__ float mask_value(const uint8_t* p, int dtype) {
  if (dtype == SAFE_DTYPE_BOOL) return *p ? 0.f : -INFINITY;
  return *reinterpret_cast<const float*>(p);
}

__global__ void k_flag_init(int32_t* flag) { *flag = 1; }

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

// One mask entry as an additive value.
__device__ __forceinline__ float entry_value(const uint8_t* p, int dtype) { return mask_value(p, dtype); }

template <bool NT>
__global__ __launch_bounds__(kMaskThreads) void k_mask_check(const uint8_t* __restrict__ mask, uintptr_t buf_lo,
                                                             uintptr_t buf_hi, int dtype, int esize, int cols,
                                                             int ncheck, int zero_required, int32_t* flag,
                                                             float* __restrict__ c_out, int early) {
  const uint32_t row = blockIdx.x;
  if (early && __atomic_load_n(flag, __ATOMIC_RELAXED) == 0) return;
  const uint8_t* base = mask + static_cast<size_t>(row) * cols * esize;
  const float first = mask_value(base, dtype);
  bool ok = isfinite(first) && !(zero_required && first != 0.f);
  // Whole aligned 16-byte blocks of [base, base + ncheck * esize) with unconditional loads, then the entries
  // outside them (buffer ends only) one at a time.
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(base);
  const uintptr_t hi = b0 + static_cast<uintptr_t>(ncheck) * esize;
  const RowBlocks rb = row_blocks(b0, hi, buf_lo, buf_hi);
  const uint8_t* wp = base + (rb.wlo - b0);
  for (uint32_t blk = threadIdx.x; ok && blk < rb.nw; blk += kMaskThreads) {
    const uintptr_t a = rb.wlo + static_cast<uintptr_t>(blk) * 16;
    ok = block_ok(load_s<NT>(reinterpret_cast<const uint4*>(wp) + blk), a, b0, hi, dtype, first);
  }
  uintptr_t e[4];
  row_edges(b0, hi, rb, &e[0], &e[1], &e[2], &e[3]);
  for (int r = 0; r < 2; ++r)
    for (uintptr_t x = e[2 * r] + static_cast<uintptr_t>(threadIdx.x) * esize; ok && x < e[2 * r + 1];
         x += static_cast<uintptr_t>(kMaskThreads) * esize)
      ok = entry_value(base + (x - b0), dtype) == first;
  const int all_ok = __syncthreads_and(ok ? 1 : 0);
  if (threadIdx.x == 0) {
    if (!all_ok) __atomic_store_n(flag, 0, __ATOMIC_RELAXED);
    if (c_out != nullptr) c_out[row] = all_ok ? first : NAN;
  }
}


constexpr int kScanRows = 4;

// U: 16-byte loads per row and thread issued before any is tested (2 for rows of 512 blocks or more; a row
// of 4096 bytes is one block per thread, and a second load would only repeat the last block).
template <bool NT, int U>
__global__ __launch_bounds__(kMaskThreads) void k_mask_scan(const uint8_t* __restrict__ mask, uintptr_t buf_lo,
                                                            uintptr_t buf_hi, int dtype, int esize, int cols,
                                                            int nrows, int ncheck, int zero_required, int32_t* flag) {
  bool ok = true;
  for (int r0 = blockIdx.x * kScanRows; r0 < nrows; r0 += gridDim.x * kScanRows) {
    if (__atomic_load_n(flag, __ATOMIC_RELAXED) == 0) return;
    // the workgroup's rows (a row past the end repeats the last row, whose verdict it then cannot change)
    const uint8_t* base[kScanRows];
    float first[kScanRows];
    RowBlocks rb[kScanRows];
    uint32_t nmax = 0;
#pragma unroll
    for (int rr = 0; rr < kScanRows; ++rr) {
      const int row = min(r0 + rr, nrows - 1);
      base[rr] = mask + static_cast<size_t>(row) * cols * esize;
      first[rr] = mask_value(base[rr], dtype);
      ok = ok && isfinite(first[rr]) && !(zero_required && first[rr] != 0.f);
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(base[rr]);
      rb[rr] = row_blocks(b0, b0 + static_cast<uintptr_t>(ncheck) * esize, buf_lo, buf_hi);
      nmax = max(nmax, rb[rr].nw);
    }
    // whole blocks: kScanRows x U loads in flight per thread; a block index past a row's last block
    // reloads that row's last block (never out of its row, result ignored)
    for (uint32_t j0 = threadIdx.x; j0 < nmax; j0 += kMaskThreads * U) {
      uint4 v[kScanRows][U];
#pragma unroll
      for (int rr = 0; rr < kScanRows; ++rr) {
        const uint4* wp = reinterpret_cast<const uint4*>(base[rr] + (rb[rr].wlo - reinterpret_cast<uintptr_t>(base[rr])));
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t blk = j0 + u * kMaskThreads;
          v[rr][u] = rb[rr].nw > 0 ? load_s<NT>(wp + min(blk, rb[rr].nw - 1)) : make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll
      for (int rr = 0; rr < kScanRows; ++rr) {
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(base[rr]);
        const uintptr_t hi = b0 + static_cast<uintptr_t>(ncheck) * esize;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t blk = j0 + u * kMaskThreads;
          const uintptr_t a = rb[rr].wlo + static_cast<uintptr_t>(blk) * 16;
          ok = (blk >= rb[rr].nw || block_ok(v[rr][u], a, b0, hi, dtype, first[rr])) && ok;
        }
      }
    }
    // entries outside the whole blocks (the ends of a buffer whose base or length is not a multiple of 16)
#pragma unroll
    for (int rr = 0; rr < kScanRows; ++rr) {
      const uintptr_t b0 = reinterpret_cast<uintptr_t>(base[rr]);
      const uintptr_t hi = b0 + static_cast<uintptr_t>(ncheck) * esize;
      uintptr_t e[4];
      row_edges(b0, hi, rb[rr], &e[0], &e[1], &e[2], &e[3]);
      for (int q = 0; q < 2; ++q)
        for (uintptr_t x = e[2 * q] + static_cast<uintptr_t>(threadIdx.x) * esize; x < e[2 * q + 1];
             x += static_cast<uintptr_t>(kMaskThreads) * esize)
          ok = ok && entry_value(base[rr] + (x - b0), dtype) == first[rr];
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
  // the whole mask buffer: no load leaves it
  const uintptr_t buf_lo = reinterpret_cast<uintptr_t>(mask);
  const uintptr_t buf_hi = buf_lo + static_cast<uintptr_t>(mB) * mH * N * static_cast<uintptr_t>(cols) * esize;
  const bool nt = static_cast<double>(buf_hi - buf_lo) > kStreamBytes;
  if (c_out == nullptr) {
    const size_t slice_bytes = static_cast<size_t>(mH) * N * cols * esize;
    const int nrows = mH * N;
    const uint32_t grid = static_cast<uint32_t>(std::min<int64_t>((nrows + kScanRows - 1) / kScanRows, 2048));
    for (int b = 0; b < mB; ++b) {
      const int tspan = mB == 1 ? tmax_all : tv[b];
      const int nc = ncheck_of(tspan), z = zero_of(tspan);
      const uint8_t* mb = static_cast<const uint8_t*>(mask) + b * slice_bytes;
      const bool wide = static_cast<int64_t>(nc) * esize >= 512 * 16;
      auto kern = nt ? (wide ? k_mask_scan<true, 2> : k_mask_scan<true, 1>)
                     : (wide ? k_mask_scan<false, 2> : k_mask_scan<false, 1>);
      kern<<<grid, kMaskThreads, 0, s>>>(mb, buf_lo, buf_hi, mask_dtype, esize, cols, nrows, nc, z, flag);
    }
  } else if (mB == 1) {
    const int nc = ncheck_of(tmax_all), z = zero_of(tmax_all);
    (nt ? k_mask_check<true> : k_mask_check<false>)<<<static_cast<uint32_t>(mH) * N, kMaskThreads, 0, s>>>(
        static_cast<const uint8_t*>(mask), buf_lo, buf_hi, mask_dtype, esize, cols, nc, z, flag, c_out, early);
  } else {
    const size_t slice_bytes = static_cast<size_t>(mH) * N * cols * esize;
    for (int b = 0; b < mB; ++b) {
      const int nc = ncheck_of(tv[b]), z = zero_of(tv[b]);
      (nt ? k_mask_check<true> : k_mask_check<false>)<<<static_cast<uint32_t>(mH) * N, kMaskThreads, 0, s>>>(
          static_cast<const uint8_t*>(mask) + b * slice_bytes, buf_lo, buf_hi, mask_dtype, esize, cols, nc, z, flag,
          c_out ? c_out + static_cast<size_t>(b) * mH * N : nullptr, early);
    }
  }
  return hipGetLastError();
}

}  // namespace safe

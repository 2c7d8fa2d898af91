// Row gather / scatter between the full-token cached state and a packed sensitive-row buffer
// (SAFE-DiT technical summary, Methodology 3: only the S rows of the state change in an SRSU step).
// Pure data movement: 16-byte vector copies, one lane per 16-byte chunk, HBM-bound; nontemporal when the
// launch moves more than the MALL holds.
#include "common.hpp"

namespace safe {

template <bool SCATTER, bool NT>
__global__ __launch_bounds__(256) void k_rows_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   const int32_t* __restrict__ rows, uint32_t k, uint32_t N,
                                                   uint32_t cpr, uint32_t total) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t c = blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
    const uint32_t part = c % cpr;
    const uint32_t bhr = c / cpr;
    const uint32_t r = bhr % k;
    const uint32_t bh = bhr / k;
    const int32_t row = rows[r];
    if (row < 0 || static_cast<uint32_t>(row) >= N) continue;
    const size_t sidx = (static_cast<size_t>(bh) * N + static_cast<uint32_t>(row)) * cpr + part;
    if (SCATTER)
      store_s<NT>(dst + sidx, load_s<NT>(src + c));
    else
      store_s<NT>(dst + c, load_s<NT>(src + sidx));
  }
}

// Same copy when a row is a power-of-two number of 16-byte chunks (every bf16 / fp32 row of d = 64): the
// chunk -> (row, part) split is a shift and a mask instead of two integer divisions, which shortens each
// thread's address computation ahead of its load (about 5-8% on the kernel at 5120 rows of 2 x 24 heads).
template <bool SCATTER, bool NT>
__global__ __launch_bounds__(256) void k_rows_copy_p2(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                      const int32_t* __restrict__ rows, uint32_t k, uint32_t N,
                                                      uint32_t cpr_log2, uint32_t total) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= total) return;
  const uint32_t part = c & ((1u << cpr_log2) - 1u);
  const uint32_t bhr = c >> cpr_log2;
  const uint32_t bh = bhr / k;
  const int32_t row = rows[bhr - bh * k];
  if (row < 0 || static_cast<uint32_t>(row) >= N) return;
  const size_t sidx = ((static_cast<size_t>(bh) * N + static_cast<uint32_t>(row)) << cpr_log2) | part;
  if (SCATTER)
    store_s<NT>(dst + sidx, load_s<NT>(src + c));
  else
    store_s<NT>(dst + c, load_s<NT>(src + sidx));
}

template <bool SCATTER, bool NT>
static void rows_copy(const void* src, void* dst, const int32_t* rows, uint32_t k, uint32_t N, uint32_t cpr,
                      uint32_t total, hipStream_t s) {
  const uint4* sp = static_cast<const uint4*>(src);
  uint4* dp = static_cast<uint4*>(dst);
  if ((cpr & (cpr - 1)) == 0) {
    const uint32_t cpr_log2 = static_cast<uint32_t>(__builtin_ctz(cpr));
    k_rows_copy_p2<SCATTER, NT><<<(total + 255) / 256, 256, 0, s>>>(sp, dp, rows, k, N, cpr_log2, total);
    return;
  }
  uint32_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  k_rows_copy<SCATTER, NT><<<blocks, 256, 0, s>>>(sp, dp, rows, k, N, cpr, total);
}

hipError_t launch_rows_copy(const void* src, void* dst, const int32_t* rows, int k, int B, int H, int N,
                            int row_bytes, bool scatter, hipStream_t s) {
  const uint32_t cpr = static_cast<uint32_t>(row_bytes / 16);
  const uint32_t total = static_cast<uint32_t>(B) * H * static_cast<uint32_t>(k) * cpr;
  if (total == 0) return hipSuccess;
  const bool nt = 2.0 * 16.0 * total > kStreamBytes;  // bytes read + written
  if (scatter) {
    if (nt) rows_copy<true, true>(src, dst, rows, k, N, cpr, total, s);
    else rows_copy<true, false>(src, dst, rows, k, N, cpr, total, s);
  } else {
    if (nt) rows_copy<false, true>(src, dst, rows, k, N, cpr, total, s);
    else rows_copy<false, false>(src, dst, rows, k, N, cpr, total, s);
  }
  return hipGetLastError();
}

}  // namespace safe

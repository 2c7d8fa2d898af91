// Which bytes the mask-elision scan reads (shared by the kernels in mask_check.hip and the host-side
// bounds test in tests/test_abi.py, which compiles this header on the CPU).
//
// A row's entries occupy the byte span [b0, hi) of the mask buffer [buf_lo, buf_hi).  The scan reads the
// aligned 16-byte blocks that lie inside both the buffer and the 16-byte-rounded span -- [wlo, wlo + 16 nw) --
// with unconditional 16-byte loads (their bytes outside the row span belong to neighbouring rows of the same
// buffer and are ignored), and the entries of the span outside those blocks one entry at a time.  Entries read
// one at a time exist only at the two ends of a buffer whose base or length is not a multiple of 16, or in
// a buffer too small to hold an aligned block.  No byte outside [buf_lo, buf_hi) is ever read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace safe {

struct RowBlocks {
  uintptr_t wlo;  // first whole block
  uint32_t nw;    // number of whole blocks (0: every entry is read singly)
};

__host__ __device__ inline RowBlocks row_blocks(uintptr_t b0, uintptr_t hi, uintptr_t buf_lo, uintptr_t buf_hi) {
  const uintptr_t lo = b0 & ~static_cast<uintptr_t>(15);
  const uintptr_t up = (hi + 15) & ~static_cast<uintptr_t>(15);
  const uintptr_t blo = (buf_lo + 15) & ~static_cast<uintptr_t>(15);
  const uintptr_t bhi = buf_hi & ~static_cast<uintptr_t>(15);
  const uintptr_t wlo = lo > blo ? lo : blo;
  const uintptr_t whi = up < bhi ? up : bhi;
  return {wlo, whi > wlo ? static_cast<uint32_t>((whi - wlo) / 16) : 0u};
}

// The byte ranges of the span read one entry at a time: [e0, e1) and [e2, e3) (possibly empty).
__host__ __device__ inline void row_edges(uintptr_t b0, uintptr_t hi, RowBlocks rb, uintptr_t* e0, uintptr_t* e1,
                                          uintptr_t* e2, uintptr_t* e3) {
  if (rb.nw == 0) {
    *e0 = b0, *e1 = hi, *e2 = hi, *e3 = hi;
    return;
  }
  const uintptr_t whi = rb.wlo + static_cast<uintptr_t>(rb.nw) * 16;
  *e0 = b0;
  *e1 = rb.wlo > b0 ? (rb.wlo < hi ? rb.wlo : hi) : b0;
  *e2 = whi > b0 ? (whi < hi ? whi : hi) : b0;
  *e3 = hi;
  if (*e2 < *e1) *e2 = *e1;
}

}  // namespace safe

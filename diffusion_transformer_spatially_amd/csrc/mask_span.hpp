// Which bytes the mask-elision scan reads (shared by the kernels in mask_check.hip and the host-side
// bounds test in tests/test_abi.py, which compiles this header on the CPU).
//
// A row's entries occupy the byte span [b0, hi) of the mask buffer [buf_lo, buf_hi).  The scan visits
// every aligned 16-byte block that meets the span.  A block that lies wholly inside the buffer is read with
// one 16-byte load (its bytes outside the row span belong to neighbouring rows and are ignored); a block
// that sticks out of the buffer -- only possible for the first or last block of a buffer whose base or
// length is not a multiple of 16 -- is read one byte at a time, and only its bytes inside the row span.
// So no byte outside [buf_lo, buf_hi) is ever read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace safe {

struct RowBlocks {
  uintptr_t lo;  // address of the first aligned block that meets the span
  uint32_t n;    // number of blocks
};

__host__ __device__ inline RowBlocks row_blocks(uintptr_t b0, uintptr_t hi) {
  const uintptr_t lo = b0 & ~static_cast<uintptr_t>(15);
  return {lo, static_cast<uint32_t>((hi - lo + 15) / 16)};
}

__host__ __device__ inline bool block_whole(uintptr_t a, uintptr_t buf_lo, uintptr_t buf_hi) {
  return a >= buf_lo && a + 16 <= buf_hi;
}

// Byte range [*r0, *r1) of block a read one byte at a time when the block is not whole.
__host__ __device__ inline void block_bytes(uintptr_t a, uintptr_t b0, uintptr_t hi, uintptr_t* r0, uintptr_t* r1) {
  *r0 = a > b0 ? a : b0;
  *r1 = a + 16 < hi ? a + 16 : hi;
}

}  // namespace safe

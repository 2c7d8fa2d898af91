// bf16 attention for gfx950 (dense anchor rows or gathered sensitive rows), mask-free or with a kept
// general mask.
//
// Computes, for image query rows of (b,h) -- all N rows (anchor refresh, SAFE-DiT technical summary
// Methodology 3 "CAR") or the rows of S (Methodology 3 "SRSU"; AccelAes summary B.2 SkipSparse) --
// one joint softmax over the N image keys followed by the Tv[b] valid text keys (text padding is kept
// exactly: padded slots are never loaded), and writes the output rows into the full-token state.
//
// Shape of the work (d = 64):
//  * a workgroup of 4 waves owns 4 * 32 * QB query rows of one (b,h); each wave owns QB blocks of 32
//    rows, so every K / V operand read from LDS feeds QB matrix instructions;
//  * keys stream in tiles of BN = 64 through double-buffered LDS (16-byte chunks XOR-swizzled by row);
//  * per tile: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys are the M dimension, queries the N
//    dimension), so every lane holds the 32 logits of one query row per block: lane L owns query
//    L%32 and keys 16*(L/32) + r (r = 0..15) of each 32-key block, thanks to a fixed permutation of
//    the K rows fed to the instruction;
//  * fp32 online softmax in log2 units (scale*log2(e) folded into one FMA per logit, or into Q once
//    when no log-sum-exp is returned, v_exp_f32); the row max is combined across the two lane halves
//    with v_permlane32_swap; the output is rescaled only when some row's max grew; the row sum
//    accumulates the bf16-rounded probabilities with v_dot2_f32_bf16, i.e. exactly the values the P V
//    product uses (the fp32 probabilities when a log-sum-exp output is requested);
//  * a kept mask (bool or fp32, one query block per wave) is read straight from global memory one tile
//    ahead, each lane loading its own row's 16-key chunks, and applied to the logits after S^T;
//  * O^T += V^T P^T on the same instruction: the P^T operand is the lane's own probabilities (no data
//    movement), the V^T operand is read from row-major LDS with ds_read_b64_tr_b16;
//  * with two query blocks per wave the tile is staggered: the logits of block 1 and the output update
//    of block 0 are issued alongside the softmax of the other block, so one wave keeps its matrix and
//    vector work overlapped: each matrix instruction of one block is followed by the exp2 / pack /
//    row-sum work of 4 logits of the other, in a fixed order (sched_barrier between the groups);
//  * full image tiles run a loop without any masking; the ragged image tail and the text tiles run a
//    separate path that masks keys past the valid count and, for the warmup emission, stores the
//    text-block logits and the image-block log-sum-exp;
//  * gathered rows: Q rows are loaded from rows[r] and outputs scattered to rows[r] in the epilogue;
//  * few query rows (too few waves to fill the GPU): 8-wave workgroups, waves 0-3 take the first half
//    of the key tiles and waves 4-7 the rest, each half with its own LDS buffers; at the end the
//    second half's running max, row sum and output accumulators go through LDS to the first half,
//    which merges them (the usual rescale by exp2 of the max differences) and writes the output.
// The workgroup id is remapped so that the Q tiles of one (b,h) run on the same XCD and share K/V
// in that XCD's L2.
#include "common.hpp"

namespace safe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// elements of one K or V tile (64 keys x head dim D)
template <int D>
constexpr int kTileElems = kBN * D;

__device__ __forceinline__ float swap_halves(float x) {
  // value held by lane L ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t lane = threadIdx.x & 63;
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// XOR swizzle of the 16-byte chunk index by key row, so that both LDS read patterns of a tile step --
// 16-byte reads of 16 permuted K rows (rows differing in bits 0, 1, 2 and 4), and transposing 8-byte
// reads of 4 consecutive V rows -- spread over all 64 banks without conflicts.
//  D = 64 (128-byte rows, two rows per 256-byte bank window): row bits (1, 2, 4) go to chunk bits
//  (2, 1, 0); row bit 0 already picks the half of the window.
//  D = 128 (256-byte rows, one row per window): row bits (2, 4, 0, 1) go to chunk bits (0, 1, 2, 3);
//  the K pattern needs an injective map of the four varying row bits, the V pattern (4 consecutive
//  rows x 4 consecutive chunks) needs row bits 0 and 1 on chunk bits 2 and 3.
template <int D>
__device__ __forceinline__ int swz(int key) {
  if constexpr (D == 64) return (((key >> 1) & 1) << 2) | (((key >> 2) & 1) << 1) | ((key >> 4) & 1);
  else return ((key & 1) << 2) | (((key >> 1) & 1) << 3) | ((key >> 2) & 1) | (((key >> 4) & 1) << 1);
}
// LDS element offset of (key row, 16-byte chunk) with the chunk XOR-swizzled by the row.
template <int D>
__device__ __forceinline__ int lds_off(int key, int chunk) { return key * D + ((chunk ^ swz<D>(key)) << 3); }

struct TileSrc {
  const uint16_t* k;  // bf16 K rows (D elements), or fp8 K rows (D bytes) read through k8
  const uint16_t* v;
  int nvalid;
  __device__ const uint8_t* k8() const { return reinterpret_cast<const uint8_t*>(k); }
};

// FP8: K rows are D bytes (fp8 E4M3) instead of 2D; V stays bf16.
template <int D, bool FP8 = false>
__device__ __forceinline__ TileSrc tile_src(const AttnArgs& a, size_t bh, int t, int n_img, int tv) {
  constexpr size_t kRowK = FP8 ? D : 2 * D;  // bytes per K row
  TileSrc s;
  if (t < n_img) {
    const int j0 = t * kBN;
    s.k = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.k_img) + (bh * a.N + j0) * kRowK);
    s.v = static_cast<const uint16_t*>(a.v_img) + (bh * a.N + j0) * D;
    s.nvalid = min(kBN, a.N - j0);
  } else {
    const int j0 = (t - n_img) * kBN;
    s.k = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.k_txt) + (bh * a.T + j0) * kRowK);
    s.v = static_cast<const uint16_t*>(a.v_txt) + (bh * a.T + j0) * D;
    s.nvalid = min(kBN, tv - j0);
  }
  return s;
}

// Direct global -> LDS copies of one tile (no VGPR staging): each wave instruction writes 64
// consecutive 16-byte LDS slots; slot p holds key row p/(D/8), chunk (p%(D/8)) ^ swz(row) (the XOR swizzle), so
// the global address of each lane is chosen to land its chunk in that slot.  Rows past nvalid are
// clamped to the last valid row (never read out of bounds, never read padded text); the softmax
// masks those keys to -inf and their probabilities are exactly 0.
//
// OPAQUE (used with two query blocks per wave, where registers are scarce): the wave's first slot goes
// through an empty asm, so the compiler cannot treat the LDS destinations derived from it as loop
// invariants; it recomputes them per tile (two scalar adds) instead of hoisting all of them out of the
// tile loop, where they were spilled and each reload waited for the tile copies already in flight.
// FP8 K tiles (head dim 64): 64-byte key rows, four 16-byte chunks; chunk c of key row r sits in LDS slot
// 4r + (c ^ swz8(r)).  The K operand read of a lane half takes chunks (2g, 2g + 1) of 16 key rows that
// differ in row bits {0, 1, 2, 4}: rows with equal bits 0-1 share a 16-byte bank quad of the 256-byte
// window unless their chunks differ, which row bits 2 and 4 ensure, so each read is conflict-free.
__device__ __forceinline__ int swz8(int key) { return ((key >> 2) & 1) | (((key >> 4) & 1) << 1); }
__device__ __forceinline__ int lds8_off(int key, int chunk) { return key * 64 + ((chunk ^ swz8(key)) << 4); }  // bytes

template <int D, bool OPAQUE, bool FP8 = false>
__device__ __forceinline__ void stage_issue(const TileSrc& s, uint16_t* kl, uint16_t* vl) {
  constexpr int kChunks = D / 8;                // 16-byte chunks per key row
  constexpr int kChunkShift = D == 64 ? 3 : 4;  // log2(kChunks)
  const int lane = threadIdx.x & 63;
  int wslot = __builtin_amdgcn_readfirstlane(static_cast<int>((threadIdx.x >> 6) & 3)) * 64;
  if (OPAQUE) asm volatile("" : "+s"(wslot));
  if constexpr (FP8 && D == 64) {
    const int p = wslot + lane;  // one 16-byte slot per thread: 64 rows x 4 chunks
    const int row = p >> 2;
    const int c = (p & 3) ^ swz8(row);
    const int srow = row < s.nvalid ? row : s.nvalid - 1;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(s.k8() + srow * 64 + c * 16),
                                     (__attribute__((address_space(3))) void*)(kl + wslot * 8), 16, 0, 0);
  } else if constexpr (FP8) {
    // head dim 128: 128-byte rows, laid out as the bf16 head-dim-64 K tile (8 chunks, swz<64>)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int base = u * kWaves * 64 + wslot;
      const int p = base + lane;
      const int row = p >> 3;
      const int c = (p & 7) ^ swz<64>(row);
      const int srow = row < s.nvalid ? row : s.nvalid - 1;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(s.k8() + srow * 128 + c * 16),
                                       (__attribute__((address_space(3))) void*)(kl + base * 8), 16, 0, 0);
    }
  }
#pragma unroll
  for (int u = 0; u < kBN * kChunks / (kWaves * 64); ++u) {
    const int base = u * kWaves * 64 + wslot;  // first slot of this wave instruction
    const int p = base + lane;
    const int row = p >> kChunkShift;
    const int c = (p & (kChunks - 1)) ^ swz<D>(row);
    const int srow = row < s.nvalid ? row : s.nvalid - 1;
    if constexpr (!FP8)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(s.k + srow * D + c * 8),
                                       (__attribute__((address_space(3))) void*)(kl + base * 8), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(s.v + srow * D + c * 8),
                                     (__attribute__((address_space(3))) void*)(vl + base * 8), 16, 0, 0);
  }
}

// Copies of a full tile (all 64 keys valid, no clamping): the per-lane byte offset of each copy
// instruction's chunk within the tile does not depend on the tile, so it is computed once (off[u]) and
// added to the tile's uniform base, which lets the copy take a scalar base and a 32-bit vector offset
// instead of a 64-bit address computed per tile.
template <int D>
__device__ __forceinline__ void stage_offsets(uint32_t (&off)[D / 32]) {
  constexpr int kChunks = D / 8;
  constexpr int kChunkShift = D == 64 ? 3 : 4;
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    const int p = u * kWaves * 64 + static_cast<int>(threadIdx.x & 255);
    const int row = p >> kChunkShift;
    const int c = (p & (kChunks - 1)) ^ swz<D>(row);
    off[u] = static_cast<uint32_t>((row * D + c * 8) * 2);
  }
}

// koff8: the fp8 K copy's per-lane byte offsets within a full tile (FP8 only), one per copy instruction:
// head dim 64 one (64-byte rows), head dim 128 two (128-byte rows: the offsets of the bf16 head-dim-64 K copy).
template <int D>
__device__ __forceinline__ void stage8_offsets(uint32_t (&off)[D / 64]) {
  if constexpr (D == 64) {
    const int p = static_cast<int>(threadIdx.x & 255);
    const int row = p >> 2;
    off[0] = static_cast<uint32_t>(row * 64 + (((p & 3) ^ swz8(row)) << 4));
  } else {
    stage_offsets<64>(off);
  }
}

template <int D, bool OPAQUE, bool FP8 = false>
__device__ __forceinline__ void stage_issue_full(const TileSrc& s, uint16_t* kl, uint16_t* vl, const uint32_t (&off)[D / 32],
                                                 const uint32_t (&koff8)[D / 64]) {
  int wslot = __builtin_amdgcn_readfirstlane(static_cast<int>((threadIdx.x >> 6) & 3)) * 64;
  if (OPAQUE) asm volatile("" : "+s"(wslot));
  const char* kb = reinterpret_cast<const char*>(s.k);
  const char* vb = reinterpret_cast<const char*>(s.v);
  if constexpr (FP8) {
#pragma unroll
    for (int u = 0; u < D / 64; ++u)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb + koff8[u]),
                                       (__attribute__((address_space(3))) void*)(kl + (u * kWaves * 64 + wslot) * 8), 16, 0,
                                       0);
  }
#pragma unroll
  for (int u = 0; u < D / 32; ++u) {
    const int base = u * kWaves * 64 + wslot;
    if constexpr (!FP8)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(kb + off[u]),
                                       (__attribute__((address_space(3))) void*)(kl + base * 8), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(vb + off[u]),
                                     (__attribute__((address_space(3))) void*)(vl + base * 8), 16, 0, 0);
  }
}

// S^T block of 32 keys x 32 queries over the whole head dim (64) from fp8 K and Q on the gfx950 fp8 matrix
// instruction (format 0 = E4M3 for both operands; block scales 2^0).  Each lane half g holds bytes
// 32g .. 32g + 31 of its row of K (A) and of Q (B): whatever order the instruction gives the 64 products,
// both operands follow the same one, so the sum is the full dot product.
__device__ __forceinline__ f32x16 mfma_fp8(bf16x8 a0, bf16x8 a1, bf16x8 b0, bf16x8 b1, const f32x16& c) {
  const i32x8 av = __builtin_shufflevector(__builtin_bit_cast(i32x4, a0), __builtin_bit_cast(i32x4, a1), 0, 1, 2, 3, 4, 5,
                                           6, 7);
  const i32x8 bv = __builtin_shufflevector(__builtin_bit_cast(i32x4, b0), __builtin_bit_cast(i32x4, b1), 0, 1, 2, 3, 4, 5,
                                           6, 7);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
}

// A lane's fp8 K operand of key row `key` for bytes 64j .. 64j + 63 of the row: chunks 4j + 2g and 4j + 2g + 1
// (head dim 64: 64-byte rows; head dim 128: 128-byte rows in the layout of the bf16 head-dim-64 tile).
template <int D = 64>
__device__ __forceinline__ void read_k8(bf16x8 (&ka)[2], const uint16_t* kl, int key, int g, int j = 0) {
  if constexpr (D == 64) {
    const uint8_t* kb = reinterpret_cast<const uint8_t*>(kl);
    ka[0] = *reinterpret_cast<const bf16x8*>(kb + lds8_off(key, 2 * g));
    ka[1] = *reinterpret_cast<const bf16x8*>(kb + lds8_off(key, 2 * g + 1));
  } else {
    ka[0] = *reinterpret_cast<const bf16x8*>(kl + lds_off<64>(key, 4 * j + 2 * g));
    ka[1] = *reinterpret_cast<const bf16x8*>(kl + lds_off<64>(key, 4 * j + 2 * g + 1));
  }
}

// fp8 S^T block of 32 keys (rows kb*32 + kperm of the tile) x the wave's 32 queries over the whole head dim:
// one fp8 instruction per 64 bytes of the rows; the Q operand holds bytes 64j + 32g .. +31 in q[2j], q[2j+1].
template <int D>
__device__ __forceinline__ f32x16 logits_fp8(const uint16_t* kl, int key, int g, const bf16x8 (&q)[D / 16]) {
  f32x16 s = {};
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    bf16x8 ka[2];
    read_k8<D>(ka, kl, key, g, j);
    s = mfma_fp8(ka[0], ka[1], q[2 * j], q[2 * j + 1], s);
  }
  return s;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Per-wave running state of QB query blocks.
template <int QB, int D>
struct WaveState {
  bf16x8 q[QB][D / 16];  // Q^T operand: lane (q + 32g) holds Q[q][16ks + 8g .. +7]
  f32x16 o[QB][D / 32];  // O^T accumulators: lane holds query L%32, head dims db*32 + 8(r/4) + 4g + r%4
  float m[QB];       // running row max (raw dot-product units)
  float l[QB];       // running row sum of exp2((s - m) * c2), lane-half partial
};

// Kept general mask on the MFMA path (KM = 1: bool, a false entry makes the logit -inf; KM = 2: fp32,
// added to the scaled logit), one query block per wave.  A lane needs its own query row's entries for
// keys 16g .. 16g+15 of both 32-key halves of a tile: two 16-byte chunks (bool) or two 64-byte chunks
// (fp32), loaded into registers one tile ahead.  Chunks wholly past the tile's valid keys are not
// loaded (those keys are -inf anyway); a chunk never crosses the end of a mask row because the host
// only takes this path when N and the row length are multiples of 16.
template <int KM>
struct MaskTile {
  uint4 w[2][KM == 2 ? 4 : 1];
};

template <int KM>
__device__ __forceinline__ void mask_load(MaskTile<KM>& mt, const uint8_t* mrow, int col0, int nvalid, int g,
                                          bool zero) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int off = kb * 32 + 16 * g;
    const bool ld = !zero && off < nvalid;
    if (KM == 1) {
      mt.w[kb][0] = ld ? *reinterpret_cast<const uint4*>(mrow + col0 + off) : make_uint4(~0u, ~0u, ~0u, ~0u);
    } else {
#pragma unroll
      for (int j = 0; j < (KM == 2 ? 4 : 1); ++j)
        mt.w[kb][j] = ld ? *reinterpret_cast<const uint4*>(mrow + 4 * static_cast<size_t>(col0 + off) + 16 * j)
                         : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// Applies the mask to the 16 logits of half kb; factor turns a natural-log mask value into the units of
// the logits (1/scale for raw dot products, log2 e for pre-scaled log2 logits).
template <int KM>
__device__ __forceinline__ void mask_apply(f32x16& s, const MaskTile<KM>& mt, int kb, float factor) {
  if (KM == 1) {
    const uint32_t w[4] = {mt.w[kb][0].x, mt.w[kb][0].y, mt.w[kb][0].z, mt.w[kb][0].w};
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = ((w[i >> 2] >> (8 * (i & 3))) & 0xffu) ? s[i] : -INFINITY;
  } else if (KM == 2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 v = mt.w[kb][j];
      s[4 * j + 0] = fmaf(__uint_as_float(v.x), factor, s[4 * j + 0]);
      s[4 * j + 1] = fmaf(__uint_as_float(v.y), factor, s[4 * j + 1]);
      s[4 * j + 2] = fmaf(__uint_as_float(v.z), factor, s[4 * j + 2]);
      s[4 * j + 3] = fmaf(__uint_as_float(v.w), factor, s[4 * j + 3]);
    }
  }
}

// Fast path (no lse, no emission), head dim 64: Q was pre-multiplied by scale * log2(e) and rounded to
// bf16 once, so the logits come out of the MFMA in log2 units, and each tile's logit accumulators start
// at -m (two 64-bit moves per four registers), so the MFMA output is already s - m and each probability
// costs a single exp2 instead of an fma and an exp2.  Rounding the scaled Q to bf16 perturbs a logit by
// about 2^-9 of the root-sum-square of its products, below the bf16 rounding of the probabilities
// themselves.  Head dim 128 keeps Q exact and takes the fma per logit (s * scale * log2 e - m): with half
// the vector work per matrix instruction of head dim 64 it has the room, and on sharply peaked rows
// (logits with a standard deviation near 9) the rounded-Q error there reached the bf16 output tolerance.
// The lazy running max and its exact path are as in the general step below (m is kept in log2 units).

// One query block's softmax of a tile on the fast path (logits s are log2 units minus m): probabilities
// p and their bf16 row-sum contribution, with the lazy-max exact path.  Split out so that the two query
// blocks of a wave can be staggered against each other's matrix work.
template <bool MASKED>
__device__ __forceinline__ float fast_probs(bf16x8 (&p)[2][2], f32x16 (&s)[2], int g, int nvalid) {
  if (MASKED) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = (kb * 32 + 16 * g + i) < nvalid ? s[kb][i] : -INFINITY;
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float tsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pk[e] = pack_bf16x2(__builtin_amdgcn_exp2f(s[kb][8 * mm + 2 * e]), __builtin_amdgcn_exp2f(s[kb][8 * mm + 2 * e + 1]));
        tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), ones, tsum, false);
      }
      p[kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk[0], pk[1], pk[2], pk[3]});
    }
  return tsum;
}

// Exact path of one query block (rare): logits again from K in LDS, tile max, rescale, probabilities again.
template <bool MASKED, int D>
__device__ __forceinline__ float fast_exact(bf16x8 (&p)[2][2], const bf16x8 (&q)[D / 16], float& m, float& l,
                                            f32x16 (&o)[D / 32], const uint16_t* kl, int kperm, int g, int nvalid) {
  f32x16 sx[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + lds_off<D>(kb * 32 + kperm, 2 * ks + g));
      sx[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, q[ks], ks == 0 ? (f32x16){} : sx[kb], 0, 0, 0);
    }
  if (MASKED) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sx[kb][i] = (kb * 32 + 16 * g + i) < nvalid ? sx[kb][i] : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sx[kb][i]);
  mx = fmaxf(mx, swap_halves(mx));
  const float mnew = fmaxf(m, mx);
  if (mnew > m) {
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    m = mnew;
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) sx[kb][i] -= m;
  return fast_probs<false>(p, sx, g, kBN);
}

// 4 logits of one block (chunk c of 8: half kb = c>>2, word group mm = (c>>1)&1, quarter h = c&1):
// exp2, pack to bf16 pairs, add to the row sum.
__device__ __forceinline__ void soft_chunk(uint32_t (&pk)[2][2][4], const f32x16 (&s)[2], float& tsum, int c) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int kb = c >> 2, mm = (c >> 1) & 1, h = c & 1;
  const int i0 = 8 * mm + 4 * h;
  const uint32_t w0 = pack_bf16x2(__builtin_amdgcn_exp2f(s[kb][i0 + 0]), __builtin_amdgcn_exp2f(s[kb][i0 + 1]));
  const uint32_t w1 = pack_bf16x2(__builtin_amdgcn_exp2f(s[kb][i0 + 2]), __builtin_amdgcn_exp2f(s[kb][i0 + 3]));
  pk[kb][mm][2 * h] = w0;
  pk[kb][mm][2 * h + 1] = w1;
  tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, tsum, false);
  tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, tsum, false);
}

// Two query blocks, staggered: logits of block 0; logits of block 1 interleaved with the softmax of
// block 0; the V operands; output update of block 0 interleaved with the softmax of block 1; output
// update of block 1.  Each interleaved group is one MFMA (32 cycles) and the vector work of 4 logits
// (4 exp2, 2 packs, 2 dot products, about as long); sched_barrier pins the groups in this order, which
// the scheduler otherwise bunches into long vector runs with the matrix core idle.  The lazy-max exact
// path of a block runs between its softmax and its output update.
template <bool MASKED>
__device__ __forceinline__ void tile_step_fast2(WaveState<2, 64>& st, const uint16_t* kl, const uint16_t* vl, int kperm,
                                                int g, int li, int dc0, int nvalid) {
  bf16x8 ka[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ka[kb][ks] = *reinterpret_cast<const bf16x8*>(kl + lds_off<64>(kb * 32 + kperm, 2 * ks + g));
  f32x16 s0[2], s1[2];
  {
    const double n0 = __builtin_bit_cast(double, (f32x2){-st.m[0], -st.m[0]});
    const double n1 = __builtin_bit_cast(double, (f32x2){-st.m[1], -st.m[1]});
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      double d0[8], d1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) { d0[i] = n0; d1[i] = n1; }
      s0[kb] = __builtin_bit_cast(f32x16, d0);
      s1[kb] = __builtin_bit_cast(f32x16, d1);
    }
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s0[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][ks], st.q[0][ks], s0[kb], 0, 0, 0);
  if (MASKED) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s0[kb][i] = (kb * 32 + 16 * g + i) < nvalid ? s0[kb][i] : -INFINITY;
  }
  __builtin_amdgcn_sched_barrier(0);
  // logits of block 1 | softmax of block 0, one MFMA per 4 logits
  uint32_t pk0[2][2][4];
  float t0 = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int ks = c >> 1, kb = c & 1;
    s1[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kb][ks], st.q[1][ks], s1[kb], 0, 0, 0);
    soft_chunk(pk0, s0, t0, c);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (MASKED) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s1[kb][i] = (kb * 32 + 16 * g + i) < nvalid ? s1[kb][i] : -INFINITY;
  }
  bf16x8 p0[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
      p0[kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk0[kb][mm][0], pk0[kb][mm][1], pk0[kb][mm][2], pk0[kb][mm][3]});
  if (__any(!(t0 <= 65536.f))) t0 = fast_exact<MASKED, 64>(p0, st.q[0], st.m[0], st.l[0], st.o[0], kl, kperm, g, nvalid);
  st.l[0] += t0;
  // V^T operands (shared by both blocks)
  lds_u16* vl3 = (lds_u16*)(vl);
  bf16x8 va[2][2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int key = kb * 32 + 16 * g + 8 * mm + (li >> 2);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int col = db * 32 + dc0 + 4 * (li & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off<64>(key, col >> 3) + (col & 4)));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off<64>(key + 4, col >> 3) + (col & 4)));
        va[kb][mm][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  __builtin_amdgcn_sched_barrier(0);
  // output update of block 0 | softmax of block 1: two chunks first (covering the V reads' latency)
  uint32_t pk1[2][2][4];
  float t1 = 0.f;
  soft_chunk(pk1, s1, t1, 0);
  soft_chunk(pk1, s1, t1, 1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kb = i >> 2, mm = (i >> 1) & 1, db = i & 1;
    st.o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kb][mm][db], p0[kb][mm], st.o[0][db], 0, 0, 0);
    if (i + 2 < 8) soft_chunk(pk1, s1, t1, i + 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 p1[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
      p1[kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk1[kb][mm][0], pk1[kb][mm][1], pk1[kb][mm][2], pk1[kb][mm][3]});
  if (__any(!(t1 <= 65536.f))) t1 = fast_exact<MASKED, 64>(p1, st.q[1], st.m[1], st.l[1], st.o[1], kl, kperm, g, nvalid);
  st.l[1] += t1;
  // output update of block 1
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int db = 0; db < 2; ++db)
        st.o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kb][mm][db], p1[kb][mm], st.o[1][db], 0, 0, 0);
}

// soft_chunk on raw fp8 dot products: each probability is exp2(s * c2 - m), c2 = scale * log2(e) times the
// (b,h) dequantisation factors of Q and K (the fp8 operands cannot carry the scale, so the fma that the
// bf16 path folds into a pre-scaled Q is paid per logit here; the logit chains start at zero instead).
__device__ __forceinline__ void soft_chunk_sc(uint32_t (&pk)[2][2][4], const f32x16 (&s)[2], float& tsum, int c, float c2,
                                              float nm) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int kb = c >> 2, mm = (c >> 1) & 1, h = c & 1;
  const int i0 = 8 * mm + 4 * h;
  const uint32_t w0 = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[kb][i0 + 0], c2, nm)),
                                  __builtin_amdgcn_exp2f(fmaf(s[kb][i0 + 1], c2, nm)));
  const uint32_t w1 = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(s[kb][i0 + 2], c2, nm)),
                                  __builtin_amdgcn_exp2f(fmaf(s[kb][i0 + 3], c2, nm)));
  pk[kb][mm][2 * h] = w0;
  pk[kb][mm][2 * h + 1] = w1;
  tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, tsum, false);
  tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, tsum, false);
}

// Logits of a tile in log2 units minus m (s * c2 - m), keys past nvalid at -inf (partial fp8 tiles).
template <bool MASKED>
__device__ __forceinline__ void scale_logits(f32x16 (&s)[2], float c2, float nm, int g, int nvalid) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = fmaf(s[kb][i], c2, nm);
      s[kb][i] = (!MASKED || (kb * 32 + 16 * g + i) < nvalid) ? v : -INFINITY;
    }
}

// Exact path of one fp8 query block (rare): logits again from K in LDS, tile max in log2 units, rescale,
// probabilities again.
template <bool MASKED>
__device__ __forceinline__ float fast_exact_fp8(bf16x8 (&p)[2][2], bf16x8 q0, bf16x8 q1, float& m, float& l,
                                                f32x16 (&o)[2], const uint16_t* kl, int kperm, int g, int nvalid,
                                                float c2) {
  f32x16 sx[2];
  const f32x16 zero = {};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    bf16x8 ka[2];
    read_k8(ka, kl, kb * 32 + kperm, g);
    sx[kb] = mfma_fp8(ka[0], ka[1], q0, q1, zero);
  }
  scale_logits<MASKED>(sx, c2, 0.f, g, nvalid);
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sx[kb][i]);
  mx = fmaxf(mx, swap_halves(mx));
  const float mnew = fmaxf(m, mx);
  if (mnew > m) {
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    m = mnew;
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) sx[kb][i] -= m;
  return fast_probs<false>(p, sx, g, kBN);
}

// Two fp8 query blocks, staggered as in tile_step_fast2: logits of block 0 (one fp8 instruction per 32-key
// half); logits of block 1 beside the softmax of block 0; output update of block 0 (bf16 P V) beside the
// softmax of block 1; output update of block 1.
template <bool MASKED>
__device__ __forceinline__ void tile_step_fast2_fp8(WaveState<2, 64>& st, const uint16_t* kl, const uint16_t* vl, int kperm,
                                                    int g, int li, int dc0, float c2, int nvalid) {
  bf16x8 ka[2][2];
  read_k8(ka[0], kl, kperm, g);
  read_k8(ka[1], kl, 32 + kperm, g);
  const f32x16 zero = {};
  f32x16 s0[2], s1[2];
  s0[0] = mfma_fp8(ka[0][0], ka[0][1], st.q[0][0], st.q[0][1], zero);
  s0[1] = mfma_fp8(ka[1][0], ka[1][1], st.q[0][0], st.q[0][1], zero);
  const float nm0 = -st.m[0], nm1 = -st.m[1];
  if (MASKED) scale_logits<true>(s0, c2, nm0, g, nvalid);
  __builtin_amdgcn_sched_barrier(0);
  // logits of block 1 | softmax of block 0
  uint32_t pk0[2][2][4];
  float t0 = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c == 0) s1[0] = mfma_fp8(ka[0][0], ka[0][1], st.q[1][0], st.q[1][1], zero);
    if (c == 4) s1[1] = mfma_fp8(ka[1][0], ka[1][1], st.q[1][0], st.q[1][1], zero);
    if (MASKED) soft_chunk(pk0, s0, t0, c);
    else soft_chunk_sc(pk0, s0, t0, c, c2, nm0);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (MASKED) scale_logits<true>(s1, c2, nm1, g, nvalid);
  bf16x8 p0[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
      p0[kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk0[kb][mm][0], pk0[kb][mm][1], pk0[kb][mm][2], pk0[kb][mm][3]});
  if (__any(!(t0 <= 65536.f)))
    t0 = fast_exact_fp8<MASKED>(p0, st.q[0][0], st.q[0][1], st.m[0], st.l[0], st.o[0], kl, kperm, g, nvalid, c2);
  st.l[0] += t0;
  // V^T operands (shared by both blocks)
  lds_u16* vl3 = (lds_u16*)(vl);
  bf16x8 va[2][2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int key = kb * 32 + 16 * g + 8 * mm + (li >> 2);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int col = db * 32 + dc0 + 4 * (li & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off<64>(key, col >> 3) + (col & 4)));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off<64>(key + 4, col >> 3) + (col & 4)));
        va[kb][mm][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  __builtin_amdgcn_sched_barrier(0);
  // output update of block 0 | softmax of block 1
  uint32_t pk1[2][2][4];
  float t1 = 0.f;
  if (MASKED) {
    soft_chunk(pk1, s1, t1, 0);
    soft_chunk(pk1, s1, t1, 1);
  } else {
    soft_chunk_sc(pk1, s1, t1, 0, c2, nm1);
    soft_chunk_sc(pk1, s1, t1, 1, c2, nm1);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int kb = i >> 2, mm = (i >> 1) & 1, db = i & 1;
    st.o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kb][mm][db], p0[kb][mm], st.o[0][db], 0, 0, 0);
    if (i + 2 < 8) {
      if (MASKED) soft_chunk(pk1, s1, t1, i + 2);
      else soft_chunk_sc(pk1, s1, t1, i + 2, c2, nm1);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  bf16x8 p1[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
      p1[kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk1[kb][mm][0], pk1[kb][mm][1], pk1[kb][mm][2], pk1[kb][mm][3]});
  if (__any(!(t1 <= 65536.f)))
    t1 = fast_exact_fp8<MASKED>(p1, st.q[1][0], st.q[1][1], st.m[1], st.l[1], st.o[1], kl, kperm, g, nvalid, c2);
  st.l[1] += t1;
  // output update of block 1
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int db = 0; db < 2; ++db)
        st.o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kb][mm][db], p1[kb][mm], st.o[1][db], 0, 0, 0);
}

template <int QB, bool MASKED, int KM, int D, bool FP8 = false>
__device__ __forceinline__ void tile_step_fast(WaveState<QB, D>& st, const uint16_t* kl, const uint16_t* vl, int kperm,
                                               int g, int li, int dc0, float c2, int nvalid, const MaskTile<KM>& mt) {
  // Q pre-scaled to log2 units (bf16, head dim 64) or exact (head dim 128, fp8)
  constexpr bool kPre = D == 64 && !FP8;
  static_assert(KM == 0 || QB == 1, "a kept mask runs with one query block per wave");
  static_assert(QB == 1 || D == 64, "two query blocks per wave only at head dim 64");
  if constexpr (QB == 2) {
    if constexpr (FP8) tile_step_fast2_fp8<MASKED>(st, kl, vl, kperm, g, li, dc0, c2, nvalid);
    else tile_step_fast2<MASKED>(st, kl, vl, kperm, g, li, dc0, nvalid);
    return;
  }
  f32x16 s[QB][2];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const double nm2 = __builtin_bit_cast(double, (f32x2){-st.m[qb], -st.m[qb]});
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      double d[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) d[i] = nm2;
      if constexpr (kPre) s[qb][kb] = __builtin_bit_cast(f32x16, d);
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kb * 32 + kperm;
    if constexpr (FP8) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = logits_fp8<D>(kl, key, g, st.q[qb]);
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + lds_off<D>(key, 2 * ks + g));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.q[qb][ks], (!kPre && ks == 0) ? (f32x16){} : s[qb][kb],
                                                              0, 0, 0);
      }
    }
  }
  if constexpr (!kPre) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[qb][kb][i] = fmaf(s[qb][kb][i], c2, -st.m[qb]);
  }
  if (MASKED) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[qb][kb][i] = (kb * 32 + 16 * g + i) < nvalid ? s[qb][kb][i] : -INFINITY;
  }
  if constexpr (KM != 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) mask_apply<KM>(s[0][kb], mt, kb, kLog2e);
  }
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 p[QB][2][2];
  float tl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float tsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[e] = pack_bf16x2(__builtin_amdgcn_exp2f(s[qb][kb][8 * mm + 2 * e]),
                              __builtin_amdgcn_exp2f(s[qb][kb][8 * mm + 2 * e + 1]));
          tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), ones, tsum, false);
        }
        p[qb][kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk[0], pk[1], pk[2], pk[3]});
      }
    tl[qb] = tsum;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (__any(!(tl[qb] <= 65536.f))) {
      f32x16 sx[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kb * 32 + kperm;
        if constexpr (FP8) {
          sx[kb] = logits_fp8<D>(kl, key, g, st.q[qb]);
        } else {
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + lds_off<D>(key, 2 * ks + g));
            sx[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.q[qb][ks], ks == 0 ? (f32x16){} : sx[kb], 0, 0, 0);
          }
        }
      }
      if constexpr (!kPre) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sx[kb][i] *= c2;
      }
      if (MASKED) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sx[kb][i] = (kb * 32 + 16 * g + i) < nvalid ? sx[kb][i] : -INFINITY;
      }
      if constexpr (KM != 0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mask_apply<KM>(sx[kb], mt, kb, kLog2e);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sx[kb][i]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mnew = fmaxf(st.m[qb], mx);
      if (mnew > st.m[qb]) {
        const float alpha = __builtin_amdgcn_exp2f(st.m[qb] - mnew);
        st.l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) st.o[qb][db][i] *= alpha;
        st.m[qb] = mnew;
      }
      const float m = st.m[qb];
      float tsum = 0.f;
      if (KM != 0 && m == -INFINITY) {  // every key so far masked: nothing to add yet
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) p[qb][kb][mm] = (bf16x8){};
        tl[qb] = 0.f;
        continue;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          uint32_t pk[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pk[e] = pack_bf16x2(__builtin_amdgcn_exp2f(sx[kb][8 * mm + 2 * e] - m),
                                __builtin_amdgcn_exp2f(sx[kb][8 * mm + 2 * e + 1] - m));
            tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), ones, tsum, false);
          }
          p[qb][kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk[0], pk[1], pk[2], pk[3]});
        }
      tl[qb] = tsum;
    }
    st.l[qb] += tl[qb];
  }
  lds_u16* vl3 = (lds_u16*)(vl);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int key = kb * 32 + 16 * g + 8 * mm + (li >> 2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int col = db * 32 + dc0 + 4 * (li & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off<D>(key, col >> 3) + (col & 4)));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off<D>(key + 4, col >> 3) + (col & 4)));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          st.o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[qb][kb][mm], st.o[qb][db], 0, 0, 0);
      }
    }
  }
}

// One 64-key tile: logits, online softmax, P V.  MASKED handles partial tiles (keys >= nvalid are
// -inf) and the optional store of the tile's logits (text tiles of the warmup emission).
template <int QB, bool MASKED, bool EXACT_SUM, int KM, int D, bool FP8 = false>
__device__ __forceinline__ void tile_step(WaveState<QB, D>& st, const uint16_t* kl, const uint16_t* vl, int kperm,
                                          int g, int li, int dc0, float c2, int nvalid, float* const (&xo)[QB],
                                          float scale, const MaskTile<KM>& mt) {
  if constexpr (!EXACT_SUM) {
    tile_step_fast<QB, MASKED, KM, D, FP8>(st, kl, vl, kperm, g, li, dc0, c2, nvalid, mt);
    return;
  }
  static_assert(KM == 0 || QB == 1, "a kept mask runs with one query block per wave");
  // scale: the logit scale in the units of s (for fp8, times the (b,h) factors of Q and K: s holds dot products
  // of the codes)
  const float inv_scale = 1.f / scale;
  // ---- S^T = K Q^T
  f32x16 s[QB][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int key = kb * 32 + kperm;
    if constexpr (FP8) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = logits_fp8<D>(kl, key, g, st.q[qb]);
      continue;
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + lds_off<D>(key, 2 * ks + g));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (ks == 0)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.q[qb][0], (f32x16){}, 0, 0, 0);
        else
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.q[qb][ks], s[qb][kb], 0, 0, 0);
      }
    }
  }
  if (MASKED) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb * 32 + 16 * g + i;
          s[qb][kb][i] = key < nvalid ? s[qb][kb][i] : -INFINITY;
        }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      if (xo[qb] != nullptr) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 16 * g + i;
            if (key < nvalid) xo[qb][key] = s[qb][kb][i] * scale;
          }
      }
  }
  if constexpr (KM != 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) mask_apply<KM>(s[0][kb], mt, kb, inv_scale);
  }

  // ---- online softmax in log2 units against the running max m.  The tile's probabilities are made
  // with the current m first; only if a lane's partial tile sum exceeds 2^16 (some logit is more
  // than 16 log2-units above m, always the case on the first tile where m = -inf, or a NaN) does the
  // wave take the exact path: recompute S from the K tile still in LDS, take the tile max, rescale O
  // and l, and remake P.  m itself stays the running max of logits seen, so probabilities are <= 2^16
  // and nothing over- or underflows; the result is the same softmax up to rounding.
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  bf16x8 p[QB][2][2];
  float tl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float mc = st.m[qb] * c2;
    float tsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][8 * mm + 2 * e], c2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][8 * mm + 2 * e + 1], c2, -mc));
          pk[e] = pack_bf16x2(p0, p1);
          if (EXACT_SUM)
            tsum += p0 + p1;
          else
            tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), ones, tsum, false);
        }
        p[qb][kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk[0], pk[1], pk[2], pk[3]});
      }
    tl[qb] = tsum;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (__any(!(tl[qb] <= 65536.f))) {
      // exact path: S again (the tile is still in LDS), tile max, rescale, P again
      f32x16 sx[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int key = kb * 32 + kperm;
        if constexpr (FP8) {
          sx[kb] = logits_fp8<D>(kl, key, g, st.q[qb]);
          continue;
        }
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + lds_off<D>(key, 2 * ks + g));
          sx[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, st.q[qb][ks], ks == 0 ? (f32x16){} : sx[kb], 0, 0, 0);
        }
      }
      if (MASKED) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sx[kb][i] = (kb * 32 + 16 * g + i) < nvalid ? sx[kb][i] : -INFINITY;
      }
      if constexpr (KM != 0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) mask_apply<KM>(sx[kb], mt, kb, inv_scale);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sx[kb][i]);
      mx = fmaxf(mx, swap_halves(mx));
      const float mnew = fmaxf(st.m[qb], mx);
      if (mnew > st.m[qb]) {
        const float alpha = __builtin_amdgcn_exp2f((st.m[qb] - mnew) * c2);
        st.l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) st.o[qb][db][i] *= alpha;
        st.m[qb] = mnew;
      }
      const float mc = st.m[qb] * c2;
      float tsum = 0.f;
      if (KM != 0 && st.m[qb] == -INFINITY) {  // every key so far masked: nothing to add yet
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) p[qb][kb][mm] = (bf16x8){};
        tl[qb] = 0.f;
        continue;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          uint32_t pk[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sx[kb][8 * mm + 2 * e], c2, -mc));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sx[kb][8 * mm + 2 * e + 1], c2, -mc));
            pk[e] = pack_bf16x2(p0, p1);
            if (EXACT_SUM)
              tsum += p0 + p1;
            else
              tsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[e]), ones, tsum, false);
          }
          p[qb][kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk[0], pk[1], pk[2], pk[3]});
        }
      tl[qb] = tsum;
    }
    st.l[qb] += tl[qb];
  }

  // ---- O^T += V^T P^T.  A operand: lane (dc + 32g) gets V[keys 16g+8mm .. +7][dc] via two
  // transposing 4x16 reads; B operand: this lane's own probabilities for those keys.
  lds_u16* vl3 = (lds_u16*)(vl);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int key = kb * 32 + 16 * g + 8 * mm + (li >> 2);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int col = db * 32 + dc0 + 4 * (li & 3);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off<D>(key, col >> 3) + (col & 4)));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off<D>(key + 4, col >> 3) + (col & 4)));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          st.o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, p[qb][kb][mm], st.o[qb][db], 0, 0, 0);
      }
    }
  }
}

template <int QB, int D>
__device__ __forceinline__ void store_lse_img(const AttnArgs& a, const WaveState<QB, D>& st, int h, const int (&row)[QB],
                                              const bool (&valid)[QB], int g, float scale) {
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = st.l[qb] + swap_halves(st.l[qb]);
    if (valid[qb] && g == 0)
      a.lse_img_out[static_cast<size_t>(h) * a.N + row[qb]] = lt > 0.f ? st.m[qb] * scale + logf(lt) : -INFINITY;
  }
}

template <bool GATHER, int QB, bool EXACT_SUM, int KM, int KS, int D, bool FP8 = false>
__global__ __launch_bounds__(kThreads * KS) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_mfma(AttnArgs a) {
  static_assert(KS == 1 || (KS == 2 && !EXACT_SUM && KM == 0), "key halves only on the mask-free fast path");
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  static_assert(!FP8 || D == 64 || QB == 1, "fp8 Q / K: one query block per wave at head dim 128");
  constexpr size_t kRowK = FP8 ? D : 2 * D;  // bytes per K row
  constexpr int kRowsW = 32 * QB;
  constexpr int kBM = kWaves * kRowsW;
  // Two LDS buffers as distinct objects: every read and every DMA target below names one of them
  // statically, so the compiler can see that the prefetch into one never aliases reads of the other
  // and does not wait for the prefetch before computing.  With KS = 2 each key half of the workgroup
  // has its own pair.
  __shared__ __attribute__((aligned(16))) uint16_t k_as[KS][kTileElems<D>];
  __shared__ __attribute__((aligned(16))) uint16_t v_as[KS][kTileElems<D>];
  __shared__ __attribute__((aligned(16))) uint16_t k_bs[KS][kTileElems<D>];
  __shared__ __attribute__((aligned(16))) uint16_t v_bs[KS][kTileElems<D>];
  // Key halves at head dim 128: each half synchronises its four waves by itself (see tile_barrier below).
  constexpr bool kHalfBarrier = KS == 2 && D == 128;
  __shared__ uint32_t half_arrivals[2];
  // key half of this wave (KS = 2: waves 0-3 take the first half of the key tiles, waves 4-7 the rest)
  const int half = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 8));
  uint16_t* const k_a = k_as[half];
  uint16_t* const v_a = v_as[half];
  uint16_t* const k_b = k_bs[half];
  uint16_t* const v_b = v_bs[half];

  const int nqt = (a.R + kBM - 1) / kBM;
  const uint32_t G = static_cast<uint32_t>(a.B) * a.H * nqt;
  const uint32_t lid = xcd_remap(blockIdx.x, G);
  // Workgroup order: the query tiles of one (b,h) in a row (they share K / V in L2), except with a kept fp32
  // mask shared by the heads: there the mask stream dominates, so groups of G heads take one query tile
  // together (each mask block read once per group), then the next tile (2560^2: 19.1 -> 17.0 ms).
  int bhi, qt;
  const int hgroup = (KM != 2 || a.mask_H != 1) ? 1 : a.H % 12 == 0 ? 12 : a.H % 8 == 0 ? 8 : a.H % 4 == 0 ? 4 : 1;
  if (hgroup > 1) {
    const uint32_t per_group = static_cast<uint32_t>(nqt) * static_cast<uint32_t>(hgroup);
    const uint32_t grp = lid / per_group, rem = lid - grp * per_group;
    qt = static_cast<int>(rem / static_cast<uint32_t>(hgroup));
    bhi = static_cast<int>(grp * hgroup + (rem - static_cast<uint32_t>(qt) * hgroup));
  } else {
    bhi = static_cast<int>(lid / nqt);
    qt = static_cast<int>(lid - static_cast<uint32_t>(bhi) * nqt);
  }
  const size_t bh = static_cast<size_t>(bhi);
  const int b = bhi / a.H, h = bhi - b * a.H;
  const int tv = a.tv[b];

  const int w = (threadIdx.x >> 6) & 3;
  const int L = threadIdx.x & 63;
  const int qi = L & 31;  // query column of the MFMA tiles owned by this lane
  const int g = L >> 5;   // lane half
  const int li = L & 15;
  const int dc0 = 16 * ((L >> 4) & 1);

  int row[QB];
  bool valid[QB];
  WaveState<QB, D> st;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = qt * kBM + w * kRowsW + qb * 32 + qi;
    const bool active = r < a.R;
    const int rr = active ? (GATHER ? a.rows[r] : r) : 0;
    valid[qb] = active && rr >= 0 && rr < a.N;
    row[qb] = valid[qb] ? rr : 0;
    if constexpr (FP8) {
      // the fp8 Q operand: bytes 64j + 32g .. 64j + 32g + 31 of the row in q[2j], q[2j + 1] (the other
      // entries of st.q stay unused)
      const uint8_t* qp8 = static_cast<const uint8_t*>(a.q) + (bh * a.N + row[qb]) * D + 32 * g;
#pragma unroll
      for (int j = 0; j < D / 64; ++j) {
        st.q[qb][2 * j] = *reinterpret_cast<const bf16x8*>(qp8 + 64 * j);
        st.q[qb][2 * j + 1] = *reinterpret_cast<const bf16x8*>(qp8 + 64 * j + 16);
      }
    } else {
      const bf16x8* qp =
          reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.q) + (bh * a.N + row[qb]) * D);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) st.q[qb][ks] = qp[2 * ks + g];
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) st.o[qb][db][i] = 0.f;
    st.m[qb] = -INFINITY;
    st.l[qb] = 0.f;
  }

  const int n_img = (a.N + kBN - 1) / kBN;
  const int n_full = a.N / kBN;  // image tiles with all 64 keys valid
  const int n_txt = (tv + kBN - 1) / kBN;
  const int ntiles = n_img + n_txt;
  // this wave's key tiles [t_begin, t_end); with two key halves under the workgroup barrier the shorter
  // half passes `pad` extra barriers so that both halves pass the same number
  int t_begin = 0, t_end = ntiles, pad = 0;
  if constexpr (KS == 2) {
    const int n0 = (ntiles + 1) >> 1;
    t_begin = half ? n0 : 0;
    t_end = half ? ntiles : n0;
    pad = half && !kHalfBarrier ? 2 * n0 - ntiles : 0;
  }
  // the warmup emission only runs on the exact-sum path (the host picks it whenever an output asks for it)
  const bool emit = EXACT_SUM && b == 0 && (a.xattn_out != nullptr || a.lse_img_out != nullptr);
  // the logit scale in the units of the dot products: for fp8 codes, times the (b,h) dequantisation factors of
  // Q and K (every logit, emitted logit, lse and mask conversion takes it)
  float scale_eff = a.scale;
  if constexpr (FP8) {
    if (a.q_descale != nullptr) scale_eff *= a.q_descale[bh];
    if (a.k_descale != nullptr) scale_eff *= a.k_descale[bh];
  }
  const float c2 = scale_eff * kLog2e;
  if constexpr (!EXACT_SUM && D == 64 && !FP8) {  // the fast path's pre-scaled Q (bf16 at head dim 64 only)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const f32x8 qf = __builtin_convertvector(st.q[qb][ks], f32x8) * c2;
        st.q[qb][ks] = __builtin_convertvector(qf, bf16x8);
      }
    }
  }
  // K rows fed to the MFMA: A-row R reads key kb*32 + 16*((R>>2)&1) + 4*(R>>3) + (R&3), which makes
  // output register r of lane half g hold key 16*g + r.
  const int kperm = 16 * ((qi >> 2) & 1) + 4 * (qi >> 3) + (qi & 3);

  // kept mask: this lane's query row of the (b, h) mask slice, tile t's first column and valid keys
  const uint8_t* mrow = nullptr;
  if constexpr (KM != 0) {
    const int mb = a.mask_B == 1 ? 0 : b, mh = a.mask_H == 1 ? 0 : h;
    mrow = static_cast<const uint8_t*>(a.mask) +
           ((static_cast<size_t>(mb) * a.mask_H + mh) * a.N + row[0]) * static_cast<size_t>(a.mask_cols) * (KM == 1 ? 1 : 4);
  }
  auto mask_fetch = [&](MaskTile<KM>& mt, int t) {
    if constexpr (KM != 0) {
      const bool txt = t >= n_img;
      const int col0 = txt ? a.N + (t - n_img) * kBN : t * kBN;
      const int nvalid = txt ? min(kBN, tv - (t - n_img) * kBN) : min(kBN, a.N - t * kBN);
      mask_load<KM>(mt, mrow, col0, nvalid, g, txt && a.mask_cols == a.N);  // image-only mask: 0 on text
    }
  };
  MaskTile<KM> mcur, mnext;
  mask_fetch(mcur, 0);

  if (t_begin < t_end) stage_issue<D, (QB > 1), FP8>(tile_src<D, FP8>(a, bh, t_begin, n_img, tv), k_a, v_a);
  if (kHalfBarrier && threadIdx.x < 2) half_arrivals[threadIdx.x] = 0u;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // End of a tile: the tile copies of every wave that reads this buffer have landed and no wave reads the
  // buffer the next copy overwrites.  Normally the workgroup barrier.  Key halves at head dim 128 (one query
  // block per wave, so a wave's matrix work and its softmax alternate instead of overlapping) use a barrier
  // of the half's four waves only: under the workgroup barrier the two waves that share a SIMD, one from
  // each half, run their matrix and their softmax phases at the same time; apart, they overlap (+7% on the
  // 1024^2 sensitive-row launch; at head dim 64 the staggered query blocks already overlap inside a wave and
  // the split barrier measured 3-6% slower).  Each wave waits for its own copies and LDS reads, adds one to
  // its half's counter and sleeps until the counter shows four arrivals per tile passed.  The halves share
  // no tile buffer, and the four waves of a half run the same tiles, so each passes the same count.
  uint32_t passed = 0;
  auto tile_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (!kHalfBarrier) {
      __syncthreads();
    } else {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (L == 0) __hip_atomic_fetch_add(&half_arrivals[half], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      passed += 4u;
      while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&half_arrivals[half], __ATOMIC_RELAXED,
                                                              __HIP_MEMORY_SCOPE_WORKGROUP)) < passed)
        __builtin_amdgcn_s_sleep(1);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  };

  float* const no_store[QB] = {};
  // One tile: prefetch tile t+1 into the other buffer, compute on this one, then wait for the
  // prefetch and synchronise.
  uint32_t coff[D / 32];
  stage_offsets<D>(coff);
  uint32_t koff8[D / 64] = {};
  if constexpr (FP8) stage8_offsets<D>(koff8);
  // this (b,h)'s image K / V bases, opaque so that they stay in scalar registers instead of being reloaded
  // from the kernel arguments (a scalar load and its wait) every tile
  const uint16_t* kimg = reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(a.k_img) + bh * a.N * kRowK);
  const uint16_t* vimg = static_cast<const uint16_t*>(a.v_img) + bh * a.N * D;
  asm volatile("" : "+s"(kimg), "+s"(vimg));
  auto full_tile = [&](int t, const uint16_t* ck, const uint16_t* cv, uint16_t* nk, uint16_t* nv) {
    if (t + 1 < t_end) {
      if (t + 1 < n_full) {
        const TileSrc src{reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(kimg) +
                                                            static_cast<size_t>(t + 1) * kBN * kRowK),
                          vimg + static_cast<size_t>(t + 1) * kBN * D, kBN};
        stage_issue_full<D, (QB > 1), FP8>(src, nk, nv, coff, koff8);
      } else {
        stage_issue<D, (QB > 1), FP8>(tile_src<D, FP8>(a, bh, t + 1, n_img, tv), nk, nv);
      }
      mask_fetch(mnext, t + 1);
    }
    tile_step<QB, false, EXACT_SUM, KM, D, FP8>(st, ck, cv, kperm, g, li, dc0, c2, kBN, no_store, scale_eff, mcur);
    tile_barrier();
    if constexpr (KM != 0) mcur = mnext;
  };
  auto masked_tile = [&](int t, const uint16_t* ck, const uint16_t* cv, uint16_t* nk, uint16_t* nv) {
    if (emit && t == n_img && a.lse_img_out != nullptr) store_lse_img(a, st, h, row, valid, g, scale_eff);
    if (t + 1 < t_end) {
      stage_issue<D, (QB > 1), FP8>(tile_src<D, FP8>(a, bh, t + 1, n_img, tv), nk, nv);
      mask_fetch(mnext, t + 1);
    }
    const bool txt = t >= n_img;
    const int nvalid = txt ? min(kBN, tv - (t - n_img) * kBN) : min(kBN, a.N - t * kBN);
    float* xo[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      xo[qb] = (emit && txt && a.xattn_out != nullptr && valid[qb])
                   ? a.xattn_out + (static_cast<size_t>(h) * a.N + row[qb]) * a.T + (t - n_img) * kBN
                   : nullptr;
    tile_step<QB, true, EXACT_SUM, KM, D, FP8>(st, ck, cv, kperm, g, li, dc0, c2, nvalid, xo, scale_eff, mcur);
    tile_barrier();
    if constexpr (KM != 0) mcur = mnext;
  };

  int t = t_begin;
  const int f_end = min(t_end, n_full);
  // ---- full image tiles, two per iteration (buffer a, then buffer b)
  for (; t + 1 < f_end; t += 2) {
    full_tile(t, k_a, v_a, k_b, v_b);
    full_tile(t + 1, k_b, v_b, k_a, v_a);
  }
  if (t < f_end) {
    full_tile(t, k_a, v_a, k_b, v_b);
    ++t;
  }
  // ---- ragged image tail and text tiles (tile t sits in buffer a when t - t_begin is even)
  for (; t < t_end; ++t) {
    const bool odd = ((t - t_begin) & 1) != 0;
    masked_tile(t, odd ? k_b : k_a, odd ? v_b : v_a, odd ? k_a : k_b, odd ? v_a : v_b);
  }
  if (emit && n_txt == 0 && a.lse_img_out != nullptr) store_lse_img(a, st, h, row, valid, g, scale_eff);

  if constexpr (KS == 2) {
    for (int i = 0; i < pad; ++i) __syncthreads();
    if constexpr (kHalfBarrier) __syncthreads();  // both halves are done with their tile buffers
    // merge the second key half into the first through LDS (the tile buffers are idle now): per query
    // block, the partner wave's running max, row sum and output accumulators, each lane with the
    // lane of the same index (same rows, same register layout).  The first half of the accumulator
    // blocks goes to k_as, the second to v_as: block db of wave w at floats [((db % nb) * 4 + w) * 16 + i][64]
    // of its array, nb = D / 64 blocks per array (each array holds exactly that); max and sum go to k_bs.
    constexpr int nb = D / 64;
    static_assert(sizeof(k_as) == sizeof(float) * nb * 4 * 16 * 64 && sizeof(v_as) == sizeof(k_as), "merge area");
    float* const xk = reinterpret_cast<float*>(&k_as[0][0]);
    float* const xv = reinterpret_cast<float*>(&v_as[0][0]);
    float* const xml = reinterpret_cast<float*>(&k_bs[0][0]);  // [4 waves][2][64]
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (half == 1) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) (db < nb ? xk : xv)[(((db % nb) * 4 + w) * 16 + i) * 64 + L] = st.o[qb][db][i];
        xml[(w * 2 + 0) * 64 + L] = st.m[qb];
        xml[(w * 2 + 1) * 64 + L] = st.l[qb];
      }
      __syncthreads();
      if (half == 0) {
        const float m1 = xml[(w * 2 + 0) * 64 + L], l1 = xml[(w * 2 + 1) * 64 + L];
        const float m0 = st.m[qb];
        const float mm = fmaxf(m0, m1);
        const float a0 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
        const float a1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
        st.m[qb] = mm;
        st.l[qb] = a0 * st.l[qb] + a1 * l1;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            st.o[qb][db][i] = a0 * st.o[qb][db][i] + a1 * (db < nb ? xk : xv)[(((db % nb) * 4 + w) * 16 + i) * 64 + L];
      }
      __syncthreads();
    }
    if (half == 1) return;
  }

  // ---- epilogue: normalise, write the output rows (scatter for gathered rows) and their lse
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = st.l[qb] + swap_halves(st.l[qb]);
    if (!valid[qb]) continue;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(a.out) + (bh * a.N + row[qb]) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int dc = db * 32 + 8 * rr + 4 * g;
        uint2 v;
        v.x = pack_bf16x2(st.o[qb][db][4 * rr + 0] * inv, st.o[qb][db][4 * rr + 1] * inv);
        v.y = pack_bf16x2(st.o[qb][db][4 * rr + 2] * inv, st.o[qb][db][4 * rr + 3] * inv);
        *reinterpret_cast<uint2*>(orow + dc) = v;
      }
    if (a.lse != nullptr && g == 0) a.lse[bh * a.N + row[qb]] = lt > 0.f ? st.m[qb] * scale_eff + logf(lt) : -INFINITY;
  }
}

template <bool GATHER, int QB, bool EXACT_SUM, int KM, int D, int KS = 1, bool FP8 = false>
static void launch(const AttnArgs& a, hipStream_t s) {
  constexpr int kBM = kWaves * 32 * QB;
  const int nqt = (a.R + kBM - 1) / kBM;
  const uint32_t grid = static_cast<uint32_t>(a.B) * a.H * nqt;
  k_attn_mfma<GATHER, QB, EXACT_SUM, KM, KS, D, FP8><<<grid, kThreads * KS, 0, s>>>(a);
}

template <bool GATHER, int QB, int KM, int D, bool FP8 = false>
static void launch_sum(const AttnArgs& a, hipStream_t s) {
  const bool exact = a.lse != nullptr || a.lse_img_out != nullptr || a.xattn_out != nullptr;
  if (exact) launch<GATHER, QB, true, KM, D, 1, FP8>(a, s);
  else launch<GATHER, QB, false, KM, D, 1, FP8>(a, s);
}

template <bool GATHER>
static void launch_rows64(const AttnArgs& a, hipStream_t s) {
  if (a.mask != nullptr) {
    // kept mask: one query block per wave (the per-lane mask chunks need the registers of the second)
    if (a.mask_dtype == SAFE_DTYPE_BOOL) launch_sum<GATHER, 1, 1, 64>(a, s);
    else launch_sum<GATHER, 1, 2, 64>(a, s);
    return;
  }
  // Work shape by the number of two-block waves w2 against the GPU's 2048 wave slots (thresholds from
  // measurements of the 1024^2 rows launch at |S| = 128 ... 2048):
  //   w2 >= 2048: two query blocks per wave;
  //   the exact-sum path, or 1024 < w2 < 2048: one query block per wave (twice the waves);
  //   512 <= w2 <= 1024 (mask-free fast path): two query blocks per wave and the key range of each
  //   workgroup split into two halves run by 8 waves, merged at the end;
  //   w2 < 512: one query block per wave with the key range split in two.
  // (An 8-wave workgroup holds a whole CU, so the split only pays while its workgroups fit in about
  // one round over the 256 CUs.)
  const double waves_qb2 = static_cast<double>(a.B) * a.H * ((a.R + 63) / 64);
  const bool exact = a.lse != nullptr || a.lse_img_out != nullptr || a.xattn_out != nullptr;
  if (waves_qb2 >= 2048.0) launch_sum<GATHER, 2, 0, 64>(a, s);
  else if (exact || waves_qb2 > 1024.0) launch_sum<GATHER, 1, 0, 64>(a, s);
  else if (waves_qb2 >= 512.0) launch<GATHER, 2, false, 0, 64, 2>(a, s);
  else launch<GATHER, 1, false, 0, 64, 2>(a, s);
}

// Head dim 128: one query block per wave throughout (the Q operand and the output accumulators of one
// block already take twice the registers of a block at head dim 64); the key range is split in two
// while the one-block waves do not fill the GPU's 2048 wave slots.
// A kept fp32 mask at head dim 128 is not taken here (its per-lane mask chunks do not fit beside the
// accumulators); the caller routes it to the generic kernel.
template <bool GATHER>
static void launch_rows128(const AttnArgs& a, hipStream_t s) {
  if (a.mask != nullptr) {
    launch_sum<GATHER, 1, 1, 128>(a, s);
    return;
  }
  const double waves_qb1 = static_cast<double>(a.B) * a.H * ((a.R + 31) / 32);
  const bool exact = a.lse != nullptr || a.lse_img_out != nullptr || a.xattn_out != nullptr;
  if (exact || waves_qb1 >= 2048.0) launch_sum<GATHER, 1, 0, 128>(a, s);
  else launch<GATHER, 1, false, 0, 128, 2>(a, s);
}

// fp8 Q / K: the work shapes of the bf16 kernel at each head dim (a kept mask and the exact-sum path with one
// query block per wave, the fast path's key split), with the fp8 logit instructions.
template <bool GATHER>
static void launch_rows64_fp8(const AttnArgs& a, hipStream_t s) {
  if (a.mask != nullptr) {
    if (a.mask_dtype == SAFE_DTYPE_BOOL) launch_sum<GATHER, 1, 1, 64, true>(a, s);
    else launch_sum<GATHER, 1, 2, 64, true>(a, s);
    return;
  }
  const double waves_qb2 = static_cast<double>(a.B) * a.H * ((a.R + 63) / 64);
  const bool exact = a.lse != nullptr || a.lse_img_out != nullptr || a.xattn_out != nullptr;
  if (waves_qb2 >= 2048.0) launch_sum<GATHER, 2, 0, 64, true>(a, s);
  else if (exact || waves_qb2 > 1024.0) launch_sum<GATHER, 1, 0, 64, true>(a, s);
  else if (waves_qb2 >= 512.0) launch<GATHER, 2, false, 0, 64, 2, true>(a, s);
  else launch<GATHER, 1, false, 0, 64, 2, true>(a, s);
}

template <bool GATHER>
static void launch_rows128_fp8(const AttnArgs& a, hipStream_t s) {
  if (a.mask != nullptr) {  // bool only (the host rejects an fp32 mask here)
    launch_sum<GATHER, 1, 1, 128, true>(a, s);
    return;
  }
  const double waves_qb1 = static_cast<double>(a.B) * a.H * ((a.R + 31) / 32);
  const bool exact = a.lse != nullptr || a.lse_img_out != nullptr || a.xattn_out != nullptr;
  if (exact || waves_qb1 >= 2048.0) launch_sum<GATHER, 1, 0, 128, true>(a, s);
  else launch<GATHER, 1, false, 0, 128, 2, true>(a, s);
}

hipError_t launch_attn_mfma_fp8(const AttnArgs& a, int d, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  if (d == 128 && a.mask != nullptr && a.mask_dtype != SAFE_DTYPE_BOOL) return hipErrorInvalidValue;
  if (d == 128) {
    if (a.rows != nullptr) launch_rows128_fp8<true>(a, s);
    else launch_rows128_fp8<false>(a, s);
  } else {
    if (a.rows != nullptr) launch_rows64_fp8<true>(a, s);
    else launch_rows64_fp8<false>(a, s);
  }
  return hipGetLastError();
}

hipError_t launch_attn_mfma_bf16(const AttnArgs& a, int d, hipStream_t s) {
  if (a.R == 0) return hipSuccess;
  if (d == 128 && a.mask != nullptr && a.mask_dtype != SAFE_DTYPE_BOOL) return hipErrorInvalidValue;
  if (d == 128) {
    if (a.rows != nullptr) launch_rows128<true>(a, s);
    else launch_rows128<false>(a, s);
  } else {
    if (a.rows != nullptr) launch_rows64<true>(a, s);
    else launch_rows64<false>(a, s);
  }
  return hipGetLastError();
}

}  // namespace safe

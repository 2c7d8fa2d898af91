// Mask-free bf16 attention for gfx950 (dense anchor rows or gathered sensitive rows).
//
// Computes, for image query rows of (b,h) -- all N rows (anchor refresh, SAFE-DiT technical summary
// Methodology 3 "CAR") or the rows of S (Methodology 3 "SRSU"; AccelAes summary B.2 SkipSparse) --
// one joint softmax over the N image keys followed by the Tv[b] valid text keys (text padding is kept
// exactly: padded slots are never loaded), and writes the output rows into the full-token state.
//
// Shape of the work (d = 64):
//  * a workgroup owns BM = 128 query rows of one (b,h): 4 waves x 32 rows;
//  * keys stream in tiles of BN = 64 through double-buffered LDS (16-byte chunks XOR-swizzled by row);
//  * per tile and wave: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys are the M dimension, queries
//    the N dimension), so every lane holds the 32 logits of one query row: lane L owns query L%32 and
//    keys 16*(L/32) + r (r = 0..15) of each 32-key block thanks to a fixed permutation of the K rows
//    fed to the MFMA;
//  * fp32 online softmax in log2 units (scale*log2(e) folded into one FMA per logit, v_exp_f32),
//    row max combined across the two lane halves with v_permlane32_swap, rescale of the output only
//    when some row's max grew;
//  * O^T += V^T P^T on the same MFMA: the P^T operand is the lane's own logits converted to bf16 (no
//    data movement), the V^T operand is read from row-major LDS with ds_read_b64_tr_b16;
//  * gathered rows: Q rows are loaded from rows[r] and outputs scattered to rows[r] in the epilogue.
// The workgroup id is remapped so that the Q tiles of one (b,h) run on the same XCD and share K/V
// in that XCD's L2.
#include "common.hpp"

namespace safe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr int kD = 64;
constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr int kTileElems = kBN * kD;

__device__ __forceinline__ float swap_halves(float x) {
  // value held by lane L ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const uint32_t lane = threadIdx.x & 63;
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// LDS element offset of (key row, 16-byte chunk) with the chunk XOR-swizzled by the row.
__device__ __forceinline__ int lds_off(int key, int chunk) { return key * kD + ((chunk ^ (key & 7)) << 3); }

struct TileSrc {
  const uint16_t* k;
  const uint16_t* v;
  int nvalid;
};

__device__ __forceinline__ TileSrc tile_src(const AttnArgs& a, size_t bh, int t, int n_img, int tv) {
  TileSrc s;
  if (t < n_img) {
    const int j0 = t * kBN;
    s.k = static_cast<const uint16_t*>(a.k_img) + (bh * a.N + j0) * kD;
    s.v = static_cast<const uint16_t*>(a.v_img) + (bh * a.N + j0) * kD;
    s.nvalid = min(kBN, a.N - j0);
  } else {
    const int j0 = (t - n_img) * kBN;
    s.k = static_cast<const uint16_t*>(a.k_txt) + (bh * a.T + j0) * kD;
    s.v = static_cast<const uint16_t*>(a.v_txt) + (bh * a.T + j0) * kD;
    s.nvalid = min(kBN, tv - j0);
  }
  return s;
}

// Each thread moves 2 K chunks and 2 V chunks (16 B each) per tile; rows past nvalid become zeros.
__device__ __forceinline__ void stage_load(uint4 (&r)[4], const TileSrc& s) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ci = threadIdx.x + kThreads * u;
    const int row = ci >> 3, c = ci & 7;
    const bool ok = row < s.nvalid;
    r[u] = ok ? *reinterpret_cast<const uint4*>(s.k + row * kD + c * 8) : make_uint4(0, 0, 0, 0);
    r[2 + u] = ok ? *reinterpret_cast<const uint4*>(s.v + row * kD + c * 8) : make_uint4(0, 0, 0, 0);
  }
}
__device__ __forceinline__ void stage_store(const uint4 (&r)[4], uint16_t* kl, uint16_t* vl) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ci = threadIdx.x + kThreads * u;
    const int row = ci >> 3, c = ci & 7;
    *reinterpret_cast<uint4*>(kl + lds_off(row, c)) = r[u];
    *reinterpret_cast<uint4*>(vl + lds_off(row, c)) = r[2 + u];
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(kThreads) void k_attn_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][kTileElems];

  const int nqt = (a.R + kBM - 1) / kBM;
  const uint32_t G = static_cast<uint32_t>(a.B) * a.H * nqt;
  const uint32_t lid = xcd_remap(blockIdx.x, G);
  const int bhi = static_cast<int>(lid / nqt);
  const int qt = static_cast<int>(lid - static_cast<uint32_t>(bhi) * nqt);
  const size_t bh = static_cast<size_t>(bhi);
  const int b = bhi / a.H, h = bhi - b * a.H;
  const int tv = a.tv[b];

  const int w = threadIdx.x >> 6;
  const int L = threadIdx.x & 63;
  const int qi = L & 31;   // query column of the MFMA tiles owned by this lane
  const int g = L >> 5;    // lane half
  const int li = L & 15;
  const int dc0 = 16 * ((L >> 4) & 1);

  const int r = qt * kBM + w * 32 + qi;
  const bool active = r < a.R;
  int row = active ? (a.rows ? a.rows[r] : r) : 0;
  const bool valid_row = active && row >= 0 && row < a.N;
  if (!valid_row) row = 0;

  // Q^T operand: lane (q + 32g) holds Q[q][16ks + 8g .. +7]
  bf16x8 qreg[4];
  {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.q) + (bh * a.N + row) * kD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qreg[ks] = qp[2 * ks + g];
  }

  const int n_img = (a.N + kBN - 1) / kBN;
  const int n_txt = (tv + kBN - 1) / kBN;
  const int ntiles = n_img + n_txt;
  const bool emit = b == 0 && (a.xattn_out != nullptr || a.lse_img_out != nullptr);
  const float c2 = a.scale * kLog2e;

  f32x16 o[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
  float m = -INFINITY, l = 0.f;

  uint4 st[4];
  {
    const TileSrc s0 = tile_src(a, bh, 0, n_img, tv);
    stage_load(st, s0);
    stage_store(st, k_lds[0], v_lds[0]);
  }
  __syncthreads();

  // K rows fed to the MFMA: A-row R reads key kb*32 + 16*((R>>2)&1) + 4*(R>>3) + (R&3), which makes
  // output register r of lane half g hold key 16*g + r.
  const int kperm = 16 * ((qi >> 2) & 1) + 4 * (qi >> 3) + (qi & 3);

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) stage_load(st, tile_src(a, bh, t + 1, n_img, tv));

    const uint16_t* kl = k_lds[buf];
    const bool txt = t >= n_img;
    const int nvalid = txt ? min(kBN, tv - (t - n_img) * kBN) : min(kBN, a.N - t * kBN);

    // ---- S^T = K Q^T
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      const int key = kb * 32 + kperm;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + lds_off(key, 2 * ks + g));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], s[kb], 0, 0, 0);
      }
    }
    if (nvalid < kBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 16 * g + i >= nvalid) s[kb][i] = -INFINITY;
    }
    if (emit && txt && a.xattn_out != nullptr && valid_row) {
      const int j0 = (t - n_img) * kBN;
      float* xo = a.xattn_out + (static_cast<size_t>(h) * a.N + row) * a.T + j0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kb * 32 + 16 * g + i < nvalid) xo[kb * 32 + 16 * g + i] = s[kb][i] * a.scale;
    }

    // ---- online softmax (log2 units)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, swap_halves(mx));
    const float mnew = fmaxf(m, mx);
    if (__any(mnew > m)) {
      const float alpha = __builtin_amdgcn_exp2f((m - mnew) * c2);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m = mnew;
    }
    const float mc = m * c2;
    bf16x8 p[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * mm + 2 * e], c2, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * mm + 2 * e + 1], c2, -mc));
          l += p0 + p1;
          pk[e] = pack_bf16x2(p0, p1);
        }
        p[kb][mm] = __builtin_bit_cast(bf16x8, (uint4){pk[0], pk[1], pk[2], pk[3]});
      }
    }

    if (emit && t == n_img - 1 && a.lse_img_out != nullptr) {
      const float lt = l + swap_halves(l);
      if (valid_row && g == 0)
        a.lse_img_out[static_cast<size_t>(h) * a.N + row] = lt > 0.f ? m * a.scale + logf(lt) : -INFINITY;
    }

    // ---- O^T += V^T P^T  (A operand: lane (dc + 32g) gets V[keys 16g+8mm .. +7][dc] via two
    // transposing 4x16 reads; B operand: this lane's own probabilities for those keys)
    {
      lds_u16* vl3 = (lds_u16*)(&v_lds[buf][0]);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int col = db * 32 + dc0 + 4 * (li & 3);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const int key = kb * 32 + 16 * g + 8 * mm + (li >> 2);
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off(key, col >> 3) + (col & 4)));
            const s16x4 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vl3 + lds_off(key + 4, col >> 3) + (col & 4)));
            const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, both), p[kb][mm], o[db], 0, 0,
                                                             0);
          }
        }
      }
    }

    if (has_next) stage_store(st, k_lds[buf ^ 1], v_lds[buf ^ 1]);
    __syncthreads();
  }

  // ---- epilogue: normalise, write the output row (scatter for gathered rows) and its lse
  const float lt = l + swap_halves(l);
  if (!valid_row) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + (bh * a.N + row) * kD;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int dc = db * 32 + 8 * rr + 4 * g;
      uint2 v;
      v.x = pack_bf16x2(o[db][4 * rr + 0] * inv, o[db][4 * rr + 1] * inv);
      v.y = pack_bf16x2(o[db][4 * rr + 2] * inv, o[db][4 * rr + 3] * inv);
      *reinterpret_cast<uint2*>(orow + dc) = v;
    }
  if (a.lse != nullptr && g == 0) a.lse[bh * a.N + row] = lt > 0.f ? m * a.scale + logf(lt) : -INFINITY;
}

hipError_t launch_attn_mfma_bf16(const AttnArgs& a, hipStream_t s) {
  const int nqt = (a.R + kBM - 1) / kBM;
  const uint32_t grid = static_cast<uint32_t>(a.B) * a.H * nqt;
  if (grid == 0) return hipSuccess;
  k_attn_mfma<<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace safe

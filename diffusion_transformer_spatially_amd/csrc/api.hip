// C ABI entry points: argument validation, dispatch to the gfx950 kernels, status mapping.
// No allocation, no retained pointers; every launch goes to the caller's stream.
#include <cmath>
#include <cstring>

#include "common.hpp"
#include "launch.hpp"

using namespace safe;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

safe_status from_hip(hipError_t e) { return e == hipSuccess ? SAFE_OK : SAFE_ERR_HIP; }

// A kept mask runs on the MFMA kernel when each lane's 16-entry mask chunks are aligned and never cross a
// mask row (N and the row length multiples of 16, 16-byte aligned base), no emission is asked (the
// emission of masked logits stays on the generic kernel) and, at head dim 128, the mask is bool (fp32
// mask chunks do not fit in registers beside a 128-dim block's accumulators); otherwise on the generic
// kernel.
bool mfma_takes_mask(const safe_attn_desc* d) {
  return d->xattn_out == nullptr && d->lse_img_out == nullptr && d->N % 16 == 0 && d->mask_cols % 16 == 0 &&
         (reinterpret_cast<uintptr_t>(d->mask) & 15u) == 0 && (d->d == 64 || d->mask_dtype == SAFE_DTYPE_BOOL);
}

safe_status check_attn(const safe_attn_desc* d) {
  if (d == nullptr) return SAFE_ERR_NULL;
  if (d->dtype != SAFE_DTYPE_BF16 && d->dtype != SAFE_DTYPE_F32 && d->dtype != SAFE_DTYPE_FP8_E4M3)
    return SAFE_ERR_DTYPE;
  if (d->B < 1 || d->H < 1 || d->N < 1 || d->T < 0 || d->d < 1) return SAFE_ERR_SHAPE;
  if (d->B > SAFE_MAX_BATCH) return SAFE_ERR_UNSUPPORTED;
  if (d->d != 64 && d->d != 128) return SAFE_ERR_UNSUPPORTED;
  if (d->q == nullptr || d->k_img == nullptr || d->v_img == nullptr || d->out == nullptr ||
      d->text_valid_len == nullptr)
    return SAFE_ERR_NULL;
  int tmax = 0;
  for (int b = 0; b < d->B; ++b) {
    const int t = d->text_valid_len[b];
    if (t < 0 || t > d->T) return SAFE_ERR_RANGE;
    tmax = t > tmax ? t : tmax;
  }
  if (tmax > 0 && (d->k_txt == nullptr || d->v_txt == nullptr)) return SAFE_ERR_NULL;
  if (!aligned16(d->q) || !aligned16(d->k_img) || !aligned16(d->v_img) || !aligned16(d->out)) return SAFE_ERR_ALIGN;
  if (tmax > 0 && (!aligned16(d->k_txt) || !aligned16(d->v_txt))) return SAFE_ERR_ALIGN;
  if (!std::isfinite(d->scale)) return SAFE_ERR_RANGE;
  // 32-bit grid and index limits of the kernels
  const double elems = static_cast<double>(d->B) * d->H * (static_cast<double>(d->N) + d->T) * d->d;
  if (elems > 4.0e12) return SAFE_ERR_SHAPE;
  if (d->mask != nullptr) {
    if (d->mask_dtype != SAFE_DTYPE_F32 && d->mask_dtype != SAFE_DTYPE_BOOL) return SAFE_ERR_DTYPE;
    if (!(d->mask_B == 1 || d->mask_B == d->B) || !(d->mask_H == 1 || d->mask_H == d->H)) return SAFE_ERR_SHAPE;
    if (!(d->mask_cols == d->N || d->mask_cols == d->N + d->T)) return SAFE_ERR_SHAPE;
    if (d->mask_dtype == SAFE_DTYPE_F32 && (reinterpret_cast<uintptr_t>(d->mask) & 3u) != 0) return SAFE_ERR_ALIGN;
  }
  if (d->dtype == SAFE_DTYPE_FP8_E4M3) {
    if ((reinterpret_cast<uintptr_t>(d->q_descale) & 3u) != 0 || (reinterpret_cast<uintptr_t>(d->k_descale) & 3u) != 0)
      return SAFE_ERR_ALIGN;
  }
  return SAFE_OK;
}

AttnArgs make_args(const safe_attn_desc* d, const int32_t* rows, int R) {
  AttnArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = d->q;
  a.k_img = d->k_img;
  a.v_img = d->v_img;
  a.k_txt = d->k_txt;
  a.v_txt = d->v_txt;
  a.out = d->out;
  a.lse = d->lse;
  a.xattn_out = d->xattn_out;
  a.lse_img_out = d->lse_img_out;
  a.rows = rows;
  a.mask = d->mask;
  a.mask_dtype = d->mask_dtype;
  a.mask_B = d->mask_B;
  a.mask_H = d->mask_H;
  a.mask_cols = d->mask_cols;
  a.q_descale = d->dtype == SAFE_DTYPE_FP8_E4M3 ? d->q_descale : nullptr;
  a.k_descale = d->dtype == SAFE_DTYPE_FP8_E4M3 ? d->k_descale : nullptr;
  a.B = d->B;
  a.H = d->H;
  a.N = d->N;
  a.T = d->T;
  a.R = R;
  a.scale = d->scale == 0.f ? 1.0f / std::sqrt(static_cast<float>(d->d)) : d->scale;
  for (int b = 0; b < d->B; ++b) a.tv[b] = d->text_valid_len[b];
  return a;
}

safe_status run_attn(const safe_attn_desc* d, const int32_t* rows, int R, hipStream_t s) {
  const AttnArgs a = make_args(d, rows, R);
  if (R == 0) return SAFE_OK;
  // bf16 and fp8: the MFMA kernel unless a kept mask is one it does not take (then the generic kernel)
  const bool mfma = d->mask == nullptr || mfma_takes_mask(d);
  if (d->dtype == SAFE_DTYPE_FP8_E4M3 && mfma) return from_hip(launch_attn_mfma_fp8(a, d->d, s));
  if (d->dtype == SAFE_DTYPE_BF16 && mfma) return from_hip(launch_attn_mfma_bf16(a, d->d, s));
  return from_hip(launch_attn_generic(a, d->dtype, d->d, s));
}

}  // namespace

extern "C" {

safe_status safe_attn_dense(const safe_attn_desc* desc, hipStream_t stream) {
  const safe_status st = check_attn(desc);
  if (st != SAFE_OK) return st;
  return run_attn(desc, nullptr, desc->N, stream);
}

safe_status safe_attn_rows(const safe_attn_desc* desc, const int32_t* rows, int32_t k, hipStream_t stream) {
  const safe_status st = check_attn(desc);
  if (st != SAFE_OK) return st;
  if (k < 0 || k > desc->N) return SAFE_ERR_RANGE;
  if (k == 0) return SAFE_OK;
  if (rows == nullptr) return SAFE_ERR_NULL;
  return run_attn(desc, rows, k, stream);
}

static safe_status mask_check_validate(const void* mask, int32_t mask_dtype, int32_t mask_B, int32_t mask_H, int32_t N,
                                       int32_t mask_cols, int32_t T, const int32_t* text_valid_len, int32_t B,
                                       const int32_t* flag_ws) {
  if (mask == nullptr || text_valid_len == nullptr || flag_ws == nullptr) return SAFE_ERR_NULL;
  if (mask_dtype != SAFE_DTYPE_F32 && mask_dtype != SAFE_DTYPE_BOOL) return SAFE_ERR_DTYPE;
  if (B < 1 || B > SAFE_MAX_BATCH || N < 1 || T < 0 || mask_H < 1) return SAFE_ERR_SHAPE;
  if (!(mask_B == 1 || mask_B == B)) return SAFE_ERR_SHAPE;
  if (!(mask_cols == N || mask_cols == N + T)) return SAFE_ERR_SHAPE;
  for (int b = 0; b < B; ++b)
    if (text_valid_len[b] < 0 || text_valid_len[b] > T) return SAFE_ERR_RANGE;
  if (static_cast<double>(mask_H) * N > 2.0e9) return SAFE_ERR_SHAPE;
  if (mask_dtype == SAFE_DTYPE_F32 && (reinterpret_cast<uintptr_t>(mask) & 3u) != 0) return SAFE_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(flag_ws) & 3u) != 0) return SAFE_ERR_ALIGN;
  return SAFE_OK;
}

safe_status safe_mask_is_row_constant(const void* mask, int32_t mask_dtype, int32_t mask_B, int32_t mask_H, int32_t N,
                                      int32_t mask_cols, int32_t T, const int32_t* text_valid_len, int32_t B,
                                      int32_t* flag_ws, int32_t* is_const, float* c_out, hipStream_t stream) {
  if (is_const == nullptr) return SAFE_ERR_NULL;
  const safe_status v = mask_check_validate(mask, mask_dtype, mask_B, mask_H, N, mask_cols, T, text_valid_len, B, flag_ws);
  if (v != SAFE_OK) return v;
  hipError_t e = launch_mask_check(mask, mask_dtype, mask_B, mask_H, N, mask_cols, T, text_valid_len, B, flag_ws,
                                   c_out, stream);
  if (e != hipSuccess) return SAFE_ERR_HIP;
  int32_t h = 0;
  e = hipMemcpyAsync(&h, flag_ws, sizeof h, hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return SAFE_ERR_HIP;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return SAFE_ERR_HIP;
  *is_const = h ? 1 : 0;
  return SAFE_OK;
}

safe_status safe_mask_check_launch(const void* mask, int32_t mask_dtype, int32_t mask_B, int32_t mask_H, int32_t N,
                                   int32_t mask_cols, int32_t T, const int32_t* text_valid_len, int32_t B,
                                   int32_t* flag_ws, float* c_out, hipStream_t stream) {
  const safe_status v = mask_check_validate(mask, mask_dtype, mask_B, mask_H, N, mask_cols, T, text_valid_len, B, flag_ws);
  if (v != SAFE_OK) return v;
  return from_hip(launch_mask_check(mask, mask_dtype, mask_B, mask_H, N, mask_cols, T, text_valid_len, B, flag_ws,
                                    c_out, stream));
}

safe_status safe_pcsp_accumulate(const float* x, const float* lse_img, int32_t H, int32_t N, int32_t T, int32_t Tv,
                                 int32_t c0, int32_t c1, float* scores, int32_t accumulate, hipStream_t stream) {
  if (x == nullptr || scores == nullptr) return SAFE_ERR_NULL;
  if (H < 1 || N < 1 || T < 1) return SAFE_ERR_SHAPE;
  if (Tv < 0 || Tv > T || c0 < 0 || c0 > c1 || c1 > Tv) return SAFE_ERR_RANGE;
  if (static_cast<double>(H) * 4 > 48.0 * 1024) return SAFE_ERR_UNSUPPORTED;  // LDS per workgroup
  if ((reinterpret_cast<uintptr_t>(x) & 3u) != 0) return SAFE_ERR_ALIGN;
  return from_hip(launch_pcsp_accumulate(x, lse_img, H, N, T, Tv, c0, c1, scores, accumulate, stream));
}

safe_status safe_affinity_accumulate(const float* x, const float* lse_img, int32_t H, int32_t N, int32_t T,
                                     int32_t Tv, const uint8_t* sel, float* scores, int32_t accumulate,
                                     hipStream_t stream) {
  if (x == nullptr || scores == nullptr || sel == nullptr) return SAFE_ERR_NULL;
  if (H < 1 || N < 1 || T < 1) return SAFE_ERR_SHAPE;
  if (Tv < 0 || Tv > T) return SAFE_ERR_RANGE;
  if (static_cast<double>(H) * 4 > 48.0 * 1024) return SAFE_ERR_UNSUPPORTED;  // LDS per workgroup
  if ((reinterpret_cast<uintptr_t>(x) & 3u) != 0) return SAFE_ERR_ALIGN;
  return from_hip(launch_affinity_accumulate(x, lse_img, H, N, T, Tv, sel, scores, accumulate, stream));
}

safe_status safe_percentile_count(int32_t N, int32_t pct_bp, int32_t* k_out) {
  if (k_out == nullptr) return SAFE_ERR_NULL;
  if (N < 0) return SAFE_ERR_SHAPE;
  if (pct_bp < 0 || pct_bp > 10000) return SAFE_ERR_RANGE;
  if (N == 0) {
    *k_out = 0;
    return SAFE_OK;
  }
  const int64_t num = static_cast<int64_t>(pct_bp) * (N - 1);  // p (N - 1) / 100 = num / 10000, exactly
  *k_out = static_cast<int32_t>(N - (num + 9999) / 10000);
  return SAFE_OK;
}

safe_status safe_stepcache_extrapolate(const float* eps_a, const float* eps_b, int64_t n, float w, float* out,
                                       hipStream_t stream) {
  if (n < 0 || n >= (int64_t(1) << 40)) return SAFE_ERR_SHAPE;
  if (n == 0) return SAFE_OK;
  if (eps_a == nullptr || eps_b == nullptr || out == nullptr) return SAFE_ERR_NULL;
  return from_hip(launch_stepcache(eps_a, eps_b, static_cast<size_t>(n), w, out, stream));
}

safe_status safe_stepcache_plan(int32_t steps, int32_t delta, int32_t* src_a, int32_t* src_b, float* w) {
  if (steps < 0 || delta < 1) return SAFE_ERR_SHAPE;
  if (steps > 0 && (src_a == nullptr || src_b == nullptr || w == nullptr)) return SAFE_ERR_NULL;
  for (int32_t s = 0; s < steps; ++s) {
    const int32_t b = delta * (s / delta);
    if (s == b) {
      src_a[s] = src_b[s] = -1;
      w[s] = 0.f;
    } else if (b == 0) {
      src_a[s] = src_b[s] = 0;
      w[s] = 0.f;
    } else {
      src_a[s] = b - delta;
      src_b[s] = b;
      w[s] = static_cast<float>(static_cast<double>(s - b) / delta);
    }
  }
  return SAFE_OK;
}

safe_status safe_trajectory_plan(int32_t steps, int32_t anchor_every, int32_t* kinds) {
  if (steps < 0 || anchor_every < 1) return SAFE_ERR_SHAPE;
  if (steps > 0 && kinds == nullptr) return SAFE_ERR_NULL;
  for (int32_t t = 0; t < steps; ++t) kinds[t] = (t % anchor_every == 0) ? SAFE_STEP_DENSE : SAFE_STEP_ROWS;
  return SAFE_OK;
}


size_t safe_rows_ffn_workspace_bytes(int32_t B, int32_t k, int32_t F) {
  if (B < 0 || k < 0 || F < 0) return 0;
  return static_cast<size_t>(B) * static_cast<size_t>(k) * static_cast<size_t>(F) * 2;
}

safe_status safe_rows_ffn(const void* x, const int32_t* rows, int32_t k, int32_t B, int32_t N, int32_t D, int32_t F,
                          const void* w1, const float* b1, const void* w2, const float* b2, void* cache, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  if (B < 1 || N < 1 || D < 1 || F < 1) return SAFE_ERR_SHAPE;
  if (k < 0 || k > N) return SAFE_ERR_RANGE;
  if (k == 0) return SAFE_OK;
  if (x == nullptr || rows == nullptr || w1 == nullptr || w2 == nullptr || cache == nullptr || ws == nullptr)
    return SAFE_ERR_NULL;
  if (D % 128 != 0 || F % 128 != 0) return SAFE_ERR_UNSUPPORTED;
  if (static_cast<double>(B) * N * D > 2.0e9 || static_cast<double>(B) * k * F > 2.0e9) return SAFE_ERR_SHAPE;
  if (ws_bytes < safe_rows_ffn_workspace_bytes(B, k, F)) return SAFE_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(cache) || !aligned16(ws) ||
      (b1 != nullptr && !aligned16(b1)) || (b2 != nullptr && !aligned16(b2)))
    return SAFE_ERR_ALIGN;
  return from_hip(launch_rows_ffn(static_cast<const uint16_t*>(x), rows, k, B, N, D, F,
                                  static_cast<const uint16_t*>(w1), b1, static_cast<const uint16_t*>(w2), b2,
                                  static_cast<uint16_t*>(cache), static_cast<uint16_t*>(ws), stream));
}

safe_status safe_rows_qkv(const void* x, const int32_t* rows, int32_t k, int32_t B, int32_t N, int32_t H, int32_t d,
                          const void* wqkv, const float* bqkv, void* q, void* k_cache, void* v_cache,
                          hipStream_t stream) {
  if (B < 1 || N < 1 || H < 1 || d < 1) return SAFE_ERR_SHAPE;
  if (k < 0 || k > N) return SAFE_ERR_RANGE;
  if (k == 0) return SAFE_OK;
  if (x == nullptr || rows == nullptr || wqkv == nullptr || q == nullptr || k_cache == nullptr || v_cache == nullptr)
    return SAFE_ERR_NULL;
  const int64_t D = static_cast<int64_t>(H) * d;
  if (D % 128 != 0 || d % 16 != 0) return SAFE_ERR_UNSUPPORTED;
  if (static_cast<double>(B) * N * D > 2.0e9) return SAFE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(wqkv) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (bqkv != nullptr && !aligned16(bqkv)))
    return SAFE_ERR_ALIGN;
  return from_hip(launch_rows_qkv(static_cast<const uint16_t*>(x), rows, k, B, N, H, d,
                                  static_cast<const uint16_t*>(wqkv), bqkv, static_cast<uint16_t*>(q),
                                  static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), stream));
}

safe_status safe_pcsp_partition(const float* scores, int32_t N, int32_t k, int32_t* S, int32_t* C, uint8_t* is_sens,
                                float* s01, hipStream_t stream) {
  if (scores == nullptr || is_sens == nullptr) return SAFE_ERR_NULL;
  if (N < 1 || N > (1 << 24)) return SAFE_ERR_SHAPE;
  if (k < 0 || k > N) return SAFE_ERR_RANGE;
  if ((k > 0 && S == nullptr) || (k < N && C == nullptr)) return SAFE_ERR_NULL;
  return from_hip(launch_pcsp_partition(scores, N, k, S, C, is_sens, s01, stream));
}

safe_status safe_swcfg_combine(const float* eps, const float* s, int32_t C, int32_t Hl, int32_t Wl, int32_t side,
                               float g_ctx, float g_sens, float* out, hipStream_t stream) {
  if (eps == nullptr || s == nullptr || out == nullptr) return SAFE_ERR_NULL;
  if (C < 1 || Hl < 1 || Wl < 1 || side < 1) return SAFE_ERR_SHAPE;
  if (Hl % side != 0 || Wl % side != 0) return SAFE_ERR_SHAPE;
  if (static_cast<double>(C) * Hl * Wl * 2 > 2.0e9) return SAFE_ERR_SHAPE;
  return from_hip(launch_swcfg(eps, s, C, Hl, Wl, side, g_ctx, g_sens, out, stream));
}

static safe_status rows_copy(const void* src, const int32_t* rows, int32_t k, int32_t B, int32_t H, int32_t N,
                             int32_t d, int32_t dtype, void* dst, bool scatter, hipStream_t stream) {
  if (dtype != SAFE_DTYPE_BF16 && dtype != SAFE_DTYPE_F32) return SAFE_ERR_DTYPE;
  if (B < 1 || H < 1 || N < 1 || d < 1) return SAFE_ERR_SHAPE;
  if (k < 0 || k > N) return SAFE_ERR_RANGE;
  if (k == 0) return SAFE_OK;
  if (src == nullptr || dst == nullptr || rows == nullptr) return SAFE_ERR_NULL;
  const int esize = dtype == SAFE_DTYPE_BF16 ? 2 : 4;
  const int row_bytes = d * esize;
  if (row_bytes % 16 != 0) return SAFE_ERR_UNSUPPORTED;
  if (!aligned16(src) || !aligned16(dst)) return SAFE_ERR_ALIGN;
  if (static_cast<double>(B) * H * k * (row_bytes / 16) > 4.0e9) return SAFE_ERR_SHAPE;
  return from_hip(launch_rows_copy(src, dst, rows, k, B, H, N, row_bytes, scatter, stream));
}

safe_status safe_gather_rows(const void* state, const int32_t* rows, int32_t k, int32_t B, int32_t H, int32_t N,
                             int32_t d, int32_t dtype, void* packed, hipStream_t stream) {
  return rows_copy(state, rows, k, B, H, N, d, dtype, packed, false, stream);
}

safe_status safe_scatter_rows(const void* packed, const int32_t* rows, int32_t k, int32_t B, int32_t H, int32_t N,
                              int32_t d, int32_t dtype, void* state, hipStream_t stream) {
  return rows_copy(packed, rows, k, B, H, N, d, dtype, state, true, stream);
}

const char* safe_status_string(safe_status s) {
  switch (s) {
    case SAFE_OK: return "SAFE_OK";
    case SAFE_ERR_NULL: return "SAFE_ERR_NULL";
    case SAFE_ERR_SHAPE: return "SAFE_ERR_SHAPE";
    case SAFE_ERR_DTYPE: return "SAFE_ERR_DTYPE";
    case SAFE_ERR_RANGE: return "SAFE_ERR_RANGE";
    case SAFE_ERR_WORKSPACE: return "SAFE_ERR_WORKSPACE";
    case SAFE_ERR_UNSUPPORTED: return "SAFE_ERR_UNSUPPORTED";
    case SAFE_ERR_HIP: return "SAFE_ERR_HIP";
    case SAFE_ERR_ALIGN: return "SAFE_ERR_ALIGN";
    default: return "SAFE_ERR_UNKNOWN";
  }
}

int32_t safe_version(void) { return 210; }

}  // extern "C"

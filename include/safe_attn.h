/*
 * safe_attn.h -- C ABI of the spatially-adaptive DiT attention step for MI355X (gfx950).
 *
 * The operations follow the SAFE-DiT technical summary (gist.science, Korean page "기술 요약:
 * SAFE-DiT" and Italian page "SAFE-DiT: Semantics-Aware Fast-path Execution for High-Resolution
 * Diffusion Transformers", Methodology 1-4) and the SkipSparse component of the AccelAes summary
 * (gist.science, Korean page, Method B.2).
 *
 * Conventions shared by every call
 * - Every tensor pointer is caller-owned DEVICE memory unless the argument says "host".  Tensors are
 *   dense, row-major, with the last dimension contiguous.  The library allocates nothing, keeps no
 *   pointer after a call returns and holds no state besides its loaded code objects (which include the
 *   fixed scratch array of safe_rows_ffn_noalloc) and the per-device address of that array.
 * - Work is enqueued on `stream` (NULL = the default stream) and is asynchronous unless stated.
 * - Arguments are validated before anything is launched.  On a validation failure a non-zero
 *   status is returned, nothing is launched and no output is written.  A launch failure returns
 *   SAFE_ERR_HIP.  Faults inside a kernel surface at the caller's next synchronisation.
 * - NaN and Inf in floating-point inputs are not checked; they propagate per IEEE.
 * - Calls are thread-safe; calls that write the same output buffer concurrently race.
 *
 * Attention notation: B batch entries (a cond/uncond pair has B = 2, entry 0 = cond), H heads, head
 * width d, N image tokens (query rows and image keys), T text slots of which the first Tv[b] are
 * valid (trailing padding).  Q, K_img, V_img, out: [B,H,N,d].  K_txt, V_txt: [B,H,T,d].
 */
#ifndef SAFE_ATTN_H
#define SAFE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t safe_status;
enum {
  SAFE_OK = 0,
  SAFE_ERR_NULL = 1,        /* a required pointer is NULL */
  SAFE_ERR_SHAPE = 2,       /* a size is out of its documented range or inconsistent */
  SAFE_ERR_DTYPE = 3,       /* unknown dtype code */
  SAFE_ERR_RANGE = 4,       /* k > N, Tv > T, c0 > c1, ... */
  SAFE_ERR_WORKSPACE = 5,   /* a workspace is missing or too small */
  SAFE_ERR_UNSUPPORTED = 6, /* valid request the library does not implement (e.g. d not 64 or 128) */
  SAFE_ERR_HIP = 7,         /* a HIP runtime call failed */
  SAFE_ERR_ALIGN = 8        /* a pointer lacks the alignment stated for it */
};

enum {
  SAFE_DTYPE_BF16 = 0,     /* bfloat16, 2 bytes */
  SAFE_DTYPE_F32 = 1,      /* float, 4 bytes */
  SAFE_DTYPE_BOOL = 2,     /* 1 byte, 0 = masked out (-inf), non-zero = kept (0) */
  SAFE_DTYPE_FP8_E4M3 = 3  /* 1 byte, OCP FP8 E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no inf, max 448) */
};

#define SAFE_MAX_BATCH 64

/*
 * Attention request (SAFE-DiT summary, Methodology 1 and 3).
 *
 * Logits of image query row i of (b,h):  L[j] = scale * q_i . k_j + M[i,j] over the keys
 *   j in [image 0..N) followed by [text 0..Tv[b]) -- one joint softmax over both blocks.
 * M is the kept mask (0 when mask == NULL).  Text slots t >= Tv[b] take no part whatever K/V hold.
 * o_i = sum_j softmax(L)_j v_j; lse_i = log sum_j exp(L_j) (natural log).  A row whose every logit
 * is -inf (possible only with a mask) gets o_i = 0 and lse_i = -inf.
 *
 * dtype           SAFE_DTYPE_BF16 or SAFE_DTYPE_F32, for q, k_*, v_*, out; or SAFE_DTYPE_FP8_E4M3: q, k_img
 *                 and k_txt are FP8 E4M3 values whose real value is the stored value times the (b,h) entry
 *                 of q_descale / k_descale, while v_img, v_txt and out are bf16 (the probabilities stay
 *                 bf16 for P V).  FP8 takes d == 64 or 128, the lse, the warmup emission and every kept
 *                 mask as bf16 does (the masks the MFMA kernel does not take -- N or the mask row length
 *                 not a multiple of 16, an unaligned mask, a mask beside the emission, an fp32 mask at
 *                 d == 128 -- run on the general kernel, which decodes the codes exactly to fp32).
 * B, H, N, T, d   1 <= B <= SAFE_MAX_BATCH, H >= 1, N >= 1, T >= 0, d == 64 or d == 128 (the head
 *                 dims of the DiT backbones the pages evaluate across; other values: SAFE_ERR_UNSUPPORTED).
 * text_valid_len  HOST array [B], 0 <= Tv[b] <= T.
 * scale           logit scale; 0 selects 1/sqrt(d).
 * mask            NULL (the mask-free fast path; use it after elision), or a kept additive mask
 *                 [mask_B, mask_H, N, mask_cols] with mask_B in {1, B}, mask_H in {1, H},
 *                 mask_cols in {N, N+T}; mask_dtype SAFE_DTYPE_F32 or SAFE_DTYPE_BOOL.  With
 *                 mask_cols == N the mask covers the image block and the text block is 0.
 *                 +inf and NaN mask entries are not supported (NaN propagates).
 * out             [B,H,N,d], same dtype as q.  Dense calls write every row; row calls only rows[].
 * lse             NULL or fp32 [B,H,N]; written for the computed rows.
 * xattn_out       NULL or fp32 [H,N,T]: for batch entry 0 and t < Tv[0], the text-block logits
 *                 L[N+t] of the computed rows (slots t >= Tv[0] are not written).
 * lse_img_out     NULL or fp32 [H,N]: for batch entry 0, log-sum-exp of the image-block logits.
 *                 These two are the warmup cross-attention responses the PCSP scores are built from.
 * q_descale       NULL (every factor 1) or device fp32 [B,H]: dequantisation factor of q per (b,h) (FP8 only).
 * k_descale       NULL or device fp32 [B,H]: the same for k_img and k_txt (FP8 only).
 * Alignment: q, k_*, v_*, out 16-byte aligned.
 */
typedef struct safe_attn_desc {
  int32_t dtype;
  int32_t B, H, N, T, d;
  const void* q;
  const void* k_img;
  const void* v_img;
  const void* k_txt;
  const void* v_txt;
  const int32_t* text_valid_len; /* host [B] */
  float scale;
  const void* mask;
  int32_t mask_dtype, mask_B, mask_H, mask_cols;
  void* out;
  float* lse;
  float* xattn_out;
  float* lse_img_out;
  const float* q_descale;
  const float* k_descale;
} safe_attn_desc;

/* Dense anchor step (CAR, SAFE-DiT summary Methodology 3): recompute all N image rows of `out`. */
safe_status safe_attn_dense(const safe_attn_desc* desc, hipStream_t stream);

/*
 * Sensitive-row step (SRSU, SAFE-DiT summary Methodology 3; SkipSparse, AccelAes summary B.2):
 * only query rows rows[0..k) attend -- still to every image key and every valid text key -- and their
 * outputs are written to out[b,h,rows[r],:] for every (b,h).  Every other row of `out` is left
 * bitwise untouched (it holds the cached context state).  rows: device int32 [k], indices in [0,N),
 * ascending and unique (the same set for every b and h); an entry outside [0,N) is skipped.  k == 0
 * is a no-op; k == N with rows = 0..N-1 equals safe_attn_dense.  0 <= k <= N.
 */
safe_status safe_attn_rows(const safe_attn_desc* desc, const int32_t* rows, int32_t k, hipStream_t stream);

/*
 * Exact mask-elision check (SAFE-DiT summary Methodology 1 and Key Contributions 2).  A mask is
 * removable when, for every slice (mb, mh) and row i, its entries over the keys that row attends to
 * -- image columns 0..N and, if mask_cols == N+T, text columns N..N+max Tv[b] over the batch
 * entries b using the slice -- are all IEEE-equal (+0 == -0) to one finite constant c_i.  With
 * mask_cols == N the implicit text block is 0, so c_i must be 0 whenever a batch entry using the
 * slice has Tv[b] > 0.  Bool entries read non-zero as 0 and zero as -inf.  No tolerance.
 *
 * mask            device [mask_B, mask_H, N, mask_cols], dtype SAFE_DTYPE_F32 or SAFE_DTYPE_BOOL.
 * text_valid_len  HOST [B].
 * flag_ws         device int32[1] scratch owned by the caller.
 * is_const        HOST out: 1 if the whole mask is removable, else 0.
 * c_out           NULL or device fp32 [mask_B*mask_H*N]: c_i per row, NaN where a row is not
 *                 constant.  When c_out is NULL the scan may stop early once a row fails.
 * SYNCHRONOUS: returns after the result is on the host (the verdict is a host dispatch decision,
 * taken once per trajectory).  Elide = call safe_attn_dense / safe_attn_rows with mask == NULL.
 */
safe_status safe_mask_is_row_constant(const void* mask, int32_t mask_dtype, int32_t mask_B, int32_t mask_H,
                                      int32_t N, int32_t mask_cols, int32_t T, const int32_t* text_valid_len,
                                      int32_t B, int32_t* flag_ws, int32_t* is_const, float* c_out,
                                      hipStream_t stream);

/*
 * The same exact elision check without the host round trip: launches the scan on `stream` and returns;
 * when the stream reaches that point, flag_ws holds the verdict (1: the mask is removable, 0: it is not)
 * and c_out (if not NULL) the per-row constants.  For callers that know the mask before they need the
 * decision (a fixed mask across the steps of a trajectory): they read flag_ws later, e.g. with an
 * asynchronous copy and an event, and the check's kernels run beside other work meanwhile.  Arguments
 * and validation as safe_mask_is_row_constant, without is_const.
 */
safe_status safe_mask_check_launch(const void* mask, int32_t mask_dtype, int32_t mask_B, int32_t mask_H, int32_t N,
                                   int32_t mask_cols, int32_t T, const int32_t* text_valid_len, int32_t B,
                                   int32_t* flag_ws, float* c_out, hipStream_t stream);

/*
 * PCSP aggregation (SAFE-DiT summary Methodology 2): attention mass from image tokens to the text
 * content slots [c0, c1), summed over heads.  For each head h and image token i,
 *   LSE = log( exp(lse_img[h,i]) + sum_{t<Tv} exp(x[h,i,t]) )      (lse_img == NULL: text only)
 *   a_i = sum_h sum_{t in [c0,c1)} exp(x[h,i,t] - LSE)
 * scores[i] = (accumulate ? scores[i] : 0) + a_i.  Repeated calls add warmup steps (and layers).
 * x: device fp32 [H,N,T] (slots t >= Tv ignored); lse_img: NULL or device fp32 [H,N];
 * 0 <= c0 <= c1 <= Tv <= T; H, N >= 1.  Deterministic: heads are summed in index order.
 */
safe_status safe_pcsp_accumulate(const float* x, const float* lse_img, int32_t H, int32_t N, int32_t T, int32_t Tv,
                                 int32_t c0, int32_t c1, float* scores, int32_t accumulate, hipStream_t stream);

/*
 * PCSP partition (SAFE-DiT summary Methodology 2): S = the k largest scores, equal scores ordered by
 * lower index, written in ascending index order; C = the other N-k indices, ascending.  NaN ranks
 * below every number, -0 equals +0.  is_sens[i] = 1 for i in S else 0.  s01 (optional) = min-max
 * normalised scores (a - min)/(max - min) over non-NaN scores, 0 when max == min (the sensitivity
 * s_i of Methodology 4).  Exact: integer selection on order-preserving keys, one workgroup.
 * scores: device fp32 [N]; S: int32 [k]; C: int32 [N-k] (may be NULL when k == N); is_sens: u8 [N];
 * s01: NULL or fp32 [N].  1 <= N <= 1<<24, 0 <= k <= N.
 */
safe_status safe_pcsp_partition(const float* scores, int32_t N, int32_t k, int32_t* S, int32_t* C,
                                uint8_t* is_sens, float* s01, hipStream_t stream);

/*
 * SW-CFG combine (SAFE-DiT summary Methodology 4; AccelAes summary B.2 spatial CFG):
 *   gamma_i = g_ctx + (g_sens - g_ctx) * s[i]
 *   out[c,y,x] = eps_u + gamma_{tok(y,x)} * (eps_c - eps_u),  tok(y,x) = (y/ph)*side + x/pw,
 * eps: device fp32 [2,C,Hl,Wl] with [0] = conditional, [1] = unconditional prediction;
 * s: device fp32 [side*side]; out: device fp32 [C,Hl,Wl] (must not alias eps).
 * Hl and Wl must be positive multiples of side (ph = Hl/side, pw = Wl/side).
 */
safe_status safe_swcfg_combine(const float* eps, const float* s, int32_t C, int32_t Hl, int32_t Wl, int32_t side,
                               float g_ctx, float g_sens, float* out, hipStream_t stream);

/*
 * Row gather / scatter of the cached state (SAFE-DiT summary Methodology 3: S rows updated in a
 * full-token state).  gather: packed[b,h,r,:] = state[b,h,rows[r],:]; scatter: the inverse, other
 * state rows untouched.  state [B,H,N,d], packed [B,H,k,d], dtype SAFE_DTYPE_BF16 or SAFE_DTYPE_F32,
 * rows device int32 [k] in [0,N) (entries outside are skipped), d*esize a multiple of 16 bytes,
 * pointers 16-byte aligned.  0 <= k <= N.
 */
safe_status safe_gather_rows(const void* state, const int32_t* rows, int32_t k, int32_t B, int32_t H, int32_t N,
                             int32_t d, int32_t dtype, void* packed, hipStream_t stream);
safe_status safe_scatter_rows(const void* packed, const int32_t* rows, int32_t k, int32_t B, int32_t H, int32_t N,
                              int32_t d, int32_t dtype, void* state, hipStream_t stream);

/*
 * AesMask affinity (AccelAes summary, 2. Methodology B.1: the attention between chosen aesthetic prompt
 * tokens and the image tokens, aggregated into an affinity map).  The PCSP quantity above with the
 * content set given by a selection of text slots instead of a range:
 *   a_i = sum_h sum_{t < Tv, sel[t] != 0} exp(x[h,i,t] - LSE),   LSE as for safe_pcsp_accumulate,
 * scores[i] = (accumulate ? scores[i] : 0) + a_i.  sel: device u8 [T] (which slots are aesthetic tokens
 * is the caller's choice); other arguments, layouts and errors as safe_pcsp_accumulate.  The binary
 * mask of the method is then safe_pcsp_partition with k from safe_percentile_count (is_sens = mask).
 */
safe_status safe_affinity_accumulate(const float* x, const float* lse_img, int32_t H, int32_t N, int32_t T,
                                     int32_t Tv, const uint8_t* sel, float* scores, int32_t accumulate,
                                     hipStream_t stream);

/*
 * Token count of a percentile threshold (AccelAes summary, Methodology B.1: the mask keeps the tokens
 * above a percentile of the affinity map).  *k_out = N - ceil(p (N - 1) / 100) with p = pct_bp / 100
 * (pct_bp in hundredths of a percent, 0..10000): for distinct scores, the number of tokens at or above
 * numpy's linearly interpolated p-th percentile.  Host only; no GPU work.  N >= 0; SAFE_ERR_RANGE for
 * pct_bp outside [0, 10000]; SAFE_ERR_NULL for k_out == NULL.
 */
safe_status safe_percentile_count(int32_t N, int32_t pct_bp, int32_t* k_out);

/*
 * StepCache extrapolation (AccelAes summary, 2. Methodology B.3: full model runs at a step interval,
 * linear extrapolation of the noise prediction in between):
 *   out[i] = eps_b[i] + w * (eps_b[i] - eps_a[i]),   i < n,
 * eps_a the older and eps_b the newer full prediction, w the step offset past eps_b in units of the
 * interval (safe_stepcache_plan gives it).  Device fp32 arrays of n elements, any layout; out may alias
 * eps_a or eps_b element for element.  n >= 0 (0: nothing is launched), n < 2^40.
 */
safe_status safe_stepcache_extrapolate(const float* eps_a, const float* eps_b, int64_t n, float w, float* out,
                                       hipStream_t stream);

/*
 * StepCache plan (AccelAes summary, Methodology B.3).  Host only.  For step s < steps: s % delta == 0
 * is a full step (src_a[s] = src_b[s] = -1, w[s] = 0); otherwise, with b = delta * (s / delta),
 * src_b[s] = b and, when b > 0, src_a[s] = b - delta and w[s] = (s - b) / delta (the line through the
 * last two full predictions), or, before the second full step, src_a[s] = b = 0 and w[s] = 0 (the one
 * full prediction reused).  Host arrays of `steps` entries; steps >= 0, delta >= 1.
 */
safe_status safe_stepcache_plan(int32_t steps, int32_t delta, int32_t* src_a, int32_t* src_b, float* w);

/*
 * Trajectory plan (SAFE-DiT summary, Methodology 2-3: after the warmup aggregation and the fixed
 * partition, periodic dense anchor refreshes and sensitive-row updates in between).  Host only.
 * kinds[t] = SAFE_STEP_DENSE when t % anchor_every == 0, else SAFE_STEP_ROWS, for t < steps (the warmup
 * steps come before step 0).  kinds: host int32 [steps]; steps >= 0, anchor_every >= 1.
 */
enum { SAFE_STEP_DENSE = 0, SAFE_STEP_ROWS = 1 };
safe_status safe_trajectory_plan(int32_t steps, int32_t anchor_every, int32_t* kinds);

/*
 * Sensitive-row FFN with the context rows cached (SAFE-DiT summary, Methodology 3: only the rows of S
 * are recomputed in a non-anchor step; AccelAes summary, Methodology B.2 SkipSparse: the FFN of the
 * background tokens is skipped and its cached output reused).  For every batch entry b and r < k:
 *   cache[b, rows[r], :] = gelu_tanh(x[b, rows[r], :] W1^T + b1) W2^T + b2,
 * other rows of cache untouched.  x: device bf16 [B, N, D] hidden states; W1: bf16 [F, D]; W2: bf16
 * [D, F] (nn.Linear layout [out, in]); b1: fp32 [F] or NULL; b2: fp32 [D] or NULL; cache: bf16 [B, N, D]
 * (may be x itself only if no later row reads a row already written: pass a separate buffer);
 * rows: device int32 [k] in [0, N) (entries outside are skipped); ws: device workspace of at least
 * safe_rows_ffn_workspace_bytes(B, k, F) bytes (the bf16 hidden activation of the k rows).
 * D and F multiples of 128; x, W1, W2, cache, ws 16-byte aligned, b1 / b2 16-byte aligned.  k = 0: no-op.
 */
safe_status safe_rows_ffn(const void* x, const int32_t* rows, int32_t k, int32_t B, int32_t N, int32_t D, int32_t F,
                          const void* w1, const float* b1, const void* w2, const float* b2, void* cache, void* ws,
                          size_t ws_bytes, hipStream_t stream);
size_t safe_rows_ffn_workspace_bytes(int32_t B, int32_t k, int32_t F);

/*
 * Sensitive-row QKV projection (SAFE-DiT summary, Methodology 3: fresh projections for the rows of S,
 * K / V of the context rows kept from the cache): y = x[b, rows[r], :] Wqkv^T + bqkv, feature j of y goes
 * to tensor j / D (0: q, 1: k_cache, 2: v_cache), head (j % D) / d, channel j % d, at row rows[r] of the
 * head-major [B, H, N, d] tensors (the layout safe_attn_* read).  x: device bf16 [B, N, D], D = H * d;
 * Wqkv: bf16 [3D, D]; bqkv: fp32 [3D] or NULL; q / k_cache / v_cache: bf16 [B, H, N, d], other rows
 * untouched.  D a multiple of 128, d a multiple of 16; pointers 16-byte aligned.  k = 0: no-op.
 */
safe_status safe_rows_qkv(const void* x, const int32_t* rows, int32_t k, int32_t B, int32_t N, int32_t H, int32_t d,
                          const void* wqkv, const float* bqkv, void* q, void* k_cache, void* v_cache,
                          hipStream_t stream);

/*
 * Allocation-free form of safe_rows_ffn, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same operation, arguments, layouts
 * and kernels as safe_rows_ffn, without the workspace: the bf16 hidden activation (B * k * F * 2 bytes) lives
 * in a fixed device array of the library, one per GPU, of safe_rows_ffn_noalloc_max_bytes() bytes (32 MiB;
 * the 1024^2 block, B = 2, k = 1229, F = 6144, needs 30.2 MB).  A larger request returns SAFE_ERR_WORKSPACE
 * and launches nothing.  The array is looked up on the current device, which must be the stream's.  Calls
 * that overlap on one GPU (other streams or threads) share the array and race; calls on different GPUs do
 * not.  The call allocates nothing (no hipMalloc, no allocating library routine); the array is reserved
 * when the library's code object is loaded on the GPU and is held until the process ends.
 */
safe_status safe_rows_ffn_noalloc(const void* x, const int32_t* rows, int32_t k, int32_t B, int32_t N, int32_t D,
                                  int32_t F, const void* w1, const float* b1, const void* w2, const float* b2,
                                  void* cache, hipStream_t stream);
size_t safe_rows_ffn_noalloc_max_bytes(void);

/* Human-readable name of a status code (static storage). */
const char* safe_status_string(safe_status s);
/* Library version: major*10000 + minor*100 + patch. */
int32_t safe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SAFE_ATTN_H */

/*
 * mla.h - C ABI of libmla: single-step MLA / GQLA decode attention on gfx950.
 *
 * Method (pages named by title and section):
 *  - "MLA and GRPO architecture", section 2, "The Mathematics of MLA": every token's
 *    keys and values come from one cached latent c_t through per-head up-projections
 *    k_t = W_UK c_t, v_t = W_UV c_t; "Decoupled Rotary Position Embeddings": a separate
 *    RoPE key k^R_t is cached beside c_t, so a cache row is [c_t ; k^R_t].
 *  - "How to upgrade GQA models to MLA...", "Under the hood", Decompression Multiplex:
 *    by associativity W_UK moves onto the query, so decode scores the query against
 *    the latent directly and the keys are never decompressed (the absorbed form).
 *  - "GQLA: Group-Query Latent Attention..." (abstract) and the AI Radio episode on it
 *    ("The paper's summary"): with up-projections shared by groups of query heads the
 *    same weights also allow a GQA path over a per-group expanded cache (per-group K and
 *    V plus the shared RoPE key); both paths give the same attention.
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers owned by the caller; the library allocates
 *    nothing and never synchronises (its only global state is the fixed scratch array of
 *    mla_decode_step_noalloc and the checked build's bad-page flag, below;
 *    mla_checked_bad_pages is its only synchronous call).  Every call is asynchronous
 *    on `stream` (0 = the null stream).  Tensors are dense, row-major, in the layouts
 *    given below; `dtype` (MLA_F32 or MLA_BF16) is the element type of q, q_abs, the
 *    caches and the weights.  Split partials, latent outputs and final outputs are fp32.
 *  - Query head h uses weight head w(h) = h / (n_heads / n_wheads): n_wheads = n_heads
 *    is MLA, n_wheads = G < n_heads is GQLA with contiguous groups.
 *  - ctx_lens[b] = T_b counts every cached token of sequence b INCLUDING its s_q new
 *    ones; query row s (0 <= s < s_q) attends to tokens 0 .. T_b - s_q + s (causal
 *    within the new tokens).  ctx_lens and page_table are device data and must satisfy
 *    0 <= T_b <= max_pages * page_size and 0 <= page_table[b][i] < num_pages for
 *    i < ceil(T_b / page_size); entries past that are never read (use -1).  libmla.so
 *    does not validate these device values: breaking them is undefined behaviour.  The
 *    checked build libmla_checked.so bounds-checks both on the device: a length outside
 *    [0, max_pages * page_size] is clamped into it and a page entry outside [0, num_pages)
 *    is replaced by page 0, and either raises the flag that mla_checked_bad_pages reports.
 *  - Split-KV: sequence b is cut into n_splits chunks.  split_tokens == 0: chunk length
 *    L_b = ceil(ceil(T_b / n_splits) / page_size) * page_size; split_tokens > 0: fixed
 *    L = split_tokens (a multiple of page_size, and n_splits * L must cover
 *    max_pages * page_size).  Chunk u covers tokens [u*L, min((u+1)*L, T_b)).  A chunk
 *    with no visible token yields o = 0 and lse = -inf.
 *  - Errors: arguments are validated on the host before any HIP call; a failing check
 *    returns its status and launches nothing.  A launch failure returns MLA_ERR_HIP.
 */
#ifndef MLA_H
#define MLA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL                                 */
  MLA_ERR_SHAPE = 2,       /* a size is non-positive or inconsistent                     */
  MLA_ERR_UNSUPPORTED = 3, /* valid but not implemented (dims, dtype, page size)         */
  MLA_ERR_HIP = 4,         /* a HIP launch or runtime call failed                        */
  MLA_ERR_TOO_LARGE = 5    /* the step's workspaces exceed mla_decode_step_noalloc's
                              fixed scratch (MLA_NOALLOC_SCRATCH_BYTES)                  */
} mla_status_t;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype_t;

typedef struct {
  int32_t batch;         /* B                                                          */
  int32_t s_q;           /* new query tokens per sequence (1, or 2 for MTP decode)     */
  int32_t n_heads;       /* query heads H                                              */
  int32_t n_wheads;      /* weight heads: H for MLA, G groups for GQLA; H % n_wheads == 0 */
  int32_t d_c;           /* latent width (512)                                         */
  int32_t d_rope;        /* decoupled RoPE key width (64)                              */
  int32_t d_nope;        /* no-position query/key head width (128)                     */
  int32_t d_v;           /* value head width (128)                                     */
  int32_t page_size;     /* tokens per cache page; must be 64                          */
  int32_t max_pages;     /* row stride of page_table                                   */
  int32_t num_pages;     /* pages in each pool                                         */
  int32_t n_splits;      /* S >= 1 split-KV chunks per sequence                         */
  int32_t split_tokens;  /* 0 = even page-aligned chunks, >0 = fixed chunk length      */
  float softmax_scale;   /* sigma applied to q.k                                      */
  mla_dtype_t dtype;     /* element type of q, q_abs, caches and weights               */
} mla_shape_t;

/* Supported dimensions: d_c, d_rope, d_nope, d_v multiples of 8 with d_c <= 1024,
 * d_c + d_rope <= 1024, d_nope + d_rope <= 1024, d_v <= 1024; page_size == 64.  The
 * bf16 shape d_c = 512, d_rope = 64 runs on the matrix-core kernels, others on the
 * generic kernels (same results up to rounding order). */

/* a1 - query absorption.
 * q_abs[b,s,h, 0:d_c]      = sum_i q[b,s,h,i] * w_uk[w(h), i, :]      (i < d_nope)
 * q_abs[b,s,h, d_c:d_c+dR] = q[b,s,h, d_nope : d_nope+d_rope]           (RoPE part copied)
 * q     [B, s_q, H, d_nope + d_rope]   dtype; RoPE part already rotated
 * w_uk  [n_wheads, d_nope, d_c]        dtype
 * q_abs [B, s_q, H, d_c + d_rope]      dtype (fp32 accumulate, one rounding to dtype)
 * Page: "How to upgrade GQA models to MLA...", Under the hood (Decompression Multiplex). */
mla_status_t mla_absorb_q(const mla_shape_t* shape, const void* q, const void* w_uk,
                          void* q_abs, hipStream_t stream);

/* a2 - absorbed decode over the paged latent cache, split-KV with online softmax.
 * For every (b, s, h) and chunk u, over the visible tokens t of u:
 *   z_t = softmax_scale * <q_abs[b,s,h], R_b[t]>,  R_b[t] = kv_pool[page_table[b][t/P], t%P]
 *   o_part[b,s,h,u,:] = sum_t softmax_u(z)_t * R_b[t][0:d_c],  lse_part = log sum_t e^{z_t}
 * q_abs      [B, s_q, H, D]        dtype, D = d_c + d_rope
 * kv_pool    [num_pages, P, D]     dtype; row = [c_t ; k^R_t]
 * page_table [B, max_pages]        int32;  ctx_lens [B] int32
 * o_part     [B, s_q, H, S, d_c]   fp32;   lse_part [B, s_q, H, S] fp32
 * Pages: "MLA and GRPO architecture" s.2 (cached state, decompression); GQLA abstract
 * and AI Radio "Key concepts" (the latent serves as shared key and value). */
mla_status_t mla_decode_absorbed(const mla_shape_t* shape, const void* q_abs,
                                 const void* kv_pool, const int32_t* page_table,
                                 const int32_t* ctx_lens, float* o_part, float* lse_part,
                                 hipStream_t stream);

/* a3 - merge split partials: lse = log sum_u e^{lse_u}, o = sum_u e^{lse_u - lse} o_u.
 * o_part [B, s_q, H, S, width] fp32, lse_part [B, s_q, H, S] fp32 ->
 * o [B, s_q, H, width] fp32, lse [B, s_q, H] fp32 (lse may be NULL).
 * width = d_c after mla_decode_absorbed, d_v after gqla_decode_gqa.  Rows whose chunks
 * are all empty give o = 0, lse = -inf.  (Log-sum-exp identity of softmax over disjoint
 * token sets; the chunking itself is not on the pages.) */
mla_status_t mla_splitkv_combine(const mla_shape_t* shape, int32_t width,
                                 const float* o_part, const float* lse_part, float* o,
                                 float* lse, hipStream_t stream);

/* a4 - value up-projection after the latent reduction.
 * out[b,s,h,:] = w_uv[w(h)] @ o_lat[b,s,h,:]
 * o_lat [B, s_q, H, d_c] fp32;  w_uv [n_wheads, d_v, d_c] dtype;  out [B, s_q, H, d_v] fp32
 * Page: "MLA and GRPO architecture" s.2 "The Mathematics of MLA" (v = W_UV c), moved
 * after the reduction by associativity. */
mla_status_t mla_out_uv(const mla_shape_t* shape, const float* o_lat, const void* w_uv,
                        float* out, hipStream_t stream);

/* a5 - GQLA GQA path over the per-group expanded cache, split-KV with online softmax.
 * Head h in group j = w(h):  z_t = softmax_scale * (<q_nope, K[t,j]> + <q_rope, kR[t]>),
 *   o_part[b,s,h,u,:] = sum_t softmax_u(z)_t V[t,j],  lse_part as in a2.
 * q       [B, s_q, H, d_nope + d_rope]     dtype
 * k_pool  [num_pages, P, G, d_nope]        dtype  (G = n_wheads)
 * v_pool  [num_pages, P, G, d_v]           dtype
 * kr_pool [num_pages, P, d_rope]           dtype
 * o_part  [B, s_q, H, S, d_v] fp32;  lse_part [B, s_q, H, S] fp32
 * Pages: GQLA abstract; AI Radio "The paper's summary" (per-group K, V and shared RoPE key). */
mla_status_t gqla_decode_gqa(const mla_shape_t* shape, const void* q, const void* k_pool,
                             const void* v_pool, const void* kr_pool,
                             const int32_t* page_table, const int32_t* ctx_lens,
                             float* o_part, float* lse_part, hipStream_t stream);

/* a6 - build the GQA path's per-group cache from the latent cache (set-up, not per step).
 * For every pool row [c ; k^R]: k_pool[p,r,j] = w_uk[j] @ c, v_pool[p,r,j] = w_uv[j] @ c,
 * kr_pool[p,r] = k^R; fp32 accumulate, rounded once to dtype.  Every row of the pool is
 * converted, padding rows included.  Shapes as in a5 / a1 / a4.  Page: AI Radio episode
 * on GQLA, "The paper's summary". */
mla_status_t gqla_expand_cache(const mla_shape_t* shape, const void* kv_pool,
                               const void* w_uk, const void* w_uv, void* k_pool,
                               void* v_pool, void* kr_pool, hipStream_t stream);

/* Cache append, the write side of a step: for every new token (b, s) at position
 * t = ctx_lens[b] - s_q + s (the last token query row s sees):
 *   c   = w_dkv @ h[b,s]                      (d_c)
 *   k^R = RoPE_t(w_kr @ h[b,s])               (d_rope; pairs (2i, 2i+1) turned by
 *                                              t * rope_base^(-2i / d_rope))
 *   kv_pool[page_table[b][t / P], t % P, :] = [c ; k^R]   (fp32 accumulate, one rounding)
 * h [B, s_q, d_model] dtype;  w_dkv [d_c, d_model] dtype;  w_kr [d_rope, d_model] dtype.
 * d_model must be a multiple of 8 (else MLA_ERR_UNSUPPORTED) and rope_base > 0.  Tokens
 * with t < 0, or whose page-table entry is negative or >= num_pages, are not written; no
 * other pool row is touched.  Pages: "MLA and GRPO architecture" s.2, "The Mathematics of
 * MLA" (c = W_DKV h) and "Decoupled Rotary Position Embeddings" (only the dedicated key is
 * rotated); the rotation convention and the key's projection are not on the pages. */
mla_status_t mla_cache_append(const mla_shape_t* shape, int32_t d_model, float rope_base,
                              const void* h, const void* w_dkv, const void* w_kr,
                              const int32_t* page_table, const int32_t* ctx_lens,
                              void* kv_pool, hipStream_t stream);

/* Projections around the path, unfolded and folded offline ("How to upgrade GQA models to
 * MLA...", Under the hood, Decompression Multiplex: by associativity W_UK is multiplied into
 * the query weights W^Q ahead of time, so the query lands in the latent space directly; the
 * value side folds W_UV into the output projection W^O the same way, which the pages do not
 * name).  All six need dtype MLA_BF16 (weights and x bf16), d_model a multiple of 256,
 * H * (d_nope + d_rope), H * (d_c + d_rope) and d_model multiples of 64, H * d_v and H * d_c
 * multiples of 256 and d_rope even (else MLA_ERR_UNSUPPORTED); fp32 accumulate.
 *   x     [B, s_q, d_model]                 hidden states of the new tokens (bf16)
 *   w_q   [H, d_nope + d_rope, d_model]     query weights, no-position rows first
 *   w_o   [d_model, H * d_v]                output projection
 * The query's RoPE rows are rotated at the token's position t = ctx_lens[b] - s_q + s with
 * the cache key's rotation (pairs (2i, 2i+1) turned by t * rope_base^(-2i / d_rope)).
 *
 * mla_project_q:        q[b,s,h] = [W^Q_nope[h] x ; RoPE_t(W^Q_rope[h] x)]  -> q [B,s_q,H,d_nope+d_rope]
 *                       bf16, the input of mla_absorb_q.
 * mla_fold_q_weights:   w_q_folded[h] = [W_UK[w(h)]^T W^Q_nope[h] ; W^Q_rope[h]]
 *                       [H, d_c + d_rope, d_model] bf16 (set-up, once per weight set).
 * mla_project_q_folded: q_abs[b,s,h] = [w_q_folded_lat[h] x ; RoPE_t(W^Q_rope[h] x)]
 *                       -> q_abs [B,s_q,H,d_c+d_rope] bf16, the input of mla_decode_absorbed
 *                       (no mla_absorb_q).
 * mla_out_project:      y[b,s] = W^O out[b,s] (out [B,s_q,H,d_v] fp32 from mla_out_uv)
 *                       -> y [B,s_q,d_model] fp32.
 * mla_fold_o_weights:   w_o_folded[:, h d_c + c] = sum_i W^O[:, h d_v + i] W_UV[w(h)][i][c]
 *                       [d_model, H * d_c] bf16 (set-up).
 * mla_out_project_folded: y[b,s] = w_o_folded o_lat[b,s] (o_lat [B,s_q,H,d_c] fp32 from
 *                       mla_splitkv_combine) -> y fp32 (no mla_out_uv).
 * y is accumulated with atomic adds over K ranges when d_model alone gives few workgroups,
 * so its last bits may differ between calls. */
mla_status_t mla_project_q(const mla_shape_t* shape, int32_t d_model, float rope_base,
                           const void* x, const void* w_q, const int32_t* ctx_lens, void* q,
                           hipStream_t stream);
mla_status_t mla_fold_q_weights(const mla_shape_t* shape, int32_t d_model, const void* w_q,
                                const void* w_uk, void* w_q_folded, hipStream_t stream);
mla_status_t mla_project_q_folded(const mla_shape_t* shape, int32_t d_model, float rope_base,
                                  const void* x, const void* w_q_folded,
                                  const int32_t* ctx_lens, void* q_abs, hipStream_t stream);
mla_status_t mla_out_project(const mla_shape_t* shape, int32_t d_model, const float* out,
                             const void* w_o, float* y, hipStream_t stream);
mla_status_t mla_fold_o_weights(const mla_shape_t* shape, int32_t d_model, const void* w_o,
                                const void* w_uv, void* w_o_folded, hipStream_t stream);
mla_status_t mla_out_project_folded(const mla_shape_t* shape, int32_t d_model,
                                    const float* o_lat, const void* w_o_folded, float* y,
                                    hipStream_t stream);

/* Whole absorbed step a1 -> a2 -> a3 -> a4 on one stream.  The caller provides the
 * workspaces: q_abs [B,s_q,H,D] dtype, o_part [B,s_q,H,S,d_c] fp32,
 * lse_part [B,s_q,H,S] fp32, o_lat [B,s_q,H,d_c] fp32.  out [B,s_q,H,d_v] fp32,
 * lse [B,s_q,H] fp32 (may be NULL).  For bf16 with d_c = 512, d_v = 128, S <= 64, H a
 * multiple of 8 and 2 H ceil(B s_q / 32) >= 256 (enough workgroups to fill the GPU), a3 and
 * a4 run as one kernel; out, lse and o_lat are bitwise those of the separate entry points
 * either way. */
mla_status_t mla_decode_step(const mla_shape_t* shape, const void* q, const void* w_uk,
                             const void* w_uv, const void* kv_pool,
                             const int32_t* page_table, const int32_t* ctx_lens,
                             void* q_abs, float* o_part, float* lse_part, float* o_lat,
                             float* out, float* lse, hipStream_t stream);

/* Size of the scratch array that mla_decode_step_noalloc uses on each device: 64 MiB. */
#define MLA_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)

/* mla_decode_step without caller workspaces, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, kernels and results as mla_decode_step (out and lse
 * bitwise equal), but q_abs, o_part, lse_part and o_lat live in one file-scope device
 * array of MLA_NOALLOC_SCRATCH_BYTES that each device running the library holds from its
 * first use until the process ends.  The workspaces, each rounded up to 256 bytes, must
 * fit: rows = B*s_q*H, rows*(d_c+d_rope)*sizeof(dtype) + rows*S*d_c*4 + rows*S*4 +
 * rows*d_c*4 <= MLA_NOALLOC_SCRATCH_BYTES, else MLA_ERR_TOO_LARGE and nothing runs
 * (e.g. B = 4, H = 128, S = 32 at bf16 takes 33.6 MiB; B = 64, s_q = 2, H = 128, S = 6
 * does not fit).  Allocates nothing: the array's device address is looked up once per
 * device (hipGetSymbolAddress, on the first call with that device current).  Every call on
 * one device shares that device's array and leaves its workspaces there: calls that
 * overlap in time on one device (different streams or host threads without ordering)
 * race and give meaningless results; calls ordered on one stream are safe. */
mla_status_t mla_decode_step_noalloc(const mla_shape_t* shape, const void* q,
                                     const void* w_uk, const void* w_uv, const void* kv_pool,
                                     const int32_t* page_table, const int32_t* ctx_lens,
                                     float* out, float* lse, hipStream_t stream);

/* Whole GQA-path step a5 -> a3 on one stream: o_part [B,s_q,H,S,d_v] and lse_part are
 * caller workspaces; out [B,s_q,H,d_v] fp32, lse [B,s_q,H] fp32 (may be NULL). */
mla_status_t gqla_decode_step(const mla_shape_t* shape, const void* q, const void* k_pool,
                              const void* v_pool, const void* kr_pool,
                              const int32_t* page_table, const int32_t* ctx_lens,
                              float* o_part, float* lse_part, float* out, float* lse,
                              hipStream_t stream);

/* Cache scalars per token and layer.  MQA-absorb / MLA: d_c + d_rope ("MLA and GRPO
 * architecture", Decoupled RoPE).  GQA path: G * (d_nope + d_v) + d_rope (AI Radio, "The
 * paper's summary").  Return -1 for a NULL or invalid shape. */
int64_t mla_cache_scalars_per_token(const mla_shape_t* shape);
int64_t gqla_cache_scalars_per_token(const mla_shape_t* shape);

/* Which kernel family a2 / a5 would run for this shape: 1 = matrix-core (MFMA) kernel,
 * 0 = generic kernel, -1 = invalid or unsupported shape.  Host-only, no HIP call. */
int32_t mla_decode_kernel_kind(const mla_shape_t* shape);
int32_t gqla_decode_kernel_kind(const mla_shape_t* shape);

/* Checked builds only.  libmla_checked.so (the same sources compiled with MLA_CHECKED)
 * bounds-checks the device data that the decode entry points (a2, a5 and the two step
 * helpers) read: a context length outside [0, max_pages * page_size] is clamped into that
 * range before it indexes the page table, and a page-table entry outside [0, num_pages) is
 * replaced by page 0, so nothing outside the table row or the pool is read.  Either sets a
 * per-device flag; the outputs of such a call are meaningless.  Returns 1 if the current
 * device's flag was set since the last call, else 0, and clears it (read and clear are one
 * atomic exchange on the device); -1 in libmla.so (no checks; such values are undefined
 * behaviour there); -2 on a HIP error.  Synchronous on the null stream: synchronize the
 * streams of the checked calls first, or a flag they raise later is reported by the next
 * query.  For callers that cannot trust their page tables or lengths (debugging). */
int32_t mla_checked_bad_pages(void);

/* Static description of a status code (never NULL). */
const char* mla_status_str(mla_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */

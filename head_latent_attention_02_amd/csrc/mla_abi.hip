// C ABI of libmla: argument validation, kernel selection and the two step helpers.
// Every check runs on the host before any HIP call; the library allocates nothing.
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "launch.hpp"
#include "mla.h"

namespace {

// The bad-page flag of checked builds (see checked_page): one word per device, set by the
// decode kernels, read and cleared by mla_checked_bad_pages.
__device__ unsigned int g_bad_pages;

// This device's flag for the kernels (checked builds), nullptr if it cannot be found.
unsigned int* bad_page_flag() {
  if (!mla::kChecked) return nullptr;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_bad_pages)) != hipSuccess) return nullptr;
  return static_cast<unsigned int*>(p);
}

constexpr int kMaxDim = 1024;

bool mult8(int v) { return v % 8 == 0; }

mla_status_t validate(const mla_shape_t* s) {
  if (!s) return MLA_ERR_NULL;
  if (s->batch <= 0 || s->s_q <= 0 || s->n_heads <= 0 || s->n_wheads <= 0 || s->d_c <= 0 ||
      s->d_rope < 0 || s->d_nope <= 0 || s->d_v <= 0 || s->page_size <= 0 ||
      s->max_pages <= 0 || s->num_pages <= 0 || s->n_splits <= 0 || s->split_tokens < 0)
    return MLA_ERR_SHAPE;
  if (s->n_heads % s->n_wheads != 0) return MLA_ERR_SHAPE;
  if (!(s->softmax_scale > 0.f) || !isfinite(s->softmax_scale)) return MLA_ERR_SHAPE;
  if (s->dtype != MLA_F32 && s->dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (s->page_size != 64) return MLA_ERR_UNSUPPORTED;
  if (!mult8(s->d_c) || !mult8(s->d_rope) || !mult8(s->d_nope) || !mult8(s->d_v))
    return MLA_ERR_UNSUPPORTED;
  if (s->d_c > kMaxDim || s->d_v > kMaxDim || s->d_c + s->d_rope > kMaxDim ||
      s->d_nope + s->d_rope > kMaxDim)
    return MLA_ERR_UNSUPPORTED;
  if (s->split_tokens > 0) {
    if (s->split_tokens % s->page_size != 0) return MLA_ERR_SHAPE;
    if (static_cast<int64_t>(s->n_splits) * s->split_tokens <
        static_cast<int64_t>(s->max_pages) * s->page_size)
      return MLA_ERR_SHAPE;
  }
  // grid dimensions used by the launchers
  if (s->batch > 65535 || (s->s_q * static_cast<int64_t>(s->n_heads) + 3) / 4 > 65535 ||
      s->n_splits > 65535)
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status_t hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

}  // namespace

extern "C" {

const char* mla_status_str(mla_status_t st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer argument";
    case MLA_ERR_SHAPE: return "invalid or inconsistent shape";
    case MLA_ERR_UNSUPPORTED: return "unsupported dimensions, dtype or page size";
    case MLA_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

int64_t mla_cache_scalars_per_token(const mla_shape_t* s) {
  if (validate(s) != MLA_OK) return -1;
  return static_cast<int64_t>(s->d_c) + s->d_rope;
}

int64_t gqla_cache_scalars_per_token(const mla_shape_t* s) {
  if (validate(s) != MLA_OK) return -1;
  return static_cast<int64_t>(s->n_wheads) * (s->d_nope + s->d_v) + s->d_rope;
}

int32_t mla_decode_kernel_kind(const mla_shape_t* s) {
  if (validate(s) != MLA_OK) return -1;
  return mla::decode_absorbed_mfma_supported(*s) ? 1 : 0;
}

int32_t gqla_decode_kernel_kind(const mla_shape_t* s) {
  if (validate(s) != MLA_OK) return -1;
  return mla::gqa_decode_mfma_supported(*s) ? 1 : 0;
}

mla_status_t mla_absorb_q(const mla_shape_t* s, const void* q, const void* w_uk, void* q_abs,
                          hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!q || !w_uk || !q_abs) return MLA_ERR_NULL;
  return hip_status(mla::launch_absorb_q(*s, q, w_uk, q_abs, stream));
}

mla_status_t mla_decode_absorbed(const mla_shape_t* s, const void* q_abs, const void* kv_pool,
                                 const int32_t* page_table, const int32_t* ctx_lens,
                                 float* o_part, float* lse_part, hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!q_abs || !kv_pool || !page_table || !ctx_lens || !o_part || !lse_part)
    return MLA_ERR_NULL;
  unsigned int* bad = bad_page_flag();
  if (mla::kChecked && !bad) return MLA_ERR_HIP;
  if (mla::decode_absorbed_mfma_supported(*s))
    return hip_status(mla::launch_decode_absorbed_mfma(*s, q_abs, kv_pool, page_table,
                                                       ctx_lens, o_part, lse_part, bad,
                                                       stream));
  return hip_status(mla::launch_decode_absorbed_generic(*s, q_abs, kv_pool, page_table,
                                                        ctx_lens, o_part, lse_part, bad,
                                                        stream));
}

mla_status_t mla_splitkv_combine(const mla_shape_t* s, int32_t width, const float* o_part,
                                 const float* lse_part, float* o, float* lse,
                                 hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!o_part || !lse_part || !o) return MLA_ERR_NULL;
  if (width <= 0) return MLA_ERR_SHAPE;
  if (width > kMaxDim) return MLA_ERR_UNSUPPORTED;
  return hip_status(mla::launch_combine(*s, width, o_part, lse_part, o, lse, stream));
}

mla_status_t mla_out_uv(const mla_shape_t* s, const float* o_lat, const void* w_uv,
                        float* out, hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  return hip_status(mla::launch_out_uv(*s, o_lat, w_uv, out, stream));
}

mla_status_t gqla_decode_gqa(const mla_shape_t* s, const void* q, const void* k_pool,
                             const void* v_pool, const void* kr_pool,
                             const int32_t* page_table, const int32_t* ctx_lens,
                             float* o_part, float* lse_part, hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!q || !k_pool || !v_pool || !page_table || !ctx_lens || !o_part || !lse_part)
    return MLA_ERR_NULL;
  if (s->d_rope > 0 && !kr_pool) return MLA_ERR_NULL;
  unsigned int* bad = bad_page_flag();
  if (mla::kChecked && !bad) return MLA_ERR_HIP;
  if (mla::gqa_decode_mfma_supported(*s))
    return hip_status(mla::launch_gqa_decode_mfma(*s, q, k_pool, v_pool, kr_pool, page_table,
                                                  ctx_lens, o_part, lse_part, bad, stream));
  return hip_status(mla::launch_gqa_decode_generic(*s, q, k_pool, v_pool, kr_pool, page_table,
                                                   ctx_lens, o_part, lse_part, bad, stream));
}

mla_status_t gqla_expand_cache(const mla_shape_t* s, const void* kv_pool, const void* w_uk,
                               const void* w_uv, void* k_pool, void* v_pool, void* kr_pool,
                               hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!kv_pool || !w_uk || !w_uv || !k_pool || !v_pool) return MLA_ERR_NULL;
  if (s->d_rope > 0 && !kr_pool) return MLA_ERR_NULL;
  return hip_status(
      mla::launch_expand_cache(*s, kv_pool, w_uk, w_uv, k_pool, v_pool, kr_pool, stream));
}

mla_status_t mla_cache_append(const mla_shape_t* s, int32_t d_model, float rope_base,
                              const void* h, const void* w_dkv, const void* w_kr,
                              const int32_t* page_table, const int32_t* ctx_lens,
                              void* kv_pool, hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!h || !w_dkv || !w_kr || !page_table || !ctx_lens || !kv_pool) return MLA_ERR_NULL;
  if (d_model <= 0 || !(rope_base > 0.f) || !isfinite(rope_base)) return MLA_ERR_SHAPE;
  if (!mult8(d_model)) return MLA_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(s->batch) * s->s_q + 7) / 8 > 65535) return MLA_ERR_UNSUPPORTED;
  return hip_status(mla::launch_cache_append(*s, d_model, rope_base, h, w_dkv, w_kr,
                                             page_table, ctx_lens, kv_pool, stream));
}

mla_status_t mla_decode_step(const mla_shape_t* s, const void* q, const void* w_uk,
                             const void* w_uv, const void* kv_pool, const int32_t* page_table,
                             const int32_t* ctx_lens, void* q_abs, float* o_part,
                             float* lse_part, float* o_lat, float* out, float* lse,
                             hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!q || !w_uk || !w_uv || !kv_pool || !page_table || !ctx_lens || !q_abs || !o_part ||
      !lse_part || !o_lat || !out)
    return MLA_ERR_NULL;
  v = mla_absorb_q(s, q, w_uk, q_abs, stream);
  if (v != MLA_OK) return v;
  v = mla_decode_absorbed(s, q_abs, kv_pool, page_table, ctx_lens, o_part, lse_part, stream);
  if (v != MLA_OK) return v;
  if (mla::combine_out_uv_supported(*s))
    return hip_status(
        mla::launch_combine_out_uv(*s, o_part, lse_part, w_uv, o_lat, lse, out, stream));
  v = mla_splitkv_combine(s, s->d_c, o_part, lse_part, o_lat, lse, stream);
  if (v != MLA_OK) return v;
  return mla_out_uv(s, o_lat, w_uv, out, stream);
}

mla_status_t gqla_decode_step(const mla_shape_t* s, const void* q, const void* k_pool,
                              const void* v_pool, const void* kr_pool,
                              const int32_t* page_table, const int32_t* ctx_lens,
                              float* o_part, float* lse_part, float* out, float* lse,
                              hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!out) return MLA_ERR_NULL;
  v = gqla_decode_gqa(s, q, k_pool, v_pool, kr_pool, page_table, ctx_lens, o_part, lse_part,
                      stream);
  if (v != MLA_OK) return v;
  return mla_splitkv_combine(s, s->d_v, o_part, lse_part, out, lse, stream);
}

}  // extern "C"

int32_t mla_checked_bad_pages(void) {
  if (!mla::kChecked) return -1;
  unsigned int v = 0;
  const unsigned int zero = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_bad_pages), sizeof(v), 0, hipMemcpyDeviceToHost) !=
      hipSuccess)
    return -2;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_bad_pages), &zero, sizeof(zero), 0,
                        hipMemcpyHostToDevice) != hipSuccess)
    return -2;
  return v ? 1 : 0;
}

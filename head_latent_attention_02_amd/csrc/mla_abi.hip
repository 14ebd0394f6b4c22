// C ABI of libmla: argument validation, kernel selection and the step helpers.
// Every check runs on the host before any HIP call; the library allocates nothing.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"
#include "mla.h"

// Workspaces of mla_decode_step_noalloc (q_abs, o_part, lse_part, o_lat of one step).
// Each device that runs the library holds its own copy until the process ends.  In host
// code this name is only a handle for hipGetSymbolAddress, never a device address.
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

// The bad-page flag of checked builds (see checked_page): one word per device, set by the
// decode kernels, read and cleared by mla_checked_bad_pages.
__device__ unsigned int g_bad_pages;
// Where mla_checked_bad_pages's kernel leaves the value it swapped out of g_bad_pages.
__device__ unsigned int g_bad_pages_taken;

// Reads and clears the flag in one atomic exchange, so a flag that a checked kernel still
// running on another stream raises is either returned now or kept for the next query.
__global__ void take_bad_pages_kernel(unsigned int* flag, unsigned int* taken) {
  *taken = atomicExch(flag, 0u);
}

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
  // grid dimensions used by the launchers: y and z extents stay within 65535, and every
  // one-dimensional grid (workgroups x threads) within 2^31 threads
  const int64_t rows = static_cast<int64_t>(s->s_q) * s->n_heads;   // query rows per sequence
  const int64_t units = static_cast<int64_t>(s->batch) * s->n_splits;
  const int64_t row_blocks = (rows + 31) / 32;
  if (s->batch > 65535 || (rows + 3) / 4 > 65535 || s->n_splits > 65535)
    return MLA_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(s->batch) * s->s_q > 262140) return MLA_ERR_UNSUPPORTED;
  if (rows * s->batch > (int64_t{1} << 24)) return MLA_ERR_UNSUPPORTED;   // merge: 128 threads/row
  const int64_t per_unit = row_blocks > s->n_wheads ? row_blocks : s->n_wheads;
  if (((units + 7) / 8) * 8 * per_unit > (int64_t{1} << 22)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status_t hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Byte offsets of the step's workspaces inside the scratch array, each rounded up to 256.
struct StepScratch {
  int64_t q_abs, o_part, lse_part, o_lat, total;
};

StepScratch step_scratch_layout(const mla_shape_t& s) {
  auto up = [](int64_t x) { return (x + 255) & ~static_cast<int64_t>(255); };
  const int64_t rows = static_cast<int64_t>(s.batch) * s.s_q * s.n_heads;
  const int64_t es = s.dtype == MLA_BF16 ? 2 : 4;
  StepScratch l;
  l.q_abs = 0;
  l.o_part = up(rows * (s.d_c + s.d_rope) * es);
  l.lse_part = l.o_part + up(rows * s.n_splits * s.d_c * 4);
  l.o_lat = l.lse_part + up(rows * s.n_splits * 4);
  l.total = l.o_lat + up(rows * s.d_c * 4);
  return l;
}

// Device address of the scratch array on each device, looked up once per device.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch array's device address on the current device.
mla_status_t current_scratch(unsigned char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
        return MLA_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = static_cast<unsigned char*>(p);
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_str(mla_status_t st) {
  switch (st) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "null pointer argument";
    case MLA_ERR_SHAPE: return "invalid or inconsistent shape";
    case MLA_ERR_UNSUPPORTED: return "unsupported dimensions, dtype or page size";
    case MLA_ERR_HIP: return "HIP launch or runtime error";
    case MLA_ERR_TOO_LARGE:
      return "workspaces exceed the fixed scratch of mla_decode_step_noalloc";
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

// The projections around the path (offline absorption): shared argument checks.
static mla_status_t validate_proj(const mla_shape_t* s, int32_t d_model) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (d_model <= 0) return MLA_ERR_SHAPE;
  if (!mla::projections_supported(*s, d_model)) return MLA_ERR_UNSUPPORTED;
  if ((static_cast<int64_t>(s->batch) * s->s_q + 31) / 32 > 65535) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

mla_status_t mla_project_q(const mla_shape_t* s, int32_t d_model, float rope_base,
                           const void* x, const void* w_q, const int32_t* ctx_lens, void* q,
                           hipStream_t stream) {
  mla_status_t v = validate_proj(s, d_model);
  if (v != MLA_OK) return v;
  if (!x || !w_q || !ctx_lens || !q) return MLA_ERR_NULL;
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return MLA_ERR_SHAPE;
  return hip_status(mla::launch_project_q(*s, d_model, rope_base, x, w_q, ctx_lens, q, false,
                                          stream));
}

mla_status_t mla_fold_q_weights(const mla_shape_t* s, int32_t d_model, const void* w_q,
                                const void* w_uk, void* w_q_folded, hipStream_t stream) {
  mla_status_t v = validate_proj(s, d_model);
  if (v != MLA_OK) return v;
  if (!w_q || !w_uk || !w_q_folded) return MLA_ERR_NULL;
  return hip_status(mla::launch_fold_q(*s, d_model, w_q, w_uk, w_q_folded, stream));
}

mla_status_t mla_project_q_folded(const mla_shape_t* s, int32_t d_model, float rope_base,
                                  const void* x, const void* w_q_folded,
                                  const int32_t* ctx_lens, void* q_abs, hipStream_t stream) {
  mla_status_t v = validate_proj(s, d_model);
  if (v != MLA_OK) return v;
  if (!x || !w_q_folded || !ctx_lens || !q_abs) return MLA_ERR_NULL;
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return MLA_ERR_SHAPE;
  return hip_status(mla::launch_project_q(*s, d_model, rope_base, x, w_q_folded, ctx_lens,
                                          q_abs, true, stream));
}

mla_status_t mla_out_project(const mla_shape_t* s, int32_t d_model, const float* out,
                             const void* w_o, float* y, hipStream_t stream) {
  mla_status_t v = validate_proj(s, d_model);
  if (v != MLA_OK) return v;
  if (!out || !w_o || !y) return MLA_ERR_NULL;
  return hip_status(mla::launch_out_project(*s, d_model, out, w_o, y, false, stream));
}

mla_status_t mla_fold_o_weights(const mla_shape_t* s, int32_t d_model, const void* w_o,
                                const void* w_uv, void* w_o_folded, hipStream_t stream) {
  mla_status_t v = validate_proj(s, d_model);
  if (v != MLA_OK) return v;
  if (!w_o || !w_uv || !w_o_folded) return MLA_ERR_NULL;
  return hip_status(mla::launch_fold_o(*s, d_model, w_o, w_uv, w_o_folded, stream));
}

mla_status_t mla_out_project_folded(const mla_shape_t* s, int32_t d_model, const float* o_lat,
                                    const void* w_o_folded, float* y, hipStream_t stream) {
  mla_status_t v = validate_proj(s, d_model);
  if (v != MLA_OK) return v;
  if (!o_lat || !w_o_folded || !y) return MLA_ERR_NULL;
  return hip_status(mla::launch_out_project(*s, d_model, o_lat, w_o_folded, y, true, stream));
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

mla_status_t mla_decode_step_noalloc(const mla_shape_t* s, const void* q, const void* w_uk,
                                     const void* w_uv, const void* kv_pool,
                                     const int32_t* page_table, const int32_t* ctx_lens,
                                     float* out, float* lse, hipStream_t stream) {
  mla_status_t v = validate(s);
  if (v != MLA_OK) return v;
  if (!q || !w_uk || !w_uv || !kv_pool || !page_table || !ctx_lens || !out)
    return MLA_ERR_NULL;
  const StepScratch l = step_scratch_layout(*s);
  if (l.total > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_TOO_LARGE;
  unsigned char* base = nullptr;
  v = current_scratch(&base);
  if (v != MLA_OK) return v;
  return mla_decode_step(s, q, w_uk, w_uv, kv_pool, page_table, ctx_lens, base + l.q_abs,
                         reinterpret_cast<float*>(base + l.o_part),
                         reinterpret_cast<float*>(base + l.lse_part),
                         reinterpret_cast<float*>(base + l.o_lat), out, lse, stream);
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
  void* flag = nullptr;
  void* taken = nullptr;
  if (hipGetSymbolAddress(&flag, HIP_SYMBOL(g_bad_pages)) != hipSuccess ||
      hipGetSymbolAddress(&taken, HIP_SYMBOL(g_bad_pages_taken)) != hipSuccess)
    return -2;
  hipLaunchKernelGGL(take_bad_pages_kernel, dim3(1), dim3(1), 0, 0,
                     static_cast<unsigned int*>(flag), static_cast<unsigned int*>(taken));
  if (hipGetLastError() != hipSuccess) return -2;
  unsigned int v = 0;
  // synchronous on the null stream: waits for the exchange kernel
  if (hipMemcpy(&v, taken, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return -2;
  return v ? 1 : 0;
}

// Host-side launchers of the kernels (one translation unit per kernel family).
// Every launcher assumes its shape has been validated by the C-ABI layer.  `bad` is the
// bad-page flag of checked builds (nullptr, and unused, in unchecked ones).
#pragma once
#include <hip/hip_runtime.h>

#include "mla.h"

namespace mla {

hipError_t launch_absorb_q(const mla_shape_t& s, const void* q, const void* w_uk,
                           void* q_abs, hipStream_t st);
hipError_t launch_decode_absorbed_generic(const mla_shape_t& s, const void* q_abs,
                                          const void* pool, const int32_t* pt,
                                          const int32_t* lens, float* o_part,
                                          float* lse_part, unsigned int* bad, hipStream_t st);
hipError_t launch_decode_absorbed_mfma(const mla_shape_t& s, const void* q_abs,
                                       const void* pool, const int32_t* pt,
                                       const int32_t* lens, float* o_part, float* lse_part,
                                       unsigned int* bad, hipStream_t st);
bool decode_absorbed_mfma_supported(const mla_shape_t& s);
hipError_t launch_combine(const mla_shape_t& s, int width, const float* o_part,
                          const float* lse_part, float* o, float* lse, hipStream_t st);
// a3 + a4 in one launch for the absorbed step (bf16, d_c 512, d_v 128, <= 64 splits);
// bitwise the same results as launch_combine followed by launch_out_uv
bool combine_out_uv_supported(const mla_shape_t& s);
hipError_t launch_combine_out_uv(const mla_shape_t& s, const float* o_part,
                                 const float* lse_part, const void* w_uv, float* o_lat,
                                 float* lse, float* out, hipStream_t st);
hipError_t launch_out_uv(const mla_shape_t& s, const float* o_lat, const void* w_uv,
                         float* out, hipStream_t st);
hipError_t launch_gqa_decode_generic(const mla_shape_t& s, const void* q, const void* k,
                                     const void* v, const void* kr, const int32_t* pt,
                                     const int32_t* lens, float* o_part, float* lse_part,
                                     unsigned int* bad, hipStream_t st);
hipError_t launch_gqa_decode_mfma(const mla_shape_t& s, const void* q, const void* k,
                                  const void* v, const void* kr, const int32_t* pt,
                                  const int32_t* lens, float* o_part, float* lse_part,
                                  unsigned int* bad, hipStream_t st);
bool gqa_decode_mfma_supported(const mla_shape_t& s);
hipError_t launch_cache_append(const mla_shape_t& s, int d_model, float rope_base,
                               const void* h, const void* w_dkv, const void* w_kr,
                               const int32_t* page_table, const int32_t* ctx_lens,
                               void* pool, hipStream_t st);
hipError_t launch_expand_cache(const mla_shape_t& s, const void* pool, const void* w_uk,
                               const void* w_uv, void* k, void* v, void* kr,
                               hipStream_t st);
// a6 on the matrix cores (bf16, d_c 512, d_nope = d_v = 128)
bool expand_cache_mfma_supported(const mla_shape_t& s);
hipError_t launch_expand_cache_mfma(const mla_shape_t& s, const void* pool, const void* w_uk,
                                    const void* w_uv, void* k, void* v, void* kr,
                                    hipStream_t st);

// the projections around the path, unfolded and folded (bf16 weights)
bool projections_supported(const mla_shape_t& s, int d_model);
hipError_t launch_project_q(const mla_shape_t& s, int d_model, float rope_base, const void* x,
                            const void* w, const int32_t* lens, void* q, bool folded,
                            hipStream_t st);
hipError_t launch_out_project(const mla_shape_t& s, int d_model, const float* in,
                              const void* w, float* y, bool folded, hipStream_t st);
hipError_t launch_fold_q(const mla_shape_t& s, int d_model, const void* w_q, const void* w_uk,
                         void* w_qf, hipStream_t st);
hipError_t launch_fold_o(const mla_shape_t& s, int d_model, const void* w_o, const void* w_uv,
                         void* w_of, hipStream_t st);

}  // namespace mla

// Cache append: the write side of the decode step.  Every new token's hidden state is
// projected down to the latent (c = W_DKV h) and to the decoupled RoPE key
// (k^R = W_KR h), the key is rotated to the token's position, and the row [c ; k^R] is
// written into its paged-cache slot ("MLA and GRPO architecture", s.2, "The Mathematics
// of MLA" and "Decoupled Rotary Position Embeddings").  The rotation turns consecutive
// pairs (2i, 2i+1) by t * base^(-2i / d_rope); the pages give no convention, this is the
// rotary embedding's own definition.
//
// A weight-read-bound GEMV: W_DKV and W_KR (D x d_model) are read once per block of
// tokens; the hidden states are small and come from L2.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kApRows = 4;      // output rows (of D = d_c + d_rope) per block
constexpr int kApTok = 8;       // tokens per block
constexpr int kApThreads = 256;

__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Block (4 output rows, 8 tokens), 256 threads.  Thread t takes the 8-element chunks t,
// t + 256, ... of the d_model axis for all 4 rows and 8 tokens; the partial dot products
// meet by wave sums and LDS.  Rows of one RoPE pair are in the same block (4-aligned,
// d_c even), so the rotation happens where both are known.
template <typename T>
__global__ __launch_bounds__(kApThreads) void cache_append_kernel(
    const T* __restrict__ h, const T* __restrict__ w_dkv, const T* __restrict__ w_kr,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ ctx_lens,
    T* __restrict__ pool, int NQ, int s_q, int d_c, int d_r, int d_model, int max_pages,
    int num_pages, int P, double log_base) {
  __shared__ float red[kApThreads / 64][kApRows * kApTok];
  __shared__ float val[kApRows * kApTok];
  const int D = d_c + d_r;
  const int o0 = kApRows * blockIdx.x, n0 = kApTok * blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* wrow[kApRows];
#pragma unroll
  for (int r = 0; r < kApRows; ++r) {
    const int o = min(o0 + r, D - 1);   // rows past D compute a copy, never stored
    wrow[r] = o < d_c ? w_dkv + static_cast<size_t>(o) * d_model
                      : w_kr + static_cast<size_t>(o - d_c) * d_model;
  }
  float acc[kApRows][kApTok];
#pragma unroll
  for (int r = 0; r < kApRows; ++r)
#pragma unroll
    for (int n = 0; n < kApTok; ++n) acc[r][n] = 0.f;
  for (int k = 8 * tid; k < d_model; k += 8 * kApThreads) {
    float w[kApRows][8];
#pragma unroll
    for (int r = 0; r < kApRows; ++r) load8(wrow[r] + k, w[r]);
#pragma unroll
    for (int n = 0; n < kApTok; ++n) {
      float x[8];
      load8(h + static_cast<size_t>(min(n0 + n, NQ - 1)) * d_model + k, x);
#pragma unroll
      for (int r = 0; r < kApRows; ++r) {
        float a = acc[r][n];
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(w[r][e], x[e], a);
        acc[r][n] = a;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kApRows; ++r)
#pragma unroll
    for (int n = 0; n < kApTok; ++n) {
      const float v = wave_sum(acc[r][n]);
      if (lane == 0) red[wave][r * kApTok + n] = v;
    }
  __syncthreads();
  if (tid < kApRows * kApTok) {
    float v = 0.f;
#pragma unroll
    for (int wv = 0; wv < kApThreads / 64; ++wv) v += red[wv][tid];
    val[tid] = v;
  }
  __syncthreads();
  if (tid >= kApRows * kApTok) return;
  const int r = tid / kApTok, n = tid - r * kApTok;
  const int o = o0 + r, q = n0 + n;
  if (o >= D || q >= NQ) return;
  const int b = q / s_q, s = q - b * s_q;
  const int t = ctx_lens[b] - s_q + s;
  if (t < 0 || t / P >= max_pages) return;
  const int page = page_table[static_cast<size_t>(b) * max_pages + t / P];
  if (page < 0 || page >= num_pages) return;
  float v = val[tid];
  if (o >= d_c) {
    // pair (x0, x1) = rows (o & ~1, o | 1) of this token; angle t * base^(-2i / d_r)
    const int i = (o - d_c) >> 1;
    const float x0 = val[(r & ~1) * kApTok + n], x1 = val[(r | 1) * kApTok + n];
    const double ang = static_cast<double>(t) * exp(-log_base * (2.0 * i) / d_r);
    const double c = cos(ang), sn = sin(ang);
    v = static_cast<float>((o & 1) ? x0 * sn + x1 * c : x0 * c - x1 * sn);
  }
  stf(pool + (static_cast<size_t>(page) * P + t % P) * D + o, v);
}

}  // namespace

hipError_t launch_cache_append(const mla_shape_t& s, int d_model, float rope_base,
                               const void* h, const void* w_dkv, const void* w_kr,
                               const int32_t* page_table, const int32_t* ctx_lens,
                               void* pool, hipStream_t st) {
  const int NQ = s.batch * s.s_q, D = s.d_c + s.d_rope;
  const dim3 grid((D + kApRows - 1) / kApRows, (NQ + kApTok - 1) / kApTok);
  const double lb = log(static_cast<double>(rope_base));
  if (s.dtype == MLA_F32)
    hipLaunchKernelGGL(cache_append_kernel<float>, grid, dim3(kApThreads), 0, st,
                       static_cast<const float*>(h), static_cast<const float*>(w_dkv),
                       static_cast<const float*>(w_kr), page_table, ctx_lens,
                       static_cast<float*>(pool), NQ, s.s_q, s.d_c, s.d_rope, d_model,
                       s.max_pages, s.num_pages, s.page_size, lb);
  else
    hipLaunchKernelGGL(cache_append_kernel<bf16_t>, grid, dim3(kApThreads), 0, st,
                       static_cast<const bf16_t*>(h), static_cast<const bf16_t*>(w_dkv),
                       static_cast<const bf16_t*>(w_kr), page_table, ctx_lens,
                       static_cast<bf16_t*>(pool), NQ, s.s_q, s.d_c, s.d_rope, d_model,
                       s.max_pages, s.num_pages, s.page_size, lb);
  return hipGetLastError();
}

}  // namespace mla

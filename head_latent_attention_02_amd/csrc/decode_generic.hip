// Generic (any supported dims, fp32 or bf16) split-KV decode kernels.
//
// One wave owns one query row (b, s, h) of one chunk u and walks the chunk's visible
// tokens in order with an online softmax: for each token it forms the score with a
// wave-wide dot product, rescales the running output when the running maximum grows,
// and accumulates the value row.  Scores are kept in the log2 domain (z * log2 e) so the
// exponentials are single v_exp_f32 instructions.  These kernels are the reference
// path for shapes the matrix-core kernels do not cover (and for fp32 workloads).
//
// Absorbed form: key = value source = the cached latent row [c ; k^R] ("MLA and GRPO
// architecture", s.2; GQLA abstract / AI Radio "Key concepts": the latent serves as a
// shared key and value).  GQA form: key = [K[t, j] ; k^R[t]], value = V[t, j] (AI Radio
// episode on GQLA, "The paper's summary").
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kMaxChunks = 16;  // D <= 1024 = 16 * 64 lanes

template <typename E>
__global__ __launch_bounds__(256) void decode_absorbed_generic_kernel(
    const E* __restrict__ q_abs, const E* __restrict__ pool, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ lens, float* __restrict__ o_part,
    float* __restrict__ lse_part, int s_q, int H, int d_c, int D, int P, int max_pages,
    int S, int split_tokens, float scale, int num_pages, unsigned int* bad) {
  const int u = blockIdx.x, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);  // row = s * H + h
  if (row >= s_q * H) return;                            // no barrier in this kernel
  const int s = row / H, h = row - s * H;
  const int n_ctx = checked_len(lens[b], max_pages * P, bad);
  int lo, hi;
  split_range(n_ctx, u, S, P, split_tokens, lo, hi);
  const int top = min(hi, n_ctx - s_q + s + 1);

  const float qscale = scale * kLog2e;
  float qr[kMaxChunks], o[kMaxChunks];
  const E* qp = q_abs + ((static_cast<size_t>(b) * s_q + s) * H + h) * D;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int k = lane + 64 * i;
    qr[i] = (k < D) ? ldf(qp + k) * qscale : 0.f;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t = lo; t < top; ++t) {
    const int page = checked_page(pt[static_cast<size_t>(b) * max_pages + t / P], num_pages, bad);
    const E* rp = pool + (static_cast<size_t>(page) * P + (t % P)) * D;
    float x[kMaxChunks];
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int k = lane + 64 * i;
      x[i] = (k < D) ? ldf(rp + k) : 0.f;
      part += qr[i] * x[i];
    }
    const float z = wave_sum(part);
    const float m_new = fmaxf(m, z);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(z - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) o[i] = o[i] * alpha + p * x[i];
    m = m_new;
  }
  const size_t orow = ((static_cast<size_t>(b) * s_q + s) * H + h) * S + u;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int k = lane + 64 * i;
    if (k < d_c) o_part[orow * d_c + k] = o[i] * inv;
  }
  if (lane == 0) lse_part[orow] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
}

template <typename E>
__global__ __launch_bounds__(256) void gqa_decode_generic_kernel(
    const E* __restrict__ q, const E* __restrict__ kp, const E* __restrict__ vp,
    const E* __restrict__ krp, const int32_t* __restrict__ pt,
    const int32_t* __restrict__ lens, float* __restrict__ o_part,
    float* __restrict__ lse_part, int s_q, int H, int G, int d_n, int d_r, int d_v, int P,
    int max_pages, int S, int split_tokens, float scale, int num_pages, unsigned int* bad) {
  const int u = blockIdx.x, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (row >= s_q * H) return;
  const int s = row / H, h = row - s * H;
  const int j = h / (H / G);
  const int n_ctx = checked_len(lens[b], max_pages * P, bad);
  int lo, hi;
  split_range(n_ctx, u, S, P, split_tokens, lo, hi);
  const int top = min(hi, n_ctx - s_q + s + 1);
  const int dq = d_n + d_r;

  const float qscale = scale * kLog2e;
  float qr[kMaxChunks], o[kMaxChunks];
  const E* qp = q + ((static_cast<size_t>(b) * s_q + s) * H + h) * dq;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int k = lane + 64 * i;
    qr[i] = (k < dq) ? ldf(qp + k) * qscale : 0.f;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int t = lo; t < top; ++t) {
    const int page = checked_page(pt[static_cast<size_t>(b) * max_pages + t / P], num_pages, bad);
    const size_t slot = static_cast<size_t>(page) * P + (t % P);
    const E* krow = kp + (slot * G + j) * d_n;
    const E* rrow = krp + slot * d_r;
    const E* vrow = vp + (slot * G + j) * d_v;
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int k = lane + 64 * i;
      const float x = (k < d_n) ? ldf(krow + k) : ((k < dq) ? ldf(rrow + (k - d_n)) : 0.f);
      part += qr[i] * x;
    }
    const float z = wave_sum(part);
    const float m_new = fmaxf(m, z);
    const float alpha = exp2f(m - m_new);
    const float p = exp2f(z - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < kMaxChunks; ++i) {
      const int k = lane + 64 * i;
      const float x = (k < d_v) ? ldf(vrow + k) : 0.f;
      o[i] = o[i] * alpha + p * x;
    }
    m = m_new;
  }
  const size_t orow = ((static_cast<size_t>(b) * s_q + s) * H + h) * S + u;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int k = lane + 64 * i;
    if (k < d_v) o_part[orow * d_v + k] = o[i] * inv;
  }
  if (lane == 0) lse_part[orow] = (l > 0.f) ? (m + log2f(l)) * kLn2 : -INFINITY;
}

}  // namespace

hipError_t launch_decode_absorbed_generic(const mla_shape_t& s, const void* q_abs,
                                          const void* pool, const int32_t* pt,
                                          const int32_t* lens, float* o_part,
                                          float* lse_part, unsigned int* bad, hipStream_t st) {
  const int D = s.d_c + s.d_rope;
  dim3 grid(s.n_splits, (s.s_q * s.n_heads + 3) / 4, s.batch);
  if (s.dtype == MLA_F32)
    hipLaunchKernelGGL(decode_absorbed_generic_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(q_abs), static_cast<const float*>(pool), pt,
                       lens, o_part, lse_part, s.s_q, s.n_heads, s.d_c, D, s.page_size,
                       s.max_pages, s.n_splits, s.split_tokens, s.softmax_scale,
                       s.num_pages, bad);
  else
    hipLaunchKernelGGL(decode_absorbed_generic_kernel<bf16_t>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(q_abs), static_cast<const bf16_t*>(pool),
                       pt, lens, o_part, lse_part, s.s_q, s.n_heads, s.d_c, D, s.page_size,
                       s.max_pages, s.n_splits, s.split_tokens, s.softmax_scale,
                       s.num_pages, bad);
  return hipGetLastError();
}

hipError_t launch_gqa_decode_generic(const mla_shape_t& s, const void* q, const void* k,
                                     const void* v, const void* kr, const int32_t* pt,
                                     const int32_t* lens, float* o_part, float* lse_part,
                                     unsigned int* bad, hipStream_t st) {
  dim3 grid(s.n_splits, (s.s_q * s.n_heads + 3) / 4, s.batch);
  if (s.dtype == MLA_F32)
    hipLaunchKernelGGL(gqa_decode_generic_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), static_cast<const float*>(kr), pt, lens,
                       o_part, lse_part, s.s_q, s.n_heads, s.n_wheads, s.d_nope, s.d_rope,
                       s.d_v, s.page_size, s.max_pages, s.n_splits, s.split_tokens,
                       s.softmax_scale, s.num_pages, bad);
  else
    hipLaunchKernelGGL(gqa_decode_generic_kernel<bf16_t>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(kr), pt,
                       lens, o_part, lse_part, s.s_q, s.n_heads, s.n_wheads, s.d_nope,
                       s.d_rope, s.d_v, s.page_size, s.max_pages, s.n_splits,
                       s.split_tokens, s.softmax_scale, s.num_pages, bad);
  return hipGetLastError();
}

}  // namespace mla

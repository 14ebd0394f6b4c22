// Query absorption (a1), split combine (a3), value up-projection (a4) and the GQA-path
// cache expansion (a6).
//
// a1: q_abs = [W_UK^T q_nope ; q_rope] - the key up-projection folded onto the query
//     ("How to upgrade GQA models to MLA...", Under the hood, Decompression Multiplex).
// a3: log-sum-exp merge of per-chunk softmax partials.
// a4: out = W_UV o_lat - the value up-projection applied once after the reduction
//     ("MLA and GRPO architecture", s.2 "The Mathematics of MLA", by associativity).
// a6: per-group K = W_UK[j] c, V = W_UV[j] c and the shared RoPE key (AI Radio episode
//     on GQLA, "The paper's summary").
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kQB = 8;  // queries per block in a1 / a4

// ---------------------------------------------------------------- a1 absorb
// Block (head h, 8 queries).  The queries' no-position parts sit in LDS as fp32; each
// thread owns latent columns c (coalesced reads of W_UK[w] rows) and keeps 8 sums.
template <typename T>
__global__ __launch_bounds__(256) void absorb_q_kernel(const T* __restrict__ q,
                                                       const T* __restrict__ w_uk,
                                                       T* __restrict__ q_abs, int NQ, int H,
                                                       int Hw, int d_n, int d_r, int d_c) {
  extern __shared__ float qs[];  // [kQB][d_n]
  const int h = blockIdx.x, q0 = blockIdx.y * kQB;
  const int w = h / (H / Hw);
  const int nq = min(kQB, NQ - q0);
  const int dq = d_n + d_r, D = d_c + d_r;
  for (int idx = threadIdx.x; idx < kQB * d_n; idx += blockDim.x) {
    const int jq = idx / d_n, i = idx - jq * d_n;
    qs[idx] = (jq < nq) ? ldf(q + (static_cast<size_t>(q0 + jq) * H + h) * dq + i) : 0.f;
  }
  __syncthreads();
  const T* W = w_uk + static_cast<size_t>(w) * d_n * d_c;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float acc[kQB];
#pragma unroll
    for (int jq = 0; jq < kQB; ++jq) acc[jq] = 0.f;
    for (int i = 0; i < d_n; ++i) {
      const float wv = ldf(W + static_cast<size_t>(i) * d_c + c);
#pragma unroll
      for (int jq = 0; jq < kQB; ++jq) acc[jq] += qs[jq * d_n + i] * wv;
    }
    for (int jq = 0; jq < nq; ++jq)
      stf(q_abs + (static_cast<size_t>(q0 + jq) * H + h) * D + c, acc[jq]);
  }
  for (int idx = threadIdx.x; idx < nq * d_r; idx += blockDim.x) {
    const int jq = idx / d_r, r = idx - jq * d_r;
    const size_t qrow = static_cast<size_t>(q0 + jq) * H + h;
    q_abs[qrow * D + d_c + r] = q[qrow * dq + d_n + r];
  }
}

// ---------------------------------------------------------------- a3 combine
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      float* __restrict__ o,
                                                      float* __restrict__ lse, int S,
                                                      int width) {
  const size_t row = blockIdx.x;
  const float* lp = lse_part + row * S;
  float m = -INFINITY;
  for (int u = 0; u < S; ++u) m = fmaxf(m, lp[u]);
  if (m == -INFINITY) {
    for (int c = threadIdx.x; c < width; c += blockDim.x) o[row * width + c] = 0.f;
    if (threadIdx.x == 0 && lse) lse[row] = -INFINITY;
    return;
  }
  float tot = 0.f;
  for (int u = 0; u < S; ++u) tot += exp2f((lp[u] - m) * kLog2e);
  const float inv = 1.f / tot;
  for (int c = threadIdx.x; c < width; c += blockDim.x) {
    float acc = 0.f;
    for (int u = 0; u < S; ++u) {
      const float wgt = exp2f((lp[u] - m) * kLog2e);
      if (wgt > 0.f) acc += wgt * o_part[(row * S + u) * width + c];
    }
    o[row * width + c] = acc * inv;
  }
  if (threadIdx.x == 0 && lse) lse[row] = m + logf(tot);
}

// ---------------------------------------------------------------- a4 out_uv
// Block (head h, 8 queries): the queries' latent outputs sit in LDS; each thread owns
// value columns v and walks its W_UV row.
template <typename T>
__global__ __launch_bounds__(256) void out_uv_kernel(const float* __restrict__ o_lat,
                                                     const T* __restrict__ w_uv,
                                                     float* __restrict__ out, int NQ, int H,
                                                     int Hw, int d_c, int d_v) {
  extern __shared__ float os[];  // [kQB][d_c]
  const int h = blockIdx.x, q0 = blockIdx.y * kQB;
  const int w = h / (H / Hw);
  const int nq = min(kQB, NQ - q0);
  for (int idx = threadIdx.x; idx < kQB * d_c; idx += blockDim.x) {
    const int jq = idx / d_c, c = idx - jq * d_c;
    os[idx] = (jq < nq) ? o_lat[(static_cast<size_t>(q0 + jq) * H + h) * d_c + c] : 0.f;
  }
  __syncthreads();
  const T* W = w_uv + static_cast<size_t>(w) * d_v * d_c;
  for (int v = threadIdx.x; v < d_v; v += blockDim.x) {
    float acc[kQB];
#pragma unroll
    for (int jq = 0; jq < kQB; ++jq) acc[jq] = 0.f;
    const T* wr = W + static_cast<size_t>(v) * d_c;
    for (int c = 0; c < d_c; ++c) {
      const float wv = ldf(wr + c);
#pragma unroll
      for (int jq = 0; jq < kQB; ++jq) acc[jq] += os[jq * d_c + c] * wv;
    }
    for (int jq = 0; jq < nq; ++jq) out[(static_cast<size_t>(q0 + jq) * H + h) * d_v + v] = acc[jq];
  }
}

// ---------------------------------------------------------------- a6 expand
// Block (page p, group j, output chunk of 128 columns of [K_j | V_j]).  The page's 64
// latent rows and the chunk's weight rows are staged through LDS 32 latent columns at a
// time; each thread owns 8 tokens x 4 outputs.
constexpr int kEC = 32;    // latent columns per stage
constexpr int kEO = 128;   // outputs per block
template <typename T>
__global__ __launch_bounds__(256) void expand_kernel(const T* __restrict__ pool,
                                                     const T* __restrict__ w_uk,
                                                     const T* __restrict__ w_uv,
                                                     T* __restrict__ kout,
                                                     T* __restrict__ vout,
                                                     T* __restrict__ krout, int P, int G,
                                                     int d_c, int d_r, int d_n, int d_v) {
  __shared__ float cs[64][kEC + 1];
  __shared__ float ws[kEO][kEC + 1];
  const int p = blockIdx.x, j = blockIdx.y, o0 = blockIdx.z * kEO;
  const int D = d_c + d_r, nout = d_n + d_v;
  const int tid = threadIdx.x;
  const int tt = tid & 7;         // tokens tt, tt+8, ..., tt+56
  const int to = tid >> 3;        // outputs to, to+32, to+64, to+96
  float acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.f;
  const T* rows = pool + static_cast<size_t>(p) * P * D;
  for (int c0 = 0; c0 < d_c; c0 += kEC) {
    for (int idx = tid; idx < 64 * kEC; idx += 256) {
      const int r = idx / kEC, c = idx - r * kEC;
      cs[r][c] = (r < P) ? ldf(rows + static_cast<size_t>(r) * D + c0 + c) : 0.f;
    }
    for (int idx = tid; idx < kEO * kEC; idx += 256) {
      const int oo = idx / kEC, c = idx - oo * kEC;
      const int og = o0 + oo;
      float wv = 0.f;
      if (og < d_n)
        wv = ldf(w_uk + (static_cast<size_t>(j) * d_n + og) * d_c + c0 + c);
      else if (og < nout)
        wv = ldf(w_uv + (static_cast<size_t>(j) * d_v + (og - d_n)) * d_c + c0 + c);
      ws[oo][c] = wv;
    }
    __syncthreads();
    for (int c = 0; c < kEC; ++c) {
      float xv[8], wv[4];
#pragma unroll
      for (int a = 0; a < 8; ++a) xv[a] = cs[tt + 8 * a][c];
#pragma unroll
      for (int b = 0; b < 4; ++b) wv[b] = ws[to + 32 * b][c];
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += xv[a] * wv[b];
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int r = tt + 8 * a;
    if (r >= P) continue;
    const size_t slot = static_cast<size_t>(p) * P + r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int og = o0 + to + 32 * b;
      if (og < d_n)
        stf(kout + (slot * G + j) * d_n + og, acc[a][b]);
      else if (og < nout)
        stf(vout + (slot * G + j) * d_v + (og - d_n), acc[a][b]);
    }
  }
  if (j == 0 && blockIdx.z == 0) {
    for (int idx = tid; idx < P * d_r; idx += 256) {
      const int r = idx / d_r, c = idx - r * d_r;
      krout[(static_cast<size_t>(p) * P + r) * d_r + c] =
          rows[static_cast<size_t>(r) * D + d_c + c];
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(const mla_shape_t& s, const void* q, const void* w_uk,
                           void* q_abs, hipStream_t st) {
  const int NQ = s.batch * s.s_q;
  dim3 grid(s.n_heads, (NQ + kQB - 1) / kQB);
  const size_t lds = sizeof(float) * kQB * s.d_nope;
  if (s.dtype == MLA_F32)
    hipLaunchKernelGGL(absorb_q_kernel<float>, grid, dim3(256), lds, st,
                       static_cast<const float*>(q), static_cast<const float*>(w_uk),
                       static_cast<float*>(q_abs), NQ, s.n_heads, s.n_wheads, s.d_nope,
                       s.d_rope, s.d_c);
  else
    hipLaunchKernelGGL(absorb_q_kernel<bf16_t>, grid, dim3(256), lds, st,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(w_uk),
                       static_cast<bf16_t*>(q_abs), NQ, s.n_heads, s.n_wheads, s.d_nope,
                       s.d_rope, s.d_c);
  return hipGetLastError();
}

hipError_t launch_combine(const mla_shape_t& s, int width, const float* o_part,
                          const float* lse_part, float* o, float* lse, hipStream_t st) {
  const unsigned rows = static_cast<unsigned>(s.batch) * s.s_q * s.n_heads;
  hipLaunchKernelGGL(combine_kernel, dim3(rows), dim3(128), 0, st, o_part, lse_part, o, lse,
                     s.n_splits, width);
  return hipGetLastError();
}

hipError_t launch_out_uv(const mla_shape_t& s, const float* o_lat, const void* w_uv,
                         float* out, hipStream_t st) {
  const int NQ = s.batch * s.s_q;
  dim3 grid(s.n_heads, (NQ + kQB - 1) / kQB);
  const size_t lds = sizeof(float) * kQB * s.d_c;
  if (s.dtype == MLA_F32)
    hipLaunchKernelGGL(out_uv_kernel<float>, grid, dim3(128), lds, st, o_lat,
                       static_cast<const float*>(w_uv), out, NQ, s.n_heads, s.n_wheads,
                       s.d_c, s.d_v);
  else
    hipLaunchKernelGGL(out_uv_kernel<bf16_t>, grid, dim3(128), lds, st, o_lat,
                       static_cast<const bf16_t*>(w_uv), out, NQ, s.n_heads, s.n_wheads,
                       s.d_c, s.d_v);
  return hipGetLastError();
}

hipError_t launch_expand_cache(const mla_shape_t& s, const void* pool, const void* w_uk,
                               const void* w_uv, void* k, void* v, void* kr,
                               hipStream_t st) {
  dim3 grid(s.num_pages, s.n_wheads, (s.d_nope + s.d_v + kEO - 1) / kEO);
  if (s.dtype == MLA_F32)
    hipLaunchKernelGGL(expand_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(pool), static_cast<const float*>(w_uk),
                       static_cast<const float*>(w_uv), static_cast<float*>(k),
                       static_cast<float*>(v), static_cast<float*>(kr), s.page_size,
                       s.n_wheads, s.d_c, s.d_rope, s.d_nope, s.d_v);
  else
    hipLaunchKernelGGL(expand_kernel<bf16_t>, grid, dim3(256), 0, st,
                       static_cast<const bf16_t*>(pool), static_cast<const bf16_t*>(w_uk),
                       static_cast<const bf16_t*>(w_uv), static_cast<bf16_t*>(k),
                       static_cast<bf16_t*>(v), static_cast<bf16_t*>(kr), s.page_size,
                       s.n_wheads, s.d_c, s.d_rope, s.d_nope, s.d_v);
  return hipGetLastError();
}

}  // namespace mla

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

// 8 consecutive elements as floats (one 16-byte load for bf16, two for fp32)
__device__ __forceinline__ void load8(const bf16_t* p, float (&x)[8]) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// ---------------------------------------------------------------- a1 absorb
// Block (head h, 256 latent columns, 8 queries), 256 threads.  Thread (rs, cl) = (tid / 32,
// tid % 32) owns columns c0 + 8 cl .. +8 and weight rows rs, rs + 8, ...: each W_UK row
// chunk is one 512-byte coalesced read per 32 lanes, and every weight byte of the block
// is read once.
constexpr int kAbsCols = 256;
template <typename T>
__global__ __launch_bounds__(256) void absorb_q_kernel(const T* __restrict__ q,
                                                       const T* __restrict__ w_uk,
                                                       T* __restrict__ q_abs, int NQ, int H,
                                                       int Hw, int d_n, int d_r, int d_c) {
  extern __shared__ float smem[];
  float* qs = smem;                       // [kQB][d_n]
  float* red = smem + kQB * d_n;          // [4 waves][kQB][kAbsCols]
  const int h = blockIdx.x, c0 = blockIdx.y * kAbsCols, q0 = blockIdx.z * kQB;
  const int w = h / (H / Hw);
  const int nq = min(kQB, NQ - q0);
  const int dq = d_n + d_r, D = d_c + d_r;
  const int tid = threadIdx.x, rs = tid >> 5, cl = tid & 31;
  for (int idx = tid; idx < kQB * d_n; idx += blockDim.x) {
    const int jq = idx / d_n, i = idx - jq * d_n;
    qs[idx] = (jq < nq) ? ldf(q + (static_cast<size_t>(q0 + jq) * H + h) * dq + i) : 0.f;
  }
  __syncthreads();
  const int c = c0 + 8 * cl;
  float acc[kQB][8];
#pragma unroll
  for (int jq = 0; jq < kQB; ++jq)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[jq][e] = 0.f;
  if (c < d_c) {
    const T* W = w_uk + static_cast<size_t>(w) * d_n * d_c + c;
    // all of a thread's weight loads are issued back to back (16 in flight at d_n = 128)
#pragma unroll 16
    for (int i = rs; i < d_n; i += 8) {
      float wv[8];
      load8(W + static_cast<size_t>(i) * d_c, wv);
#pragma unroll
      for (int jq = 0; jq < kQB; ++jq) {
        const float qv = qs[jq * d_n + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[jq][e] = fmaf(qv, wv[e], acc[jq][e]);
      }
    }
  }
  // the two row slices of a wave (lane halves) meet by a shuffle, the 4 waves in LDS
#pragma unroll
  for (int jq = 0; jq < kQB; ++jq)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[jq][e] += __shfl_xor(acc[jq][e], 32, 64);
  if ((rs & 1) == 0) {
#pragma unroll
    for (int jq = 0; jq < kQB; ++jq)
#pragma unroll
      for (int e = 0; e < 8; e += 4)
        *reinterpret_cast<float4*>(&red[((rs >> 1) * kQB + jq) * kAbsCols + 8 * cl + e]) =
            make_float4(acc[jq][e], acc[jq][e + 1], acc[jq][e + 2], acc[jq][e + 3]);
  }
  __syncthreads();
  for (int idx = tid; idx < kQB * kAbsCols; idx += blockDim.x) {
    const int jq = idx / kAbsCols, cc = idx - jq * kAbsCols;
    if (jq >= nq || c0 + cc >= d_c) continue;
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) v += red[(r * kQB + jq) * kAbsCols + cc];
    stf(q_abs + (static_cast<size_t>(q0 + jq) * H + h) * D + c0 + cc, v);
  }
  if (blockIdx.y == 0) {
    for (int idx = tid; idx < nq * d_r; idx += blockDim.x) {
      const int jq = idx / d_r, r = idx - jq * d_r;
      const size_t qrow = static_cast<size_t>(q0 + jq) * H + h;
      q_abs[qrow * D + d_c + r] = q[qrow * dq + d_n + r];
    }
  }
}

// ---------------------------------------------------------------- a3 combine
// Block per query row, 128 threads, 4 consecutive columns per thread per pass.
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ o_part,
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
  const float ml = m * kLog2e;
  float tot = 0.f;
  for (int u = 0; u < S; ++u) tot += exp2f(fmaf(lp[u], kLog2e, -ml));
  const float inv = 1.f / tot;
  const float* op = o_part + row * S * width;
  for (int c = 4 * threadIdx.x; c < width; c += 4 * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // loads are unconditional so that 16 of them can be in flight; an empty split
    // (lse -inf, weight 0) may hold anything, so its values are selected away, not scaled
#pragma unroll 16
    for (int u = 0; u < S; ++u) {
      const float wgt = exp2f(fmaf(lp[u], kLog2e, -ml));
      const float4 v = *reinterpret_cast<const float4*>(op + static_cast<size_t>(u) * width + c);
      const bool use = wgt > 0.f;
      acc.x = fmaf(wgt, use ? v.x : 0.f, acc.x);
      acc.y = fmaf(wgt, use ? v.y : 0.f, acc.y);
      acc.z = fmaf(wgt, use ? v.z : 0.f, acc.z);
      acc.w = fmaf(wgt, use ? v.w : 0.f, acc.w);
    }
    *reinterpret_cast<float4*>(o + row * width + c) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (threadIdx.x == 0 && lse) lse[row] = m + logf(tot);
}

// ---------------------------------------------------------------- a4 out_uv
// Block (head h, 32 value rows, 8 queries), 256 threads.  Within a wave, lanes 8r..8r+7
// read W_UV row v0 + 8 wave + r in 128-byte segments (8 elements a lane); the queries'
// latent outputs sit in LDS.  The 8 lanes of a row meet by shuffles.
constexpr int kUvRows = 32;
template <typename T>
__global__ __launch_bounds__(256) void out_uv_kernel(const float* __restrict__ o_lat,
                                                     const T* __restrict__ w_uv,
                                                     float* __restrict__ out, int NQ, int H,
                                                     int Hw, int d_c, int d_v) {
  extern __shared__ float os[];  // [kQB][d_c]
  const int h = blockIdx.x, v0 = blockIdx.y * kUvRows, q0 = blockIdx.z * kQB;
  const int w = h / (H / Hw);
  const int nq = min(kQB, NQ - q0);
  const int tid = threadIdx.x;
  for (int idx = 4 * tid; idx < kQB * d_c; idx += 4 * blockDim.x) {
    const int jq = idx / d_c, c = idx - jq * d_c;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (jq < nq)
      v = *reinterpret_cast<const float4*>(o_lat + (static_cast<size_t>(q0 + jq) * H + h) * d_c + c);
    *reinterpret_cast<float4*>(&os[idx]) = v;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int v = v0 + 8 * wave + (lane >> 3), cg = lane & 7;
  float acc[kQB];
#pragma unroll
  for (int jq = 0; jq < kQB; ++jq) acc[jq] = 0.f;
  if (v < d_v) {
    const T* wr = w_uv + (static_cast<size_t>(w) * d_v + v) * d_c;
#pragma unroll 8
    for (int c = 8 * cg; c < d_c; c += 64) {
      float wv[8];
      load8(wr + c, wv);
#pragma unroll
      for (int jq = 0; jq < kQB; ++jq) {
        const float4 a = *reinterpret_cast<const float4*>(&os[jq * d_c + c]);
        const float4 b = *reinterpret_cast<const float4*>(&os[jq * d_c + c + 4]);
        float t = acc[jq];
        t = fmaf(a.x, wv[0], t); t = fmaf(a.y, wv[1], t);
        t = fmaf(a.z, wv[2], t); t = fmaf(a.w, wv[3], t);
        t = fmaf(b.x, wv[4], t); t = fmaf(b.y, wv[5], t);
        t = fmaf(b.z, wv[6], t); t = fmaf(b.w, wv[7], t);
        acc[jq] = t;
      }
    }
  }
#pragma unroll
  for (int jq = 0; jq < kQB; ++jq) {
    float t = acc[jq];
    t += __shfl_xor(t, 1, 64);
    t += __shfl_xor(t, 2, 64);
    t += __shfl_xor(t, 4, 64);
    acc[jq] = t;
  }
  if (v < d_v && cg == 0) {
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
  dim3 grid(s.n_heads, (s.d_c + kAbsCols - 1) / kAbsCols, (NQ + kQB - 1) / kQB);
  const size_t lds = sizeof(float) * kQB * (s.d_nope + 4 * kAbsCols);
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
  dim3 grid(s.n_heads, (s.d_v + kUvRows - 1) / kUvRows, (NQ + kQB - 1) / kQB);
  const size_t lds = sizeof(float) * kQB * s.d_c;
  if (s.dtype == MLA_F32)
    hipLaunchKernelGGL(out_uv_kernel<float>, grid, dim3(256), lds, st, o_lat,
                       static_cast<const float*>(w_uv), out, NQ, s.n_heads, s.n_wheads,
                       s.d_c, s.d_v);
  else
    hipLaunchKernelGGL(out_uv_kernel<bf16_t>, grid, dim3(256), lds, st, o_lat,
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

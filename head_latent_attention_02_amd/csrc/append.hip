// Cache append: the write side of the decode step.  Every new token's hidden state is
// projected down to the latent (c = W_DKV h) and to the decoupled RoPE key
// (k^R = W_KR h), the key is rotated to the token's position, and the row [c ; k^R] is
// written into its paged-cache slot ("MLA and GRPO architecture", s.2, "The Mathematics
// of MLA" and "Decoupled Rotary Position Embeddings").  The rotation turns consecutive
// pairs (2i, 2i+1) by t * base^(-2i / d_rope); the pages give no convention, this is the
// rotary embedding's own definition.
//
// A weight-read-bound GEMV: W_DKV and W_KR (D x d_model) are read once per block of
// tokens; the hidden states are small and come from L2.  bf16 runs on the matrix cores,
// fp32 (and shapes the matrix-core kernel does not take) on the vector units.
#include <math.h>

#include <type_traits>

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

// bf16 on the matrix cores: out[row][token] = sum_k W[row][k] h[token][k] as
// v_mfma_f32_16x16x32_bf16 with the weight rows as the A operand and the hidden states as
// the B operand, both read in their natural row-major layout (K = d_model contiguous).
// Block (16 output rows, 16 tokens), 8 waves splitting the K-steps; the partial products
// meet in LDS in wave order.  Lane l of the result holds rows 4 (l / 16) + j, j < 4, of
// token l % 16, so both rows of a RoPE pair are in one lane.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kApmWaves = 8;
constexpr int kApmBatch = 10;   // K-steps whose loads are in flight together

__global__ __launch_bounds__(64 * kApmWaves) void cache_append_mfma_kernel(
    const bf16_t* __restrict__ h, const bf16_t* __restrict__ w_dkv,
    const bf16_t* __restrict__ w_kr, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, bf16_t* __restrict__ pool, int NQ, int s_q,
    int d_c, int d_r, int d_model, int max_pages, int num_pages, int P, double log_base) {
  __shared__ f32x4_t red[kApmWaves - 1][64];
  const int D = d_c + d_r;
  const int o0 = 16 * blockIdx.x, n0 = 16 * blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, kg = lane >> 4;
  const int o = o0 + m;                       // D is a multiple of 16: always a real row
  const bf16_t* wr = (o < d_c ? w_dkv + static_cast<size_t>(o) * d_model
                              : w_kr + static_cast<size_t>(o - d_c) * d_model) + 8 * kg;
  const bool tok_ok = n0 + m < NQ;
  const bf16_t* hr = h + static_cast<size_t>(min(n0 + m, NQ - 1)) * d_model + 8 * kg;
  const int n_k = d_model / 32;
  const int per = (n_k + kApmWaves - 1) / kApmWaves;
  const int kb = wave * per, ke = min(n_k, kb + per);
  f32x4_t acc = {};
  for (int k0 = kb; k0 < ke; k0 += kApmBatch) {
    uint4 a[kApmBatch], b[kApmBatch];
#pragma unroll
    for (int t = 0; t < kApmBatch; ++t) {
      const int ks = min(k0 + t, ke - 1);
      a[t] = *reinterpret_cast<const uint4*>(wr + 32 * ks);
      b[t] = *reinterpret_cast<const uint4*>(hr + 32 * ks);
    }
    // predicated, not a break: the loop must unroll fully so a[] and b[] stay in registers
#pragma unroll
    for (int t = 0; t < kApmBatch; ++t) {
      const uint4 bv = tok_ok ? b[t] : make_uint4(0u, 0u, 0u, 0u);
      if (k0 + t < ke)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[t]),
                                                      __builtin_bit_cast(bf16x8_t, bv), acc,
                                                      0, 0, 0);
    }
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kApmWaves - 1; ++w) acc += red[w][lane];
  // lane: token n0 + lane % 16, rows o0 + 4 (lane / 16) + j
  const int q = n0 + (lane & 15);
  if (q >= NQ) return;
  const int b = q / s_q, s = q - b * s_q;
  const int t = ctx_lens[b] - s_q + s;
  if (t < 0 || t / P >= max_pages) return;
  const int page = page_table[static_cast<size_t>(b) * max_pages + t / P];
  if (page < 0 || page >= num_pages) return;
  bf16_t* dst = pool + (static_cast<size_t>(page) * P + t % P) * D + o0 + 4 * (lane >> 4);
  const int ob = o0 + 4 * (lane >> 4);
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    float x0 = acc[j], x1 = acc[j + 1];
    if (ob + j >= d_c) {   // a RoPE pair: rows ob + j (even) and ob + j + 1
      const int i = (ob + j - d_c) >> 1;
      const double ang = static_cast<double>(t) * exp(-log_base * (2.0 * i) / d_r);
      const double c = cos(ang), sn = sin(ang);
      const float y0 = static_cast<float>(x0 * c - x1 * sn);
      const float y1 = static_cast<float>(x0 * sn + x1 * c);
      x0 = y0;
      x1 = y1;
    }
    dst[j] = f32_to_bf16(x0);
    dst[j + 1] = f32_to_bf16(x1);
  }
}

// bf16 with at most 8 new tokens: the weight read spread over D / 2 workgroups (two output
// rows each, one RoPE pair for the key rows) instead of D / 16, since with so few tokens the
// step is the latency of one weight read.  Thread t owns the 8-element chunks t, t + 256,
// t + 512 of the d_model axis; every load of the thread (both weight rows and the QB hidden
// states, the latter from L2) is issued before the first product; the partial sums meet by
// wave sums and LDS.
template <int QB>
__global__ __launch_bounds__(256, 1) void cache_append_stream_kernel(
    const bf16_t* __restrict__ h, const bf16_t* __restrict__ w_dkv,
    const bf16_t* __restrict__ w_kr, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, bf16_t* __restrict__ pool, int NQ, int s_q,
    int d_c, int d_r, int d_model, int max_pages, int num_pages, int P, double log_base) {
  constexpr int kCh = 3;   // chunks per thread: d_model <= 8 * 256 * 3
  __shared__ float red[4][2 * QB];
  const int D = d_c + d_r;
  const int o0 = 2 * blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bf16_t* wr[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int o = o0 + r;
    wr[r] = o < d_c ? w_dkv + static_cast<size_t>(o) * d_model
                    : w_kr + static_cast<size_t>(o - d_c) * d_model;
  }
  const int n_ch = d_model / 8;
  uint4 wv[2][kCh], hv[QB][kCh];
#pragma unroll
  for (int j = 0; j < kCh; ++j) {
    const int c = min(tid + 256 * j, n_ch - 1);   // past the end: a valid chunk, not used
#pragma unroll
    for (int r = 0; r < 2; ++r) wv[r][j] = *reinterpret_cast<const uint4*>(wr[r] + 8 * c);
#pragma unroll
    for (int n = 0; n < QB; ++n)
      hv[n][j] = *reinterpret_cast<const uint4*>(
          h + static_cast<size_t>(min(n, NQ - 1)) * d_model + 8 * c);
  }
  // keep the scheduler from moving the conversions of early loads ahead of the later loads
  __builtin_amdgcn_sched_barrier(0);
  float acc[2][QB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int n = 0; n < QB; ++n) acc[r][n] = 0.f;
#pragma unroll
  for (int j = 0; j < kCh; ++j) {
    // a chunk past the end contributes zero (a select, not a branch, so that the compiler
    // keeps every load ahead of the first product)
    const bool live = tid + 256 * j < n_ch;
    float w[2][8];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t u[4] = {wv[r][j].x, wv[r][j].y, wv[r][j].z, wv[r][j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[r][2 * e] = __uint_as_float(u[e] << 16);
        w[r][2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int n = 0; n < QB; ++n) {
      const uint32_t u[4] = {hv[n][j].x, hv[n][j].y, hv[n][j].z, hv[n][j].w};
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = live ? __uint_as_float(u[e] << 16) : 0.f;
        x[2 * e + 1] = live ? __uint_as_float(u[e] & 0xffff0000u) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][n] = fmaf(w[r][e], x[e], acc[r][n]);
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int n = 0; n < QB; ++n) {
      const float v = wave_sum(acc[r][n]);
      if (lane == 0) red[wave][r * QB + n] = v;
    }
  __syncthreads();
  if (tid >= QB) return;
  // thread n: token n, both rows (a RoPE pair when o0 >= d_c)
  const int n = tid;
  if (n >= NQ) return;
  float x0 = ((red[0][n] + red[1][n]) + red[2][n]) + red[3][n];
  float x1 = ((red[0][QB + n] + red[1][QB + n]) + red[2][QB + n]) + red[3][QB + n];
  const int b = n / s_q, s = n - b * s_q;
  const int t = ctx_lens[b] - s_q + s;
  if (t < 0 || t / P >= max_pages) return;
  const int page = page_table[static_cast<size_t>(b) * max_pages + t / P];
  if (page < 0 || page >= num_pages) return;
  if (o0 >= d_c) {
    const int i = (o0 - d_c) >> 1;
    const double ang = static_cast<double>(t) * exp(-log_base * (2.0 * i) / d_r);
    const double c = cos(ang), sn = sin(ang);
    const float y0 = static_cast<float>(x0 * c - x1 * sn);
    const float y1 = static_cast<float>(x0 * sn + x1 * c);
    x0 = y0;
    x1 = y1;
  }
  bf16_t* dst = pool + (static_cast<size_t>(page) * P + t % P) * D + o0;
  dst[0] = f32_to_bf16(x0);
  dst[1] = f32_to_bf16(x1);
}

}  // namespace

hipError_t launch_cache_append(const mla_shape_t& s, int d_model, float rope_base,
                               const void* h, const void* w_dkv, const void* w_kr,
                               const int32_t* page_table, const int32_t* ctx_lens,
                               void* pool, hipStream_t st) {
  const int NQ = s.batch * s.s_q, D = s.d_c + s.d_rope;
  const dim3 grid((D + kApRows - 1) / kApRows, (NQ + kApTok - 1) / kApTok);
  const double lb = log(static_cast<double>(rope_base));
  // few tokens: two rows per workgroup on the vector units (d_model within three chunks of
  // 8 elements per thread)
  if (s.dtype == MLA_BF16 && NQ <= 8 && d_model % 8 == 0 && d_model <= 8 * 256 * 3 &&
      s.d_c % 2 == 0 && D % 2 == 0) {
    auto go = [&](auto qbc) {
      constexpr int QB = decltype(qbc)::value;
      hipLaunchKernelGGL((cache_append_stream_kernel<QB>), dim3(D / 2), dim3(256), 0, st,
                         static_cast<const bf16_t*>(h), static_cast<const bf16_t*>(w_dkv),
                         static_cast<const bf16_t*>(w_kr), page_table, ctx_lens,
                         static_cast<bf16_t*>(pool), NQ, s.s_q, s.d_c, s.d_rope, d_model,
                         s.max_pages, s.num_pages, s.page_size, lb);
    };
    if (NQ <= 4)
      go(std::integral_constant<int, 4>{});
    else
      go(std::integral_constant<int, 8>{});
    return hipGetLastError();
  }
  if (s.dtype == MLA_BF16 && D % 16 == 0 && d_model % 32 == 0) {
    hipLaunchKernelGGL(cache_append_mfma_kernel, dim3(D / 16, (NQ + 15) / 16),
                       dim3(64 * kApmWaves), 0, st, static_cast<const bf16_t*>(h),
                       static_cast<const bf16_t*>(w_dkv), static_cast<const bf16_t*>(w_kr),
                       page_table, ctx_lens, static_cast<bf16_t*>(pool), NQ, s.s_q, s.d_c,
                       s.d_rope, d_model, s.max_pages, s.num_pages, s.page_size, lb);
    return hipGetLastError();
  }
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

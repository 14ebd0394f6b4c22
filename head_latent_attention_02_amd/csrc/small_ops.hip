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

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

constexpr int kQB = 8;  // queries per block in a4, and in a1 above 4 queries

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 8 consecutive elements: a raw chunk (one 16-byte load for bf16, two for fp32) and its
// conversion to floats.  Kernels issue a batch of raw loads first and convert afterwards,
// so that a whole batch is in flight at once.
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16_t> {
  uint4 v;
};
template <>
struct Raw8<float> {
  float4 a, b;
};
__device__ __forceinline__ Raw8<bf16_t> load_raw8(const bf16_t* p) {
  return {*reinterpret_cast<const uint4*>(p)};
}
__device__ __forceinline__ Raw8<float> load_raw8(const float* p) {
  return {*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
}
__device__ __forceinline__ void to_f32(const Raw8<bf16_t>& r, float (&x)[8]) {
  const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void to_f32(const Raw8<float>& r, float (&x)[8]) {
  x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
  x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

// ---------------------------------------------------------------- a1 absorb
// Block (head h, 8 LANES latent columns, QB = 4 or 8 queries), 256 threads.  Thread
// (rs, cl) = (tid / LANES, tid % LANES) owns columns c0 + 8 cl .. +8 and weight rows rs,
// rs + 256 / LANES, ...: each W_UK row chunk is one coalesced read of 16 LANES bytes, and
// every weight byte of the block is read once.  4 queries per block use 128 columns (512
// blocks at 128 heads, two per CU); 8 queries use 256 columns (half the blocks, each
// re-reading its weights for fewer query blocks; measured 5 % faster on the 16- and
// 128-query steps, 1 % slower on the 4-query one).
template <int LANES>
struct AbsLayout {
  static constexpr int kCols = 8 * LANES;          // latent columns per block
  static constexpr int kSlices = 256 / LANES;      // row slices
  static constexpr int kBatch = 128 / kSlices;     // weight rows per thread in flight at once
};
template <typename T, int QB, int LANES>
__global__ __launch_bounds__(256) void absorb_q_kernel(const T* __restrict__ q,
                                                       const T* __restrict__ w_uk,
                                                       T* __restrict__ q_abs, int NQ, int H,
                                                       int Hw, int d_n, int d_r, int d_c) {
  extern __shared__ float smem[];
  float* qs = smem;                       // [d_n][QB]: row i's QB queries together
  float* red = smem + QB * d_n;           // [4 waves][QB][AbsLayout<LANES>::kCols]
  const int h = blockIdx.x, c0 = blockIdx.y * AbsLayout<LANES>::kCols, q0 = blockIdx.z * QB;
  const int w = h / (H / Hw);
  const int nq = min(QB, NQ - q0);
  const int dq = d_n + d_r, D = d_c + d_r;
  const int tid = threadIdx.x, rs = tid / LANES, cl = tid % LANES;
  const int c = c0 + 8 * cl;
  const T* W = w_uk + static_cast<size_t>(w) * d_n * d_c + c;
  // weight rows rs, rs + kSlices, ... in batches of kBatch: a batch's loads are all issued
  // before any is used, and the first batch (at d_n = 128 a thread's whole share) before
  // the queries are staged, so the two reads overlap
  Raw8<T> raw[AbsLayout<LANES>::kBatch];
  auto issue = [&](int i0) {
#pragma unroll
    for (int bt = 0; bt < AbsLayout<LANES>::kBatch; ++bt) {
      const int i = i0 + AbsLayout<LANES>::kSlices * bt;
      if (c < d_c && i < d_n) raw[bt] = load_raw8(W + static_cast<size_t>(i) * d_c);
    }
  };
  issue(rs);
  // the queries' no-position parts, 8 elements per thread and load (one load each while
  // QB * d_n <= 8 * 256), transposed into qs
  for (int idx = tid; idx < QB * d_n / 8; idx += blockDim.x) {
    const int per = d_n / 8;
    const int jq = idx / per, i8 = 8 * (idx - jq * per);
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (jq < nq) to_f32(load_raw8(q + (static_cast<size_t>(q0 + jq) * H + h) * dq + i8), x);
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[(i8 + e) * QB + jq] = x[e];
  }
  __syncthreads();
  float acc[QB][8];
#pragma unroll
  for (int jq = 0; jq < QB; ++jq)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[jq][e] = 0.f;
  if (c < d_c) {
    for (int i0 = rs; i0 < d_n; i0 += AbsLayout<LANES>::kSlices * AbsLayout<LANES>::kBatch) {
      if (i0 != rs) issue(i0);
#pragma unroll
      for (int bt = 0; bt < AbsLayout<LANES>::kBatch; ++bt) {
        const int i = i0 + AbsLayout<LANES>::kSlices * bt;
        if (i >= d_n) break;
        float wv[8];
        to_f32(raw[bt], wv);
        // the row's QB query values: 16-byte LDS reads, the same address across a
        // half-wave (a broadcast)
        float qv[QB];
#pragma unroll
        for (int k4 = 0; k4 < QB; k4 += 4) {
          const float4 t = *reinterpret_cast<const float4*>(&qs[i * QB + k4]);
          qv[k4] = t.x; qv[k4 + 1] = t.y; qv[k4 + 2] = t.z; qv[k4 + 3] = t.w;
        }
#pragma unroll
        for (int jq = 0; jq < QB; ++jq)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[jq][e] = fmaf(qv[jq], wv[e], acc[jq][e]);
      }
    }
  }
  // the row slices of a wave meet by shuffles, the 4 waves in LDS
#pragma unroll
  for (int off = LANES; off < 64; off <<= 1)
#pragma unroll
    for (int jq = 0; jq < QB; ++jq)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[jq][e] += __shfl_xor(acc[jq][e], off, 64);
  if ((tid & 63) < LANES) {
    const int wv = tid >> 6;
#pragma unroll
    for (int jq = 0; jq < QB; ++jq)
#pragma unroll
      for (int e = 0; e < 8; e += 4)
        *reinterpret_cast<float4*>(&red[(wv * QB + jq) * AbsLayout<LANES>::kCols + 8 * cl + e]) =
            make_float4(acc[jq][e], acc[jq][e + 1], acc[jq][e + 2], acc[jq][e + 3]);
  }
  __syncthreads();
  for (int idx = tid; idx < QB * AbsLayout<LANES>::kCols; idx += blockDim.x) {
    const int jq = idx / AbsLayout<LANES>::kCols, cc = idx - jq * AbsLayout<LANES>::kCols;
    if (jq >= nq || c0 + cc >= d_c) continue;
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) v += red[(r * QB + jq) * AbsLayout<LANES>::kCols + cc];
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

// q_abs[q, h, d_c : d_c + d_r] = q[q, h, d_n : d_n + d_r] for the block's queries, in 16-byte
// chunks (d_r is a multiple of 8), shared by the gridDim.y column blocks of head h: at the
// supported shapes each thread copies at most one chunk (one load, one store).
__device__ __forceinline__ void copy_rope_part(const bf16_t* __restrict__ q,
                                               bf16_t* __restrict__ q_abs, int q0, int nq,
                                               int H, int h, int d_n, int d_r, int d_c) {
  const int per_q = d_r / 8, chunks = nq * per_q;
  const int part = (chunks + gridDim.y - 1) / gridDim.y;
  const int c_lo = blockIdx.y * part, c_hi = min(chunks, c_lo + part);
  for (int i = c_lo + threadIdx.x; i < c_hi; i += blockDim.x) {
    const int jq = i / per_q, r8 = i - jq * per_q;
    const size_t qrow = static_cast<size_t>(q0 + jq) * H + h;
    *reinterpret_cast<uint4*>(q_abs + qrow * (d_c + d_r) + d_c + 8 * r8) =
        *reinterpret_cast<const uint4*>(q + qrow * (d_n + d_r) + d_n + 8 * r8);
  }
}

// a1 for a few bf16 queries (at most 8 per block), the weight read streamed at full width.
// Block (head h, 256 latent columns c0 .., QB queries), 256 threads, one block per CU at 128
// heads.  Lane l of wave wv owns columns c0 + 8 (l % 32) .. +8 and the weight rows
// i = l / 32 + 2 (wv + 4 j), j = 0 .. d_n / 8 - 1: each load instruction reads two whole
// 512-byte row segments, and a thread's d_n / 8 row loads are all issued at the start,
// right after the queries' (which the products need first), so the products of row j start
// as soon as its load lands instead of after the whole weight slice.  The two row halves of
// a wave meet by a lane swap, the four waves in LDS (summed in wave order).
constexpr int kAsC = 256;   // latent columns per block
template <int QB>
__global__ __launch_bounds__(256) void absorb_q_stream_kernel(const bf16_t* __restrict__ q,
                                                              const bf16_t* __restrict__ w_uk,
                                                              bf16_t* __restrict__ q_abs,
                                                              int NQ, int H, int Hw, int d_r,
                                                              int d_c) {
  constexpr int d_n = 128, kRowsT = d_n / 8;
  __shared__ __align__(16) float qs[d_n * QB];          // [row i][query]
  __shared__ __align__(16) float red[4][QB][kAsC];      // per-wave partial sums
  const int h = blockIdx.x, c0 = blockIdx.y * kAsC, q0 = blockIdx.z * QB;
  const int w = h / (H / Hw);
  const int nq = min(QB, NQ - q0);
  const int dq = d_n + d_r, D = d_c + d_r;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int cc = lane & 31, rp = lane >> 5;
  // (1) the queries' no-position parts: QB * d_n / 8 threads load 8 elements each
  uint4 qraw = make_uint4(0u, 0u, 0u, 0u);
  const int jq = tid / (d_n / 8), i8 = 8 * (tid % (d_n / 8));
  const bool qload = tid < QB * d_n / 8 && jq < nq;
  if (qload)
    qraw = *reinterpret_cast<const uint4*>(q + (static_cast<size_t>(q0 + jq) * H + h) * dq + i8);
  // (2) every weight row of this thread, in flight together
  const bf16_t* W = w_uk + static_cast<size_t>(w) * d_n * d_c + c0 + 8 * cc;
  uint4 raw[kRowsT];
#pragma unroll
  for (int j = 0; j < kRowsT; ++j)
    raw[j] = *reinterpret_cast<const uint4*>(W + static_cast<size_t>(rp + 2 * (wv + 4 * j)) * d_c);
  // (3) the queries into LDS, transposed
  if (tid < QB * d_n / 8) {
    const uint32_t u[4] = {qraw.x, qraw.y, qraw.z, qraw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qs[(i8 + 2 * e) * QB + jq] = __uint_as_float(u[e] << 16);
      qs[(i8 + 2 * e + 1) * QB + jq] = __uint_as_float(u[e] & 0xffff0000u);
    }
  }
  __syncthreads();
  float acc[QB][8];
#pragma unroll
  for (int k = 0; k < QB; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
  // (4) row by row in load order
#pragma unroll
  for (int j = 0; j < kRowsT; ++j) {
    const int i = rp + 2 * (wv + 4 * j);
    const uint32_t u[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
    float wf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wf[2 * e] = __uint_as_float(u[e] << 16);
      wf[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
    }
    float qv[QB];
#pragma unroll
    for (int k4 = 0; k4 < QB; k4 += 4) {
      const float4 t = *reinterpret_cast<const float4*>(&qs[i * QB + k4]);
      qv[k4] = t.x; qv[k4 + 1] = t.y; qv[k4 + 2] = t.z; qv[k4 + 3] = t.w;
    }
#pragma unroll
    for (int k = 0; k < QB; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[k][e] = fmaf(qv[k], wf[e], acc[k][e]);
  }
  // (5) the two row halves of the wave (lanes l and l + 32), then the four waves
#pragma unroll
  for (int k = 0; k < QB; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[k][e]),
                                                      __float_as_uint(acc[k][e]), false, false);
      acc[k][e] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  if (rp == 0) {
#pragma unroll
    for (int k = 0; k < QB; ++k) {
      *reinterpret_cast<float4*>(&red[wv][k][8 * cc]) =
          make_float4(acc[k][0], acc[k][1], acc[k][2], acc[k][3]);
      *reinterpret_cast<float4*>(&red[wv][k][8 * cc + 4]) =
          make_float4(acc[k][4], acc[k][5], acc[k][6], acc[k][7]);
    }
  }
  __syncthreads();
  for (int idx = tid; idx < QB * kAsC; idx += 256) {
    const int k = idx / kAsC, c = idx - k * kAsC;
    if (k >= nq) break;
    const float v = ((red[0][k][c] + red[1][k][c]) + red[2][k][c]) + red[3][k][c];
    q_abs[(static_cast<size_t>(q0 + k) * H + h) * D + c0 + c] = f32_to_bf16(v);
  }
  copy_rope_part(q, q_abs, q0, nq, H, h, d_n, d_r, d_c);
}

// a1 on the matrix cores (bf16, d_n = 128, 16 or more queries).  Block (head h, 128 latent
// columns c0 .., 32 NB queries q0 ..), 4 waves; wave w computes q_abs^T[c][q] =
// sum_i W_UK[h][i][c] q[q][i] for the 32 queries of query block w % NB and NB column blocks
// of 32, with v_mfma_f32_32x32x16_bf16: the weight slice, staged once in
// LDS (rows of 256 bytes, 16-byte chunks XOR-swizzled by row), is the A operand, read
// transposed with ds_read_b64_tr_b16; the queries' no-position parts are the B operand,
// 16-byte loads in their natural layout.  Each weight byte is read once per 32 NB queries
// (once per 8 in absorb_q_kernel), which is what the multi-query decode steps need.
constexpr int kAmC = 128;   // latent columns per block
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
__device__ __forceinline__ int am_swz(int i) { return (((i >> 1) & 1) << 2) | ((i >> 2) & 3); }

template <int NB>
__global__ __launch_bounds__(256) void absorb_q_mfma_kernel(const bf16_t* __restrict__ q,
                                                            const bf16_t* __restrict__ w_uk,
                                                            bf16_t* __restrict__ q_abs, int NQ,
                                                            int H, int Hw, int d_r, int d_c) {
  constexpr int d_n = 128;
  __shared__ __align__(16) char ws[d_n * kAmC * 2];
  const int h = blockIdx.x, c0 = blockIdx.y * kAmC, q0 = blockIdx.z * 32 * NB;
  const int wh = h / (H / Hw);
  const int dq = d_n + d_r, D = d_c + d_r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = lane & 31, g = lane >> 5;
  const int nq = min(32 * NB, NQ - q0);
  // wave w: the 32 queries of query block w % NB and the NB column blocks of 32 starting at
  // block (w / NB) NB of the block's 128 columns, so each wave loads one query block only
  const int qblk = wave % NB, cb0 = (wave / NB) * NB;
  // weight slice W_UK[wh][0:128][c0:c0+128]: 2048 chunks of 16 bytes, 8 per thread
  const bf16_t* W = w_uk + static_cast<size_t>(wh) * d_n * d_c + c0;
  uint4 wv[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int idx = tid + 256 * k, i = idx >> 4, ch = idx & 15;
    wv[k] = *reinterpret_cast<const uint4*>(W + static_cast<size_t>(i) * d_c + 8 * ch);
  }
  // B operands: query 32 qblk + n32, rows i = 16 kt + 8 g .. +8 (zeros past the last query)
  bf16x8_t qb[8];
  const int qi = 32 * qblk + n32;
  {
    const bf16_t* qp = q + (static_cast<size_t>(q0 + min(qi, nq - 1)) * H + h) * dq + 8 * g;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const bf16x8_t v = *reinterpret_cast<const bf16x8_t*>(qp + 16 * kt);
      qb[kt] = (qi < nq) ? v : bf16x8_t{};
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int idx = tid + 256 * k, i = idx >> 4, ch = idx & 15;
    *reinterpret_cast<uint4*>(ws + i * 256 + ((ch ^ am_swz(i)) * 16)) = wv[k];
  }
  __syncthreads();
  // A operand of K-step kt for column block cb: the lane mapping of the transposed read (4
  // rows x 4 columns per 16-lane group, two reads per operand); to[cb & 1][h4], and column
  // blocks 2 and 3 are 128 bytes further on
  const int q16 = lane >> 4, L = lane & 15;
  int to[2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int h4 = 0; h4 < 2; ++h4) {
      const int col = 32 * par + 16 * (q16 & 1) + 4 * (L & 3);
      const int i = 8 * (q16 >> 1) + 4 * h4 + (L >> 2);
      to[par][h4] = i * 256 + (((col >> 3) ^ am_swz(i)) * 16) + (col & 7) * 2;
    }
  f32x16_t acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x16_t{};
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int cb = cb0 + j;
      // rows 16 kt .. +16 keep the swizzle of rows 0 .. 15 (it reads row bits 1-3 only)
      const int ofs = 4096 * kt + 128 * (cb >> 1);
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(const __attribute__((address_space(3))) char*)(ws + to[cb & 1][0] + ofs));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_t*)(const __attribute__((address_space(3))) char*)(ws + to[cb & 1][1] + ofs));
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[kt], acc[j], 0, 0, 0);
    }
  }
  // lane (query n32, half g) holds columns 8 (j / 4) + 4 g + j % 4 of each column block.
  // Stored as they are, each store instruction writes 16-byte pieces of 32 query rows.  With
  // two or more query blocks (over 32 queries) the outputs are first staged in ws (free once every wave
  // has read its last operands; rows of 256 bytes, 16-byte chunks XOR-swizzled by row) and
  // leave as whole 256-byte rows, four per store instruction: a1 at 128 queries 21.5 ->
  // 17.5 us.  For one query block (16 queries) staging measured no gain, so that case keeps
  // the direct stores and their one barrier fewer.
  auto pack = [&](int j, int jg, int e) {
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[j][4 * jg + 2 * e]))) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[j][4 * jg + 2 * e + 1]))) << 16);
  };
  if constexpr (NB == 1) {
    if (qi < nq) {
      bf16_t* orow = q_abs + static_cast<size_t>(q0 + qi) * H * D + static_cast<size_t>(h) * D +
                     c0 + 4 * g;
#pragma unroll
      for (int jg = 0; jg < 4; ++jg)
        *reinterpret_cast<uint2*>(orow + 32 * cb0 + 8 * jg) = make_uint2(pack(0, jg, 0), pack(0, jg, 1));
    }
  } else {
    __syncthreads();
    char* srow = ws + (32 * qblk + n32) * 256;
    const int sw = n32 & 15;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const int ch = 4 * (cb0 + j) + jg;   // 16-byte chunk of the 256-byte row
        *reinterpret_cast<uint2*>(srow + ((ch ^ sw) * 16) + 8 * g) =
            make_uint2(pack(j, jg, 0), pack(j, jg, 1));
      }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2 * NB; ++k) {
      const int idx = tid + 256 * k, r = idx >> 4, ch = idx & 15;
      if (r < nq)
        *reinterpret_cast<uint4*>(q_abs + static_cast<size_t>(q0 + r) * H * D +
                                  static_cast<size_t>(h) * D + c0 + 8 * ch) =
            *reinterpret_cast<const uint4*>(ws + r * 256 + ((ch ^ (r & 15)) * 16));
    }
  }
  copy_rope_part(q, q_abs, q0, nq, H, h, d_n, d_r, d_c);
}

// ---------------------------------------------------------------- a3 combine
constexpr int kCombBatch = 32;
constexpr int kCombWts = 2048;
// Block per query row, 128 threads, 4 consecutive columns per thread per pass.
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      float* __restrict__ o,
                                                      float* __restrict__ lse, int S,
                                                      int width) {
  const size_t row = blockIdx.x;
  const float* lp = lse_part + row * S;
  const float* op = o_part + row * S * width;
  __shared__ float red[2][4];
  __shared__ float wts[kCombWts];  // chunk weights e^{lse_u - max} of the first kCombWts
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;   // 128 threads = 2 waves
  // the first batch of partials (at width 512 and S <= 32 a thread's whole share) is
  // loaded while the chunk weights are reduced
  float4 v[kCombBatch];
  auto issue = [&](int c, int u0) {
#pragma unroll
    for (int b = 0; b < kCombBatch; ++b)
      if (u0 + b < S)
        v[b] = *reinterpret_cast<const float4*>(op + static_cast<size_t>(u0 + b) * width + c);
  };
  // this thread's first chunk lse is loaded before the partials: loads complete in issue
  // order, so the weight reduction below waits for it alone, not for the whole batch
  const float l_first = static_cast<int>(threadIdx.x) < S ? lp[threadIdx.x] : -INFINITY;
  if (4 * threadIdx.x < width) issue(4 * threadIdx.x, 0);
  // row maximum and sum of the chunk weights, every thread taking splits t, t + 128, ...
  float m = l_first;
  for (int u = threadIdx.x + blockDim.x; u < S; u += blockDim.x) m = fmaxf(m, lp[u]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane == 0) red[0][wv] = m;
  __syncthreads();
  m = fmaxf(red[0][0], red[0][1]);
  if (m == -INFINITY) {
    for (int c = threadIdx.x; c < width; c += blockDim.x) o[row * width + c] = 0.f;
    if (threadIdx.x == 0 && lse) lse[row] = -INFINITY;
    return;
  }
  const float ml = m * kLog2e;
  float tot = 0.f;
  for (int u = threadIdx.x; u < S; u += blockDim.x) {
    const float e = exp2f(fmaf(u == static_cast<int>(threadIdx.x) ? l_first : lp[u], kLog2e, -ml));
    if (u < kCombWts) wts[u] = e;
    tot += e;
  }
  tot = wave_sum(tot);
  if (lane == 0) red[1][wv] = tot;
  __syncthreads();
  tot = red[1][0] + red[1][1];
  const float inv = 1.f / tot;
  for (int c = 4 * threadIdx.x; c < width; c += 4 * blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // splits in batches of kCombBatch whose loads are all issued before any is used; an
    // empty split (lse -inf, weight 0) may hold anything, so its values are selected
    // away, not scaled
    for (int u0 = 0; u0 < S; u0 += kCombBatch) {
      if (u0 != 0 || c != 4 * static_cast<int>(threadIdx.x)) issue(c, u0);
#pragma unroll
      for (int b = 0; b < kCombBatch; ++b) {
        if (u0 + b >= S) break;
        const float wgt = u0 + b < kCombWts ? wts[u0 + b]
                                            : exp2f(fmaf(lp[u0 + b], kLog2e, -ml));
        const bool use = wgt > 0.f;
        acc.x = fmaf(wgt, use ? v[b].x : 0.f, acc.x);
        acc.y = fmaf(wgt, use ? v[b].y : 0.f, acc.y);
        acc.z = fmaf(wgt, use ? v[b].z : 0.f, acc.z);
        acc.w = fmaf(wgt, use ? v[b].w : 0.f, acc.w);
      }
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
constexpr int kUvBatch = 8;   // weight chunks per thread in flight at once
constexpr int kUvStage = 4;   // o_lat float4 loads per thread in flight at once
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
  // the queries' latent outputs: up to kUvStage float4 loads per thread in flight at once
  for (int i0 = 4 * tid; i0 < kQB * d_c; i0 += 4 * blockDim.x * kUvStage) {
    float4 v[kUvStage];
#pragma unroll
    for (int b = 0; b < kUvStage; ++b) {
      const int idx = i0 + 4 * blockDim.x * b;
      const int jq = idx / d_c, c = idx - jq * d_c;
      v[b] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (idx < kQB * d_c && jq < nq)
        v[b] = *reinterpret_cast<const float4*>(
            o_lat + (static_cast<size_t>(q0 + jq) * H + h) * d_c + c);
    }
#pragma unroll
    for (int b = 0; b < kUvStage; ++b) {
      const int idx = i0 + 4 * blockDim.x * b;
      if (idx < kQB * d_c) *reinterpret_cast<float4*>(&os[idx]) = v[b];
    }
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const int v = v0 + 8 * wave + (lane >> 3), cg = lane & 7;
  float acc[kQB];
#pragma unroll
  for (int jq = 0; jq < kQB; ++jq) acc[jq] = 0.f;
  if (v < d_v) {
    const T* wr = w_uv + (static_cast<size_t>(w) * d_v + v) * d_c;
    // columns 8 cg + 64 b in batches of kUvBatch, loads issued before use
    for (int c0 = 8 * cg; c0 < d_c; c0 += 64 * kUvBatch) {
     Raw8<T> raw[kUvBatch];
#pragma unroll
     for (int bt = 0; bt < kUvBatch; ++bt)
       if (c0 + 64 * bt < d_c) raw[bt] = load_raw8(wr + c0 + 64 * bt);
#pragma unroll
     for (int bt = 0; bt < kUvBatch; ++bt) {
      const int c = c0 + 64 * bt;
      if (c >= d_c) break;
      float wv[8];
      to_f32(raw[bt], wv);
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

// a4 on the matrix cores (bf16 weights): out^T[v][n] = sum_c W_UV[w(h)][v][c] o[n][h][c] as
// v_mfma_f32_32x32x16_bf16 with the weight rows as the A operand (v = M, c = K, both in
// their natural row-major layout) and the latent outputs, rounded to bf16, as the B
// operand (query = N, padded to 32).  One block of 4 waves per (head, 32 value rows); the
// waves split the latent dimension (at d_c = 512 each issues all its loads at once) and
// meet in LDS; query blocks of 32 in turn.
constexpr int kUvmSteps = 8;
constexpr int kUvmWaves = 4;

__global__ __launch_bounds__(64 * kUvmWaves) void out_uv_mfma_kernel(
    const float* __restrict__ o_lat, const bf16_t* __restrict__ w_uv, float* __restrict__ out,
    int NQ, int H, int Hw, int d_c, int d_v) {
  __shared__ float red[kUvmWaves - 1][16][64];
  const int h = blockIdx.x, v0 = 32 * blockIdx.y;
  const int w = h / (H / Hw);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, m = lane & 31, g = lane >> 5;
  const int n_k = d_c / 16;
  const int per = (n_k + kUvmWaves - 1) / kUvmWaves;
  const int kb = wave * per, ke = min(n_k, kb + per);   // this wave's K-steps
  const int v = min(v0 + m, d_v - 1);   // rows past d_v read a valid row, never stored
  const bf16_t* wr = w_uv + (static_cast<size_t>(w) * d_v + v) * d_c + 8 * g;
  for (int n0 = 0; n0 < NQ; n0 += 32) {
    const int n = n0 + m;
    const float* orow = o_lat + (static_cast<size_t>(min(n, NQ - 1)) * H + h) * d_c + 8 * g;
    f32x16_t acc = {};
    for (int k0 = kb; k0 < ke; k0 += kUvmSteps) {
      uint4 a[kUvmSteps];
      float4 b[kUvmSteps][2];
#pragma unroll
      for (int t = 0; t < kUvmSteps; ++t) {
        const int ks = min(k0 + t, ke - 1);
        a[t] = *reinterpret_cast<const uint4*>(wr + 16 * ks);
        b[t][0] = *reinterpret_cast<const float4*>(orow + 16 * ks);
        b[t][1] = *reinterpret_cast<const float4*>(orow + 16 * ks + 4);
      }
#pragma unroll
      for (int t = 0; t < kUvmSteps; ++t) {
        if (k0 + t >= ke) break;
        bf16x8_t bv;
        bv[0] = static_cast<__bf16>(b[t][0].x); bv[1] = static_cast<__bf16>(b[t][0].y);
        bv[2] = static_cast<__bf16>(b[t][0].z); bv[3] = static_cast<__bf16>(b[t][0].w);
        bv[4] = static_cast<__bf16>(b[t][1].x); bv[5] = static_cast<__bf16>(b[t][1].y);
        bv[6] = static_cast<__bf16>(b[t][1].z); bv[7] = static_cast<__bf16>(b[t][1].w);
        if (n >= NQ) bv = bf16x8_t{};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[t]), bv,
                                                      acc, 0, 0, 0);
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) red[wave - 1][j][lane] = acc[j];
    }
    __syncthreads();
    // lane (query n, half g) holds value rows 8 (j / 4) + 4 g + j % 4 of the block
    if (wave == 0 && n < NQ) {
      float* orow_out = out + (static_cast<size_t>(n) * H + h) * d_v + v0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float t = acc[j];
#pragma unroll
        for (int r = 0; r < kUvmWaves - 1; ++r) t += red[r][j][lane];
        const int vv = 8 * (j >> 2) + 4 * g + (j & 3);
        if (v0 + vv < d_v) orow_out[vv] = t;
      }
    }
    __syncthreads();   // red is reused by the next query block
  }
}

// ---------------------------------------------------------------- a3 + a4 fused
// The step's split merge and value up-projection in one launch (bf16 weights, d_c = 512,
// d_v = 128, at most 64 splits, heads a multiple of 8).  Block (head h, NV of its four
// 32-row value blocks, 32 queries), 4 NV waves.  Arithmetic is the same, operation for
// operation, as combine_kernel followed by out_uv_mfma_kernel, so the results are bitwise
// those of the two separate entry points; what changes is that the merged latent rows go to
// the up-projection through LDS and that the weight loads, the partial loads and the lse
// reductions are all in flight together.
//   wave w: value rows 32 (NV half + w % NV) .. +32 and latent quarter w / NV of the
//   up-projection; all waves share the merge (one query x 512 columns per 128 threads and
//   pass).
//   NV = 2: a head's two halves are 8 blocks apart, so they run on one XCD and the second
//   one's partial reads hit its L2; both compute the merge (only half 0 stores o_lat and
//   lse).  NV = 4: one block per head and query block reads each partial once, which halves
//   the bytes each CU pulls; used when heads x query blocks alone fill the CUs.
constexpr int kFuQ = 32;          // queries per block
constexpr int kFuRow = 512 + 8;   // bf16 elements per LDS row of merged latents (padded)

template <int NV>
__global__ __launch_bounds__(256 * NV) void combine_out_uv_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    const bf16_t* __restrict__ w_uv, float* __restrict__ o_lat, float* __restrict__ lse,
    float* __restrict__ out, int NQ, int H, int Hw, int S) {
  constexpr int d_c = 512, d_v = 128;
  constexpr int kWaves = 4 * NV, kPass = 2 * NV;   // waves; queries merged per pass
  // partial loads per thread in flight at once (1024 threads leave 128 VGPRs a thread)
  constexpr int kFuBatch = NV == 2 ? 32 : 8;
  __shared__ __align__(16) bf16_t ob[kFuQ * kFuRow];   // merged latents as MFMA B rows
  __shared__ float wts[kFuQ][64];                       // chunk weights e^{lse_u - max}
  __shared__ float inv_s[kFuQ];
  __shared__ float red[NV][3][16][64];                  // quarters 1-3 per value block
  const int hx = blockIdx.x;
  const int h = NV == 2 ? (hx >> 4) * 8 + (hx & 7) : hx;
  const int half = NV == 2 ? (hx >> 3) & 1 : 0;
  const int q0 = blockIdx.y * kFuQ;
  const int nqb = min(kFuQ, NQ - q0);
  const int w = h / (H / Hw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 31, g = lane >> 5, vb = wave % NV, kq = wave / NV;
  const int v0 = 32 * (NV * half + vb);   // this wave's first value row

  // (0) the chunk lse of this wave's queries (step 3), loaded first: loads complete in
  // issue order, so step 3 then waits for these alone, not for the weights and partials
  float lq[kFuQ / kWaves];
#pragma unroll
  for (int i = 0; i < kFuQ / kWaves; ++i) {
    const int n = wave + kWaves * i;
    lq[i] = (n < nqb && lane < S) ? lse_part[(static_cast<size_t>(q0 + n) * H + h) * S + lane]
                                  : -INFINITY;
  }
  // (1) this wave's weight rows: its quarter's 8 K-steps of 16 latent columns, in flight
  uint4 a[8];
  {
    const bf16_t* wr = w_uv + (static_cast<size_t>(w) * d_v + v0 + m) * d_c + 8 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      a[t] = *reinterpret_cast<const uint4*>(wr + 16 * (8 * kq + t));
  }
  // (2) the first batch of partials of merge pass 0
  const int cq = tid >> 7, c4 = 4 * (tid & 127);
  float4 v[kFuBatch];
  auto issue = [&](int n, int u0) {
    const float* op = o_part + (static_cast<size_t>(q0 + n) * H + h) * S * d_c + c4;
#pragma unroll
    for (int b = 0; b < kFuBatch; ++b)
      if (u0 + b < S) v[b] = *reinterpret_cast<const float4*>(op + static_cast<size_t>(u0 + b) * d_c);
  };
  if (cq < nqb) issue(cq, 0);
  // (3) chunk weights, 1 / sum and lse of every query: one wave per query, lane = split
#pragma unroll
  for (int i = 0; i < kFuQ / kWaves; ++i) {
    const int n = wave + kWaves * i;
    const float l = lq[i];
    float mx = l;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float e = 0.f, inv = 0.f;
    if (mx != -INFINITY) {
      const float ml = mx * kLog2e;
      float tot = 0.f;
      if (lane < S) {
        e = exp2f(fmaf(l, kLog2e, -ml));
        tot += e;
      }
      tot = wave_sum(tot);
      inv = 1.f / tot;
      if (lane == 0 && lse && half == 0)
        lse[static_cast<size_t>(q0 + n) * H + h] = mx + logf(tot);
    } else if (lane == 0 && lse && n < nqb && half == 0) {
      lse[static_cast<size_t>(q0 + n) * H + h] = -INFINITY;
    }
    wts[n][lane] = e;
    if (lane == 0) inv_s[n] = inv;
  }
  __syncthreads();
  // (4) merge, kPass queries x 512 columns per pass; rows past the block's queries are zeros
  for (int n = cq; n < kFuQ; n += kPass) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (n < nqb) {
      for (int u0 = 0; u0 < S; u0 += kFuBatch) {
        if (n != cq || u0 != 0) issue(n, u0);
#pragma unroll
        for (int b = 0; b < kFuBatch; ++b) {
          if (u0 + b >= S) break;
          const float wgt = wts[n][u0 + b];
          const bool use = wgt > 0.f;
          acc.x = fmaf(wgt, use ? v[b].x : 0.f, acc.x);
          acc.y = fmaf(wgt, use ? v[b].y : 0.f, acc.y);
          acc.z = fmaf(wgt, use ? v[b].z : 0.f, acc.z);
          acc.w = fmaf(wgt, use ? v[b].w : 0.f, acc.w);
        }
      }
      const float inv = inv_s[n];
      acc = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      if (half == 0)
        *reinterpret_cast<float4*>(o_lat + (static_cast<size_t>(q0 + n) * H + h) * d_c + c4) =
            acc;
    }
    const uint32_t bx = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc.x));
    const uint32_t by = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc.y));
    const uint32_t bz = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc.z));
    const uint32_t bw = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc.w));
    *reinterpret_cast<uint2*>(ob + n * kFuRow + c4) = make_uint2(bx | (by << 16), bz | (bw << 16));
  }
  __syncthreads();
  // (5) up-projection: one latent quarter per wave, accumulated from zero
  f32x16_t acc2 = {};
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int ks = 8 * kq + t;
    const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(ob + m * kFuRow + 16 * ks + 8 * g);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[t]), bv,
                                                   acc2, 0, 0, 0);
  }
  if (kq > 0) {
#pragma unroll
    for (int j = 0; j < 16; ++j) red[vb][kq - 1][j][lane] = acc2[j];
  }
  __syncthreads();
  // lane (query m, half g) holds value rows 8 (j / 4) + 4 g + j % 4 of block vb; the
  // quarters are summed in order 0, 1, 2, 3.  Stored as they are, each store instruction
  // writes 4-byte pieces of 32 query rows.  With whole heads (NV = 4) the sums are staged in
  // ob (free after the up-projection's operand reads, which the barrier above ends) as
  // [query][128 value rows] fp32 and leave as whole 512-byte rows (the ragged MTP step
  // ~2 us faster); with half heads the direct stores measured as fast.
  auto quarter_sum = [&](int j) {
    float t = acc2[j];
    t += red[vb][0][j][lane];
    t += red[vb][1][j][lane];
    t += red[vb][2][j][lane];
    return t;
  };
  if constexpr (NV == 2) {
    if (kq == 0 && m < nqb) {
      float* orow = out + (static_cast<size_t>(q0 + m) * H + h) * d_v + v0;
#pragma unroll
      for (int j = 0; j < 16; ++j) orow[8 * (j >> 2) + 4 * g + (j & 3)] = quarter_sum(j);
    }
  } else {
    constexpr int kOutRow = 32 * NV + 4;   // floats per staged row (padded)
    static_assert(kFuQ * kOutRow * 4 <= static_cast<int>(sizeof(ob)), "staged outputs exceed ob");
    float* ost = reinterpret_cast<float*>(ob);
    if (kq == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        ost[m * kOutRow + 32 * vb + 8 * (j >> 2) + 4 * g + (j & 3)] = quarter_sum(j);
    }
    __syncthreads();
    constexpr int kPerRow = 8 * NV;   // float4 per row
    for (int idx = tid; idx < nqb * kPerRow; idx += 256 * NV) {
      const int r = idx / kPerRow, c4 = 4 * (idx - r * kPerRow);
      *reinterpret_cast<float4*>(out + (static_cast<size_t>(q0 + r) * H + h) * d_v +
                                 32 * NV * half + c4) =
          *reinterpret_cast<const float4*>(ost + r * kOutRow + c4);
    }
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
  // 4 queries per block when there are at most 4 (no idle accumulators), else 8
  auto go = [&](auto qb) {
    constexpr int QB = decltype(qb)::value;
    constexpr int LANES = QB == 4 ? 16 : 32;
    constexpr int kCols = AbsLayout<LANES>::kCols;
    dim3 grid(s.n_heads, (s.d_c + kCols - 1) / kCols, (NQ + QB - 1) / QB);
    const size_t lds = sizeof(float) * QB * (s.d_nope + 4 * kCols);
    if (s.dtype == MLA_F32)
      hipLaunchKernelGGL((absorb_q_kernel<float, QB, LANES>), grid, dim3(256), lds, st,
                         static_cast<const float*>(q), static_cast<const float*>(w_uk),
                         static_cast<float*>(q_abs), NQ, s.n_heads, s.n_wheads, s.d_nope,
                         s.d_rope, s.d_c);
    else
      hipLaunchKernelGGL((absorb_q_kernel<bf16_t, QB, LANES>), grid, dim3(256), lds, st,
                         static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(w_uk),
                         static_cast<bf16_t*>(q_abs), NQ, s.n_heads, s.n_wheads, s.d_nope,
                         s.d_rope, s.d_c);
  };
  // fewer bf16 queries with 128-wide no-position parts: the streaming kernel
  if (s.dtype == MLA_BF16 && s.d_nope == 128 && s.d_c % kAsC == 0 && NQ < 16) {
    auto sk = [&](auto qbc) {
      constexpr int QB = decltype(qbc)::value;
      dim3 grid(s.n_heads, s.d_c / kAsC, (NQ + QB - 1) / QB);
      hipLaunchKernelGGL((absorb_q_stream_kernel<QB>), grid, dim3(256), 0, st,
                         static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(w_uk),
                         static_cast<bf16_t*>(q_abs), NQ, s.n_heads, s.n_wheads, s.d_rope,
                         s.d_c);
    };
    if (NQ <= 4)
      sk(std::integral_constant<int, 4>{});
    else
      sk(std::integral_constant<int, 8>{});
    return hipGetLastError();
  }
  // 16 or more bf16 queries with 128-wide no-position parts: the matrix-core kernel
  if (s.dtype == MLA_BF16 && s.d_nope == 128 && s.d_c % kAmC == 0 && NQ >= 16) {
    auto mf = [&](auto nbc) {
      constexpr int NB = decltype(nbc)::value;
      dim3 grid(s.n_heads, s.d_c / kAmC, (NQ + 32 * NB - 1) / (32 * NB));
      hipLaunchKernelGGL((absorb_q_mfma_kernel<NB>), grid, dim3(256), 0, st,
                         static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(w_uk),
                         static_cast<bf16_t*>(q_abs), NQ, s.n_heads, s.n_wheads, s.d_rope,
                         s.d_c);
    };
    if (NQ <= 32)
      mf(std::integral_constant<int, 1>{});
    else if (NQ <= 64)
      mf(std::integral_constant<int, 2>{});
    else
      mf(std::integral_constant<int, 4>{});
    return hipGetLastError();
  }
  if (NQ <= 4)
    go(std::integral_constant<int, 4>{});
  else
    go(std::integral_constant<int, kQB>{});
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
  else if (s.d_c % 16 == 0)
    hipLaunchKernelGGL(out_uv_mfma_kernel, dim3(s.n_heads, (s.d_v + 31) / 32),
                       dim3(64 * kUvmWaves), 0, st, o_lat, static_cast<const bf16_t*>(w_uv),
                       out, NQ, s.n_heads, s.n_wheads, s.d_c, s.d_v);
  else
    hipLaunchKernelGGL(out_uv_kernel<bf16_t>, grid, dim3(256), lds, st, o_lat,
                       static_cast<const bf16_t*>(w_uv), out, NQ, s.n_heads, s.n_wheads,
                       s.d_c, s.d_v);
  return hipGetLastError();
}

// Workgroups of the fused kernel with whole heads (NV = 4) and with half heads (NV = 2).
static int64_t fused_blocks(const mla_shape_t& s, int nv) {
  const int64_t nq = static_cast<int64_t>(s.batch) * s.s_q;
  return (4 / nv) * static_cast<int64_t>(s.n_heads) * ((nq + kFuQ - 1) / kFuQ);
}

bool combine_out_uv_supported(const mla_shape_t& s) {
  // Below one workgroup per CU the separate kernels, which spread the merge over
  // B s_q H workgroups, are faster (32 heads x 32 queries: 17.2 us fused against 5.9 +
  // 6.0 us; 128 heads x 4 queries: 13.9 against 9.9 + 8.2 us).
  return s.dtype == MLA_BF16 && s.d_c == 512 && s.d_v == 128 && s.n_splits <= 64 &&
         s.n_heads % 8 == 0 && fused_blocks(s, 2) >= 256;
}

hipError_t launch_combine_out_uv(const mla_shape_t& s, const float* o_part,
                                 const float* lse_part, const void* w_uv, float* o_lat,
                                 float* lse, float* out, hipStream_t st) {
  const int NQ = s.batch * s.s_q;
  const dim3 qb(1, (NQ + kFuQ - 1) / kFuQ);
  if (fused_blocks(s, 4) >= 256)
    hipLaunchKernelGGL(combine_out_uv_kernel<4>, dim3(s.n_heads, qb.y), dim3(1024), 0, st,
                       o_part, lse_part, static_cast<const bf16_t*>(w_uv), o_lat, lse, out, NQ,
                       s.n_heads, s.n_wheads, s.n_splits);
  else
    hipLaunchKernelGGL(combine_out_uv_kernel<2>, dim3(2 * s.n_heads, qb.y), dim3(512), 0, st,
                       o_part, lse_part, static_cast<const bf16_t*>(w_uv), o_lat, lse, out, NQ,
                       s.n_heads, s.n_wheads, s.n_splits);
  return hipGetLastError();
}

hipError_t launch_expand_cache(const mla_shape_t& s, const void* pool, const void* w_uk,
                               const void* w_uv, void* k, void* v, void* kr,
                               hipStream_t st) {
  if (expand_cache_mfma_supported(s))
    return launch_expand_cache_mfma(s, pool, w_uk, w_uv, k, v, kr, st);
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

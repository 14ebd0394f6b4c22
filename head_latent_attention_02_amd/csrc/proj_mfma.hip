// The projections around the decode path, unfolded and with the up-projections folded in
// offline ("How to upgrade GQA models to MLA...", Under the hood, Decompression Multiplex:
// by associativity W_UK can be multiplied into the query weights W^Q ahead of time, so the
// query lands in the latent space and keys are never decompressed; the value side folds
// W_UV into the output projection the same way).
//
// proj_mfma_kernel computes C[n][m] = sum_k W[m][k] X[n][k] for a bf16 weight W [M x K]
// (K contiguous) and a few token rows X [N x K] (bf16 or fp32): the query projections
// (W^Q or the folded W~^Q, M = H * row width, K = d_model) and the output projections (W^O
// or the folded W~^O, M = d_model, K = H * d_v or H * d_c).  Decode has few tokens, so this
// is a weight stream: one workgroup per 64 weight rows (and, when that gives too few
// workgroups, per K range, the partial sums added with fp32 atomics into a zeroed output).
// Weight tiles of 64 rows x 256 K go through LDS (coalesced 512-byte row pieces in, matrix-
// core operands out); the token rows are read straight from L2.  v_mfma_f32_32x32x16_bf16
// with fp32 accumulation; the four waves split (32-row block, K half) and the two K halves
// are added through LDS.  The query projections rotate their RoPE rows in the epilogue, at
// each token's position t = T_b - s_q + s, with the cache key's rotation (pairs
// (2i, 2i+1) turned by t * base^(-2i / d_rope)).
//
// fold_q_kernel / fold_o_kernel build the folded weights once (offline), fp32 accumulate and
// one rounding to bf16:  W~^Q[h] = [W_UK[w(h)]^T W^Q_nope[h] ; W^Q_rope[h]],
// W~^O[:, h d_c + c] = sum_i W^O[:, h d_v + i] W_UV[w(h)][i][c].
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPM = 64;      // weight rows per workgroup
constexpr int kPK = 256;     // K per tile
constexpr int kPN = 32;      // tokens per matrix-core block
constexpr int kPNB = 4;      // token blocks per workgroup: 128 tokens (grid z covers more)

struct ProjSmem {
  union {
    u32x4 w[2][kPM * kPK / 8];        // two weight tiles, 16-byte chunks (64 KB)
    float part[kPNB][2][64 * 16];     // after the last tile: the K-half-1 partial sums of
                                      // each token block's two row blocks (32 KB)
  };
};

// chunk ch (of 32) of tile row r sits at chunk ch ^ (r & 15): the operand reads take one
// chunk from each of 16 consecutive rows (conflict-free), the staging stores whole rows
__device__ __forceinline__ int pswz(int r, int ch) { return ch ^ (r & 15); }

__device__ __forceinline__ bf16x8 load_x8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
// fp32 token rows (the output projections' input) are rounded to bf16 for the matrix cores,
// to nearest even, two per v_cvt_pk_bf16_f32: a software rounding cost ~5 VALU instructions
// per value here, more than the tile's MFMAs
__device__ __forceinline__ bf16x8 load_x8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  const bf16x8 v = {static_cast<__bf16>(a.x), static_cast<__bf16>(a.y),
                    static_cast<__bf16>(a.z), static_cast<__bf16>(a.w),
                    static_cast<__bf16>(b.x), static_cast<__bf16>(b.y),
                    static_cast<__bf16>(b.z), static_cast<__bf16>(b.w)};
  return v;
}

template <typename XT, typename OT, bool ATOMIC>
__global__ __launch_bounds__(256, 2) void proj_mfma_kernel(
    const bf16_t* __restrict__ W, int M, int K, const XT* __restrict__ X, int N,
    OT* __restrict__ C, int ldc, int k_split, int block_dim, int lat_dim, int rope_dim,
    const int32_t* __restrict__ lens, int s_q, double log_base) {
  __shared__ __attribute__((aligned(16))) ProjSmem sm;
  const int m0 = blockIdx.x * kPM;
  const int ka = blockIdx.y * k_split;
  const int kb = min(ka + k_split, K);
  // up to kPNB blocks of 32 tokens, so the weights stream once for up to 128 tokens
  const int n0 = blockIdx.z * kPN * kPNB;
  const int nbc = min(kPNB, (N - n0 + kPN - 1) / kPN);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n32 = lane & 31, g = lane >> 5;
  const int rb = wave & 1, kh = wave >> 1;
  const int n_tiles = (kb - ka) / kPK;
  // tile staging: thread chunk j covers row (tid + 256 j) / 32, 16-byte chunk (tid & 31)
  u32x4 stg[8];
  auto load_tile = [&](int t) {
    const int k0 = ka + t * kPK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + 256 * j, r = c >> 5, ch = c & 31;
      stg[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          W + static_cast<size_t>(m0 + r) * K + k0 + 8 * ch));
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + 256 * j, r = c >> 5, ch = c & 31;
      sm.w[buf][r * 32 + pswz(r, ch)] = stg[j];
    }
  };
  f32x16 acc[kPNB];
#pragma unroll
  for (int nb = 0; nb < kPNB; ++nb) acc[nb] = f32x16{};
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
    if (n_tiles > 1) load_tile(1);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      const int buf = t & 1;
      const int k0 = ka + t * kPK;
      // the wave's 8 K-steps of this tile: A = weight rows 32 rb + n32, B = token
      // n0 + 32 nb + n32 of each token block
      const int r = 32 * rb + n32;
      bf16x8 a[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int ks = 8 * kh + s;
        a[s] = __builtin_bit_cast(bf16x8, sm.w[buf][r * 32 + pswz(r, 2 * ks + g)]);
      }
#pragma unroll
      for (int nb = 0; nb < kPNB; ++nb) {
        if (nb < nbc) {
          const int n = n0 + kPN * nb + n32;
          const XT* xrow = X + static_cast<size_t>(n < N ? n : 0) * K + k0 + 8 * g;
          bf16x8 b[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) b[s] = n < N ? load_x8(xrow + 16 * (8 * kh + s)) : bf16x8{};
#pragma unroll
          for (int s = 0; s < 8; ++s)
            acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], acc[nb], 0, 0, 0);
        }
      }
      if (t + 1 < n_tiles) {
        store_tile(buf ^ 1);          // its last readers finished before the last barrier
        if (t + 2 < n_tiles) load_tile(t + 2);
      }
      __syncthreads();
    }
  }
  // add the K-half-1 partials of each row block (the weight tiles' LDS is free: every wave
  // passed the last tile's barrier)
  if (kh == 1) {
#pragma unroll
    for (int nb = 0; nb < kPNB; ++nb)
      if (nb < nbc) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.part[nb][rb][i * 64 + lane] = acc[nb][i];
      }
  }
  __syncthreads();
  if (kh == 1) return;
  // lane holds token n, rows m0 + 32 rb + 8 (i / 4) + 4 g + i % 4
  const int mb = m0 + 32 * rb + 4 * g;
#pragma unroll
  for (int nb = 0; nb < kPNB; ++nb) {
    const int n = n0 + kPN * nb + n32;
    if (nb >= nbc || n >= N) continue;
    f32x16 v = acc[nb];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] += sm.part[nb][rb][i * 64 + lane];
    if (rope_dim > 0) {
      const int b_ = n / s_q, s_ = n - b_ * s_q;
      const double pos = static_cast<double>(lens[b_] - s_q + s_);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const int m = mb + 8 * (i >> 2) + (i & 3);
        const int rr = m % block_dim - lat_dim;
        if (rr >= 0) {                  // an even RoPE row and its partner m + 1
          const double ang = pos * exp(-log_base * static_cast<double>(rr) / rope_dim);
          const float c = static_cast<float>(cos(ang)), sn = static_cast<float>(sin(ang));
          const float x0 = v[i], x1 = v[i + 1];
          v[i] = x0 * c - x1 * sn;
          v[i + 1] = x0 * sn + x1 * c;
        }
      }
    }
    OT* crow = C + static_cast<size_t>(n) * ldc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = mb + 8 * q;
      if constexpr (ATOMIC) {
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(crow + m + e, v[4 * q + e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) stf(crow + m + e, v[4 * q + e]);
      }
    }
  }
}

// W~^Q[h][c][d] = sum_i W_UK[w(h)][i][c] W^Q[h][i][d] (c < d_c), then the RoPE rows copied.
// One thread per (h, row c, 8 columns d).
__global__ __launch_bounds__(256) void fold_q_kernel(const bf16_t* __restrict__ w_q,
                                                     const bf16_t* __restrict__ w_uk,
                                                     bf16_t* __restrict__ w_qf, int H, int Hw,
                                                     int d_c, int d_n, int d_r, int d_model) {
  const int D = d_c + d_r, dq = d_n + d_r;
  const size_t per_head = static_cast<size_t>(D) * (d_model / 8);
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= per_head * H) return;
  const int h = static_cast<int>(idx / per_head);
  const size_t rem = idx - static_cast<size_t>(h) * per_head;
  const int row = static_cast<int>(rem / (d_model / 8));
  const int d8 = static_cast<int>(rem - static_cast<size_t>(row) * (d_model / 8)) * 8;
  const bf16_t* wq_h = w_q + static_cast<size_t>(h) * dq * d_model;
  bf16_t* dst = w_qf + (static_cast<size_t>(h) * D + row) * d_model + d8;
  if (row >= d_c) {                   // RoPE rows: unchanged
    *reinterpret_cast<u32x4*>(dst) =
        *reinterpret_cast<const u32x4*>(wq_h + static_cast<size_t>(d_n + row - d_c) * d_model + d8);
    return;
  }
  const bf16_t* uk = w_uk + static_cast<size_t>(h / (H / Hw)) * d_n * d_c + row;
  float acc[8] = {};
  for (int i = 0; i < d_n; ++i) {
    const float u = bf16_bits_to_f32(uk[static_cast<size_t>(i) * d_c]);
    const u32x4 v = *reinterpret_cast<const u32x4*>(wq_h + static_cast<size_t>(i) * d_model + d8);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += u * __uint_as_float(w4[e] << 16);
      acc[2 * e + 1] += u * __uint_as_float(w4[e] & 0xffff0000u);
    }
  }
  u32x4 o;
  o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
  o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
  o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
  o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
  *reinterpret_cast<u32x4*>(dst) = o;
}

// W~^O[m][h d_c + c] = sum_i W^O[m][h d_v + i] W_UV[w(h)][i][c].  One thread per
// (row m, head h, 8 columns c).
__global__ __launch_bounds__(256) void fold_o_kernel(const bf16_t* __restrict__ w_o,
                                                     const bf16_t* __restrict__ w_uv,
                                                     bf16_t* __restrict__ w_of, int H, int Hw,
                                                     int d_c, int d_v, int d_model) {
  const size_t per_row = static_cast<size_t>(H) * (d_c / 8);
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= per_row * d_model) return;
  const int m = static_cast<int>(idx / per_row);
  const size_t rem = idx - static_cast<size_t>(m) * per_row;
  const int h = static_cast<int>(rem / (d_c / 8));
  const int c8 = static_cast<int>(rem - static_cast<size_t>(h) * (d_c / 8)) * 8;
  const bf16_t* wo = w_o + static_cast<size_t>(m) * H * d_v + static_cast<size_t>(h) * d_v;
  const bf16_t* uv = w_uv + static_cast<size_t>(h / (H / Hw)) * d_v * d_c + c8;
  float acc[8] = {};
  for (int i = 0; i < d_v; ++i) {
    const float a = bf16_bits_to_f32(wo[i]);
    const u32x4 v = *reinterpret_cast<const u32x4*>(uv + static_cast<size_t>(i) * d_c);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += a * __uint_as_float(w4[e] << 16);
      acc[2 * e + 1] += a * __uint_as_float(w4[e] & 0xffff0000u);
    }
  }
  u32x4 o;
  o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
  o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
  o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
  o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
  *reinterpret_cast<u32x4*>(w_of + static_cast<size_t>(m) * H * d_c +
                            static_cast<size_t>(h) * d_c + c8) = o;
}

// More than 32 token rows: a matrix-product tiling instead of the weight stream above.  The
// stream reads every token row once per 64 weight rows, which from 128 tokens on moves four
// times the weight bytes through each CU; here a workgroup takes 256 weight rows x 128
// tokens, K in steps of 64, with both operands staged through LDS (double-buffered, 96 KB),
// so the token rows are read once per 256 weight rows.  Wave w: weight rows 64 w .. +64 (two
// 32-row blocks) x the 128 tokens (four 32-token blocks), eight accumulators.
constexpr int kGM = 256;     // weight rows per workgroup
constexpr int kGN = 128;     // tokens per workgroup
constexpr int kGK = 64;      // K per tile

struct GemmSmem {
  u32x4 a[2][kGM * kGK / 8];  // weight tiles [row][8 chunks of 8 bf16] (2 x 32 KB)
  u32x4 b[2][kGN * kGK / 8];  // token tiles, the same layout (2 x 16 KB)
};

// chunk c of row r sits at chunk c ^ ((r >> 1) & 7): a 128-byte row covers half the banks,
// so rows r and r ^ 1 use the two halves and the swizzle spreads 16 rows over all of them
__device__ __forceinline__ int gswz(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ u32x4 pack_x8(const bf16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 pack_x8(const float* p) {
  return __builtin_bit_cast(u32x4, load_x8(p));
}

template <typename XT, typename OT, bool ATOMIC>
__global__ __launch_bounds__(256, 1) void proj_gemm_kernel(
    const bf16_t* __restrict__ W, int M, int K, const XT* __restrict__ X, int N,
    OT* __restrict__ C, int ldc, int k_split, int block_dim, int lat_dim, int rope_dim,
    const int32_t* __restrict__ lens, int s_q, double log_base) {
  __shared__ __attribute__((aligned(16))) GemmSmem sm;
  const int m0 = blockIdx.x * kGM;
  const int ka = blockIdx.y * k_split;
  const int kb = min(ka + k_split, K);
  const int n0 = blockIdx.z * kGN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n32 = lane & 31, g = lane >> 5;
  const int n_tiles = (kb - ka) / kGK;
  // staging: weight chunk j of a thread is row (tid + 256 j) / 8, chunk tid % 8 (eight
  // threads read a row's 128 contiguous bytes); token chunks the same, four per thread
  u32x4 sa[8], sb[4];
  auto load_tile = [&](int t) {
    const int k0 = ka + t * kGK;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = tid + 256 * j, r = f >> 3, c = f & 7;
      sa[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          W + static_cast<size_t>(m0 + r) * K + k0 + 8 * c));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = tid + 256 * j, r = f >> 3, c = f & 7;
      const int n = n0 + r;
      sb[j] = n < N ? pack_x8(X + static_cast<size_t>(n) * K + k0 + 8 * c) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int f = tid + 256 * j, r = f >> 3, c = f & 7;
      sm.a[buf][r * 8 + gswz(r, c)] = sa[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int f = tid + 256 * j, r = f >> 3, c = f & 7;
      sm.b[buf][r * 8 + gswz(r, c)] = sb[j];
    }
  };
  f32x16 acc[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[rb][tb] = f32x16{};
  load_tile(0);
  store_tile(0);
  if (n_tiles > 1) load_tile(1);
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    // four K-steps of 16: A = weight row 64 wave + 32 rb + n32, B = token 32 tb + n32, both
    // 8 values at K offset 16 s + 8 g (chunk 2 s + g)
#pragma unroll
    for (int s = 0; s < kGK / 16; ++s) {
      bf16x8 a[2], b[4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = 64 * wave + 32 * rb + n32;
        a[rb] = __builtin_bit_cast(bf16x8, sm.a[buf][r * 8 + gswz(r, 2 * s + g)]);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int r = 32 * tb + n32;
        b[tb] = __builtin_bit_cast(bf16x8, sm.b[buf][r * 8 + gswz(r, 2 * s + g)]);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[rb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[rb], b[tb], acc[rb][tb], 0, 0, 0);
    }
    if (t + 1 < n_tiles) {
      store_tile(buf ^ 1);          // its last readers finished before the last barrier
      if (t + 2 < n_tiles) load_tile(t + 2);
    }
    __syncthreads();
  }
  // lane holds token 32 tb + n32 of the block, rows m0 + 64 wave + 32 rb + 8 (i / 4) + 4 g
  // + i % 4
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int n = n0 + 32 * tb + n32;
    if (n >= N) continue;
    OT* crow = C + static_cast<size_t>(n) * ldc;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      f32x16 v = acc[rb][tb];
      const int mb = m0 + 64 * wave + 32 * rb + 4 * g;
      if (rope_dim > 0) {
        const int b_ = n / s_q, s_ = n - b_ * s_q;
        const double pos = static_cast<double>(lens[b_] - s_q + s_);
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const int m = mb + 8 * (i >> 2) + (i & 3);
          const int rr = m % block_dim - lat_dim;
          if (rr >= 0) {                  // an even RoPE row and its partner m + 1
            const double ang = pos * exp(-log_base * static_cast<double>(rr) / rope_dim);
            const float c = static_cast<float>(cos(ang)), sn = static_cast<float>(sin(ang));
            const float x0 = v[i], x1 = v[i + 1];
            v[i] = x0 * c - x1 * sn;
            v[i + 1] = x0 * sn + x1 * c;
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = mb + 8 * q;
        if constexpr (ATOMIC) {
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(crow + m + e, v[4 * q + e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) stf(crow + m + e, v[4 * q + e]);
        }
      }
    }
  }
}

__global__ void zero_f32_kernel(float* p, size_t n) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// C = W X^T for M rows of W, K wide, N token rows; splits K over workgroups (fp32 atomics
// into a zeroed C) when 64-row blocks alone give fewer than ~1024 workgroups, at most
// 512 / N splits.
template <typename XT, typename OT>
hipError_t launch_proj(const bf16_t* W, int M, int K, const XT* X, int N, OT* C, int ldc,
                       int block_dim, int lat_dim, int rope_dim, const int32_t* lens, int s_q,
                       double log_base, hipStream_t st) {
  if (N > kPN && M % kGM == 0 && K % kGK == 0) {
    const int gm = M / kGM, gn = (N + kGN - 1) / kGN;
    int gs = (256 + gm * gn - 1) / (gm * gn);             // about one workgroup per CU
    gs = max(1, min(gs, min(K / kGK, 512 / N)));
    if constexpr (!std::is_same<OT, float>::value) gs = 1;
    if (rope_dim > 0) gs = 1;
    const int ks = ((K / kGK + gs - 1) / gs) * kGK;
    gs = (K + ks - 1) / ks;
    const dim3 grid(gm, gs, gn);
    if (gs > 1) {
      if constexpr (std::is_same<OT, float>::value) {
        const size_t n = static_cast<size_t>(N) * ldc;
        hipLaunchKernelGGL(zero_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                           dim3(256), 0, st, C, n);
        hipLaunchKernelGGL((proj_gemm_kernel<XT, OT, true>), grid, dim3(256), 0, st, W, M, K, X,
                           N, C, ldc, ks, block_dim, lat_dim, rope_dim, lens, s_q, log_base);
      }
    } else {
      hipLaunchKernelGGL((proj_gemm_kernel<XT, OT, false>), grid, dim3(256), 0, st, W, M, K, X,
                         N, C, ldc, ks, block_dim, lat_dim, rope_dim, lens, s_q, log_base);
    }
    return hipGetLastError();
  }
  const int m_blocks = M / kPM, n_blocks = (N + kPN * kPNB - 1) / (kPN * kPNB);
  int splits = (1024 + m_blocks * n_blocks - 1) / (m_blocks * n_blocks);
  splits = max(1, min(splits, K / kPK));
  // every split adds N x M partial sums with atomics: keep splits x N within 512 x M
  splits = max(1, min(splits, 512 / max(N, 1)));
  if constexpr (!std::is_same<OT, float>::value) splits = 1;   // bf16 outputs: no atomics
  if (rope_dim > 0) splits = 1;                                 // rotate complete sums only
  const int k_split = ((K / kPK + splits - 1) / splits) * kPK;
  splits = (K + k_split - 1) / k_split;
  const dim3 grid(m_blocks, splits, n_blocks);
  if (splits > 1) {
    if constexpr (std::is_same<OT, float>::value) {
      const size_t n = static_cast<size_t>(N) * ldc;
      hipLaunchKernelGGL(zero_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                         0, st, C, n);
      hipLaunchKernelGGL((proj_mfma_kernel<XT, OT, true>), grid, dim3(256), 0, st, W, M, K, X,
                         N, C, ldc, k_split, block_dim, lat_dim, rope_dim, lens, s_q, log_base);
    }
  } else {
    hipLaunchKernelGGL((proj_mfma_kernel<XT, OT, false>), grid, dim3(256), 0, st, W, M, K, X,
                       N, C, ldc, k_split, block_dim, lat_dim, rope_dim, lens, s_q, log_base);
  }
  return hipGetLastError();
}

}  // namespace

bool projections_supported(const mla_shape_t& s, int d_model) {
  return s.dtype == MLA_BF16 && d_model > 0 && d_model % kPK == 0 &&
         (s.n_heads * (s.d_nope + s.d_rope)) % kPM == 0 &&
         (s.n_heads * (s.d_c + s.d_rope)) % kPM == 0 && d_model % kPM == 0 &&
         (s.n_heads * s.d_v) % kPK == 0 && (s.n_heads * s.d_c) % kPK == 0 &&
         s.d_rope % 2 == 0;
}

hipError_t launch_project_q(const mla_shape_t& s, int d_model, float rope_base, const void* x,
                            const void* w, const int32_t* lens, void* q, bool folded,
                            hipStream_t st) {
  const int width = folded ? s.d_c + s.d_rope : s.d_nope + s.d_rope;
  const int lat = folded ? s.d_c : s.d_nope;
  return launch_proj(static_cast<const bf16_t*>(w), s.n_heads * width, d_model,
                     static_cast<const bf16_t*>(x), s.batch * s.s_q, static_cast<bf16_t*>(q),
                     s.n_heads * width, width, lat, s.d_rope, lens, s.s_q,
                     log(static_cast<double>(rope_base)), st);
}

hipError_t launch_out_project(const mla_shape_t& s, int d_model, const float* in,
                              const void* w, float* y, bool folded, hipStream_t st) {
  const int K = s.n_heads * (folded ? s.d_c : s.d_v);
  return launch_proj(static_cast<const bf16_t*>(w), d_model, K, in, s.batch * s.s_q, y,
                     d_model, 1, 1, 0, nullptr, 1, 0.0, st);
}

hipError_t launch_fold_q(const mla_shape_t& s, int d_model, const void* w_q, const void* w_uk,
                         void* w_qf, hipStream_t st) {
  const size_t n = static_cast<size_t>(s.n_heads) * (s.d_c + s.d_rope) * (d_model / 8);
  hipLaunchKernelGGL(fold_q_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     st, static_cast<const bf16_t*>(w_q), static_cast<const bf16_t*>(w_uk),
                     static_cast<bf16_t*>(w_qf), s.n_heads, s.n_wheads, s.d_c, s.d_nope,
                     s.d_rope, d_model);
  return hipGetLastError();
}

hipError_t launch_fold_o(const mla_shape_t& s, int d_model, const void* w_o, const void* w_uv,
                         void* w_of, hipStream_t st) {
  const size_t n = static_cast<size_t>(d_model) * s.n_heads * (s.d_c / 8);
  hipLaunchKernelGGL(fold_o_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     st, static_cast<const bf16_t*>(w_o), static_cast<const bf16_t*>(w_uv),
                     static_cast<bf16_t*>(w_of), s.n_heads, s.n_wheads, s.d_c, s.d_v, d_model);
  return hipGetLastError();
}

}  // namespace mla

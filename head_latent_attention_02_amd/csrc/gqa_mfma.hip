// Matrix-core (MFMA) GQA-path decode over the expanded per-group cache, bf16, with
// d_nope = d_v = 128, d_rope = 64, page 64 and at most 16 query rows per group.
//
// What it computes: for query row (s, h) of group j = w(h) and chunk u, the split-KV
// partials of softmax attention with keys [K_j[t] ; k^R[t]] and values V_j[t] over the
// chunk's visible tokens (AI Radio episode on GQLA, "Key concepts": the GQA path keeps
// per-group keys and values, the RoPE key is shared; "How to upgrade GQA models to
// MLA...", Under the hood: both paths give the same attention).
//
// The path streams 4224 bytes per token (8 groups x 256 B of K and V, plus 128 B of
// k^R) for 20 KFLOP, so it is bound by HBM and every design choice serves streaming:
//  * One workgroup = one (sequence b, chunk u, group j); its 4 waves take the chunk's
//    32-token tiles round robin, each with a private online softmax, and merge at the
//    end through LDS.  No barrier inside the loop.
//  * Every load instruction reads whole rows: 16 lanes per 256-byte K_j or V_j row, 8
//    lanes per 128-byte k^R row, so each touches only full cache lines.  The rows go
//    through a wave-private 20 KB LDS tile (16-byte chunks XOR-swizzled per token) that
//    re-lays them out for v_mfma_f32_32x32x16_bf16: keys as the A operand of
//    S^T = K Q^T (token = M, query row = N), values read back transposed with
//    ds_read_b64_tr_b16 as the A operand of O^T += V^T P^T.  P comes straight from the
//    score accumulators: the token order of the value product is permuted to match the
//    score layout, so P never leaves the lane that computed it.
//  * Latency is hidden across waves rather than inside one: the LDS (80 KB, the tiles and
//    the final merge buffers share it) and the registers (under 256) fit two workgroups,
//    8 waves, per CU, so while one wave waits for its tile the others compute.  (A
//    register ping-pong of two tiles per wave needs ~435 registers and allows one
//    workgroup per CU; it measured 2-3 % slower.)
//  * Workgroups of one (b, u) sit 8 apart in the grid so that all groups of a chunk run
//    on one XCD and share its L2 for the k^R rows.
// Rows past the chunk end are loaded from the tile's first token (valid data) and
// masked, so NaN padding in a last page never reaches an MFMA.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kDN = 128;            // no-position key width
constexpr int kDV = 128;            // value width
constexpr int kDR = 64;             // RoPE key width
constexpr int kPage = 64;
constexpr int kTT = 32;             // tokens per tile
constexpr int kKN = kDN / 16;       // 8 K-steps over K_j
constexpr int kKR = kDR / 16;       // 4 K-steps over k^R
constexpr int kWaves = 4;
constexpr int kMaxRows = 16;        // query rows per group (s_q * H / G)
constexpr int kVRowB = kDV * 2;     // 256-byte value rows in LDS

constexpr int kKRowB = kDN * 2;     // 256-byte key rows
constexpr int kRRowB = kDR * 2;     // 128-byte RoPE-key rows

// One tile's rows in registers on their way to LDS (16 bytes per lane and load).
struct Tile {
  u32x4 k[8];      // load i: K_j[4 i + lane / 16][8 (lane % 16), +8)
  u32x4 r[4];      // load i: k^R[8 i + lane / 8][8 (lane % 8), +8)
  u32x4 v[8];      // load i: V_j[4 i + lane / 16][8 (lane % 16), +8)
};

struct WaveTile {
  char k[kTT * kKRowB];
  char r[kTT * kRRowB];
  char v[kTT * kVRowB];
};

struct Args {
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* kr;
  const int32_t* ptb;   // page-table row of sequence b
  int G, j, lo, hi;
  int num_pages;        // pool bound, for checked builds
  unsigned int* bad;    // bad-page flag, for checked builds
};

struct Red {
  float o[kWaves][kMaxRows][kDV];   // per-wave O, after the loop
  float m[kWaves][32];
  float l[kWaves][32];
};
struct Smem {
  union {
    WaveTile tile[kWaves];   // per-wave row tiles
    Red red;                 // after the loop (80 KB in all: two workgroups per CU)
  };
};

// chunk swizzles: keys and RoPE keys are read 16 tokens x one chunk at a time, values
// 4 tokens x two chunks at a time (transposed)
__device__ __forceinline__ int kswz(int tok) { return tok & 15; }
__device__ __forceinline__ int rswz(int tok) { return tok & 7; }
__device__ __forceinline__ int vswz(int tok) { return 2 * (tok & 3); }

__device__ __forceinline__ u32x4 ld_stream(const bf16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ void load_tile(Tile& tl, const Args& a, int t0, int lane) {
  const int page = checked_page(a.ptb[t0 >> 6], a.num_pages, a.bad);
  const size_t slot0 = static_cast<size_t>(page) * kPage + (t0 & (kPage - 1));
  const int valid = a.hi - t0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tv = 4 * i + (lane >> 4);
    const size_t sv = (slot0 + ((tv < valid) ? tv : 0)) * a.G + a.j;
    tl.k[i] = ld_stream(a.k + sv * kDN + 8 * (lane & 15));
    tl.v[i] = ld_stream(a.v + sv * kDV + 8 * (lane & 15));
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = 8 * i + (lane >> 3);
    const size_t sr = slot0 + ((tr < valid) ? tr : 0);
    tl.r[i] = *reinterpret_cast<const u32x4*>(a.kr + sr * kDR + 8 * (lane & 7));
  }
}

__device__ __forceinline__ float xhalf_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct RowState {
  float m;   // running maximum (log2 units), -inf before the first visible token
  float l;   // this lane's share of the running sum
};

// One tile: scores, online softmax, value product.  vl = visible tokens of this lane's
// row in the tile (tokens 0 .. vl-1).
__device__ __forceinline__ void process_tile(const Tile& tl, const bf16x8 (&qn)[kKN],
                                             const bf16x8 (&qr)[kKR], WaveTile& wt,
                                             const int (&rdo)[2][2], int vl, float zscale,
                                             int lane, RowState& st, f32x16 (&acc)[4]) {
  const int g = lane >> 5, m = lane & 31;
  // rows into the wave's LDS tile (swizzled 16-byte chunks)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = 4 * i + (lane >> 4), c = lane & 15;
    *reinterpret_cast<u32x4*>(wt.k + t * kKRowB + ((c ^ kswz(t)) * 16)) = tl.k[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 8 * i + (lane >> 3), c = lane & 7;
    *reinterpret_cast<u32x4*>(wt.r + t * kRRowB + ((c ^ rswz(t)) * 16)) = tl.r[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = 4 * i + (lane >> 4), c = lane & 15;
    *reinterpret_cast<u32x4*>(wt.v + t * kVRowB + ((c ^ vswz(t)) * 16)) = tl.v[i];
  }
  // S^T = K Q^T: lane (token m, half g) takes chunk 2 ks + g of its key row
  f32x16 s = {};
#pragma unroll
  for (int ks = 0; ks < kKN; ++ks) {
    const bf16x8 ak = *reinterpret_cast<const bf16x8*>(
        wt.k + m * kKRowB + (((2 * ks + g) ^ kswz(m)) * 16));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qn[ks], s, 0, 0, 0);
  }
#pragma unroll
  for (int ks = 0; ks < kKR; ++ks) {
    const bf16x8 ar = *reinterpret_cast<const bf16x8*>(
        wt.r + m * kRRowB + (((2 * ks + g) ^ rswz(m)) * 16));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar, qr[ks], s, 0, 0, 0);
  }
  char* vt = wt.v;
  // lane (row n, half g) holds tokens 8 (jj / 4) + 4 g + jj % 4
  float mx = -INFINITY;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj)
    if (8 * (jj >> 2) + 4 * g + (jj & 3) < vl) mx = fmaxf(mx, s[jj]);
  mx = xhalf_max(mx * zscale);
  const float m_new = fmaxf(st.m, mx);
  if (__builtin_amdgcn_ballot_w64(m_new > st.m)) {
    const float alpha = (st.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][e] *= alpha;
    st.m = m_new;
  }
  const bool live = st.m != -INFINITY;
  bf16x8 pb[2];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const bool vis = live && (8 * (jj >> 2) + 4 * g + (jj & 3) < vl);
    const float p = vis ? __builtin_amdgcn_exp2f(fmaf(s[jj], zscale, -st.m)) : 0.f;
    st.l += p;
    pb[jj >> 3][jj & 7] = static_cast<__bf16>(p);
  }
  // O^T[col][row] += V^T P^T over the tile's 32 tokens, in the score layout's order
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int cofs = 64 * mb;   // 32 columns = 4 chunks of 16 bytes
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(__attribute__((address_space(3))) char*)(vt + (rdo[kt][0] ^ cofs)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(__attribute__((address_space(3))) char*)(vt + (rdo[kt][1] ^ cofs)));
      const bf16x8 av = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kt], acc[mb], 0, 0, 0);
    }
}

__global__ __launch_bounds__(256, 2) void gqa_decode_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kpool,
    const bf16_t* __restrict__ vpool, const bf16_t* __restrict__ krpool,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens,
    float* __restrict__ o_part, float* __restrict__ lse_part, int s_q, int H, int G,
    int max_pages, int S, int split_tokens, float zscale, int n_units, int num_pages,
    unsigned int* bad) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  const int wg = blockIdx.x;
  const int rest = wg >> 3;
  const int j = rest % G;
  const int unit = (rest / G) * 8 + (wg & 7);
  if (unit >= n_units) return;   // uniform for the workgroup, before any barrier
  const int b = unit / S, u = unit - b * S;
  const int T = checked_len(lens[b], max_pages * kPage, bad);
  Args a;
  a.k = kpool;
  a.v = vpool;
  a.kr = krpool;
  a.ptb = pt + static_cast<size_t>(b) * max_pages;
  a.num_pages = num_pages;
  a.bad = bad;
  a.G = G;
  a.j = j;
  split_range(T, u, S, kPage, split_tokens, a.lo, a.hi);
  const int n_tiles = (a.hi > a.lo) ? (a.hi - a.lo + kTT - 1) / kTT : 0;
  const int hg = H / G, R = s_q * hg;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;

  // query operand: row n = (s, hh)
  bf16x8 qn[kKN], qr[kKR];
  int row_lim = 0;   // exclusive token bound of this lane's row
  {
    const int r = (n < R) ? n : 0;
    const int s = r / hg, h = j * hg + (r - s * hg);
    const bf16_t* qp = q + ((static_cast<size_t>(b) * s_q + s) * H + h) * (kDN + kDR);
    const bf16x8 zero = {};
#pragma unroll
    for (int ks = 0; ks < kKN; ++ks)
      qn[ks] = (n < R) ? *reinterpret_cast<const bf16x8*>(qp + 16 * ks + 8 * g) : zero;
#pragma unroll
    for (int ks = 0; ks < kKR; ++ks)
      qr[ks] = (n < R) ? *reinterpret_cast<const bf16x8*>(qp + kDN + 16 * ks + 8 * g) : zero;
    row_lim = min(a.hi, T - s_q + s + 1);
  }
  // transposed-read byte offsets (column block 0) for the two halves of each K-step
  int rdo[2][2];
  {
    const int q16 = lane >> 4, L = lane & 15;
    const int mh = q16 & 1, gg = q16 >> 1;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int tok = 16 * kt + 8 * hf + 4 * gg + (L >> 2);
        const int c16 = 2 * mh + ((L & 3) >> 1);
        rdo[kt][hf] = tok * kVRowB + ((c16 ^ vswz(tok)) * 16) + 8 * (L & 1);
      }
  }
  // column block mb adds 4 mb to the chunk index (whose block-0 value is below 4), so
  // the swizzled byte offset of block mb is rdo ^ (64 mb)
  WaveTile& wt = sm.tile[wave];

  RowState st = {-INFINITY, 0.f};
  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x16{};

  for (int k = wave; k < n_tiles; k += kWaves) {
    Tile A;
    load_tile(A, a, a.lo + k * kTT, lane);
    process_tile(A, qn, qr, wt, rdo, row_lim - (a.lo + k * kTT), zscale, lane, st, acc);
  }

  // merge the 4 waves: each writes its O into the LDS the tiles used
  __syncthreads();
  const float l_tot = xhalf_sum(st.l);
  if (g == 0) {
    sm.red.m[wave][n] = st.m;
    sm.red.l[wave][n] = l_tot;
  }
  if (n < R) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        sm.red.o[wave][n][32 * mb + 8 * (e >> 2) + 4 * g + (e & 3)] = acc[mb][e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < R * kDV; idx += blockDim.x) {
    const int r = idx / kDV, c = idx - r * kDV;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.red.m[w][r]);
    float o = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float mw = sm.red.m[w][r];
        const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        lsum += f * sm.red.l[w][r];
        o += f * sm.red.o[w][r][c];
      }
    }
    const int s = r / hg, h = j * hg + (r - s * hg);
    const size_t orow = ((static_cast<size_t>(b) * s_q + s) * H + h) * S + u;
    o_part[orow * kDV + c] = (lsum > 0.f) ? o / lsum : 0.f;
    if (c == 0) lse_part[orow] = (lsum > 0.f) ? (M + log2f(lsum)) * kLn2 : -INFINITY;
  }
}

}  // namespace

bool gqa_decode_mfma_supported(const mla_shape_t& s) {
  return s.dtype == MLA_BF16 && s.d_nope == kDN && s.d_v == kDV && s.d_rope == kDR &&
         s.page_size == kPage && s.s_q * (s.n_heads / s.n_wheads) <= kMaxRows;
}

hipError_t launch_gqa_decode_mfma(const mla_shape_t& s, const void* q, const void* k,
                                  const void* v, const void* kr, const int32_t* pt,
                                  const int32_t* lens, float* o_part, float* lse_part,
                                  unsigned int* bad, hipStream_t st) {
  const int n_units = s.batch * s.n_splits;
  const unsigned grid = static_cast<unsigned>((n_units + 7) / 8) * 8u * s.n_wheads;
  hipLaunchKernelGGL(gqa_decode_mfma_kernel, dim3(grid), dim3(256), 0, st,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(kr), pt, lens,
                     o_part, lse_part, s.s_q, s.n_heads, s.n_wheads, s.max_pages,
                     s.n_splits, s.split_tokens, s.softmax_scale * kLog2e, n_units,
                     s.num_pages, bad);
  return hipGetLastError();
}

}  // namespace mla

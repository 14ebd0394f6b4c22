// Matrix-core (MFMA) absorbed decode for bf16 latent caches with d_c = 512, d_rope = 64.
//
// What it computes is the split-KV form of absorbed MLA attention: per chunk u and
// query row (s, h), softmax over the chunk's visible tokens of
// z_t = sigma <q_abs, [c_t ; k^R_t]>, reducing over the latent c_t itself
// ("MLA and GRPO architecture", s.2: the cached state is [c_t, k^R_t];
// "How to upgrade GQA models to MLA...", Under the hood: with W_UK folded onto the
// query the keys are never decompressed; AI Radio episode on GQLA, "Key concepts": on
// the MQA-absorb path the latent is the shared key and value).
//
// Two kernels share the pipeline below.  One workgroup per (sequence b, chunk u, row
// block), one per CU (~160 KB of LDS); rows are the flattened (s, h) pairs.  Blocks of 64
// rows run eight waves, two per SIMD: two score waves (32 rows each), two loader waves that
// only stream the chunk, and four value waves (128 latent columns each), placed so that
// every SIMD carries about the same matrix work (36 or 32 MFMAs per slot) and has a second
// wave to issue while the first waits.  Blocks of 32 rows (GQLA's absorbed shape) run three
// waves, one per SIMD: one score wave and two value waves (256 columns each) that also
// stream the chunk.  Both contractions run as v_mfma_f32_32x32x16_bf16: S^T[token][row] =
// C_tile . q_abs^T over the 576-wide row, and O^T[latent][row] += C_tile^T . P^T over the
// tile's 32 tokens.  Per 32-token tile ("slot" s, one workgroup barrier each):
//  * The streaming waves keep a 4-deep LDS ring: each loads half of tile s+3 into
//    registers during slot s (buffer loads; the buffer's size is the tile's valid rows, so
//    rows past the chunk end read as zeros) and stores it at the start of slot s+2, so a
//    load has two slots to land (two register buffers alternate).
//  * The value waves multiply tile s-2, reading it transposed with ds_read_b64_tr_b16 as
//    the A operand; O^T stays in the accumulators.
//  * The score waves (32 rows each, q_abs held in registers as the B operand) issue the 36
//    MFMAs of tile s and, between them, the softmax of tile s-1 in small pieces that issue
//    while the matrix core is busy; P (bf16) goes to LDS for the value waves.
//  * The softmax keeps a lazy per-row reference: it only moves when a tile's maximum exceeds
//    it by more than a slack of 32 (log2 units), so P stays below 2^32.  When it moves, the
//    score wave rescales the row's running sum by 2^(old - new) and publishes that factor
//    with P; the value waves rescale the row's accumulators by it before adding the tile.
//    Every chunk is one pass over its tiles whatever the scores do (a move costs the value
//    waves one multiply per accumulator).
//  * The row blocks of one (b, u) are 8 workgroups apart in the grid so that they run on
//    the same XCD and share its L2.
#include <math.h>
#include <stdlib.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = 576;        // cache row width (d_c + d_rope)
constexpr int kDC = 512;       // latent width
constexpr int kPage = 64;      // tokens per page
constexpr int kTT = 32;        // tokens per tile
constexpr int kKS = kD / 16;   // 36 K-steps of 16 in the score contraction
constexpr int kPRow = 40;      // P row stride in LDS (bf16): 80 B, conflict-free b128 reads

struct Work {
  const bf16_t* q_abs;
  const bf16_t* pool;
  const int32_t* ptb;   // page-table row of sequence b
  float* o_part;
  float* lse_part;
  size_t qrow0;         // first query row of this workgroup (global row index)
  int lo, hi, n_tiles, T, s_q, H, y, S, u;
  float zscale;
  float slack;          // lazy-reference slack (log2 units)
  int num_pages;        // pool bound, for checked builds
  unsigned int* bad;    // bad-page flag, for checked builds
};

namespace ring {

constexpr int kRowB = kD * 2;              // 1152 bytes per cache row
constexpr int kTileB = kTT * kRowB;        // 36864 bytes per tile
constexpr int kNB = 4;                     // ring depth in tiles
constexpr int kLoads = kTileB / 1024 / 2;  // 18 of a tile's 36 1-KB loads per value wave

// XOR swizzle of the 16-byte chunk index inside a ring row (rows are 1152 bytes, so
// consecutive rows start half a bank cycle apart).  Score reads take one chunk from each
// of 16 consecutive rows: rows of equal parity get 8 distinct chunks, so a 16-lane pass
// is conflict-free.  Transposed reads take two chunks from each of 4 consecutive rows
// aligned to 4: rows t and t+2 differ in swizzle bits 1-2, so they never share a pair.
// (Measured on gfx950: 130 B/clk/CU for the score pattern vs 98 with a swizzle that only
// separates 8 consecutive rows.)
__device__ __forceinline__ int rswz(int tok) { return (((tok >> 1) & 1) << 2) | ((tok >> 2) & 3); }

struct Smem {
  char ring[kNB][kTileB];
  bf16_t pbuf[2][64 * kPRow];
  float lfin[64];
  float alpha[2][64];  // [tile & 1][row]: factor the accumulators take before that tile
  int moved[2][2];     // [tile & 1][score wave]: some row of the wave moved its reference
  uint32_t plan[2][kLoads / 2][64];   // value wave VW's per-lane load offsets
};

// The softmax of tile k runs in slot k+1 and writes alpha[k & 1] and moved[k & 1] there; the
// value waves read them in slot k+2 (after the barrier ending slot k+1), before multiplying
// tile k, and the next write of that parity is in slot k+3.

// One wave's share of a tile, in registers between its global loads and its LDS stores.
template <int NL>
struct Stage {
  u32x4 r[NL];
};

// Ring byte 16*c of a tile holds chunk (c % 72) ^ rswz(c / 72) of tile row c / 72; load j
// of a wave covers ring bytes [1024 (first + stride j), +1024), 16 per lane, so each load
// instruction reads about 1 KB of consecutive cache rows.  The loads go through a buffer
// resource whose base is the tile's first row and whose size is the tile's valid rows:
// the per-lane byte offsets are fixed for the whole kernel (one register per load), and
// rows past a chunk's end (only in its last tile) read as zeros, which are masked later.
// Block b + 18 holds the same chunks as block b, 16 rows (18432 bytes) further down (the
// swizzle ignores row bit 4), so a wave's 18 loads need only 9 offset registers.  The
// distance is added to the per-lane offset (not passed as the scalar offset), so the
// buffer's range check, which covers the per-lane offset, still zeroes rows past the end.
constexpr int kHalfRowsB = 16 * kRowB;

// The offsets sit in LDS (read back once per tile), which keeps 9 registers free in the
// value waves: their loop is one register short of spilling otherwise.
__device__ __forceinline__ void make_plan(uint32_t (&pl)[kLoads / 2][64], int lane, int vw) {
#pragma unroll
  for (int j = 0; j < kLoads / 2; ++j) {
    const int c = (vw + 2 * j) * 64 + lane;
    const int row = c / 72;
    pl[j][lane] = static_cast<uint32_t>(row * kD + (((c - row * 72) ^ rswz(row)) * 8)) * 2u;
  }
}

// gfx9 buffer resource word 3 for raw (untyped) dword access
constexpr int kBufWord3 = 0x00020000;
constexpr int kSlc = 2;   // streaming (non-temporal) cache policy

// Value wave vw's loads: j < 9 cover blocks vw + 2 j, j >= 9 the blocks 18 further on.
__device__ __forceinline__ void load_stage(Stage<kLoads>& st,
                                           const uint32_t (&pl)[kLoads / 2][64],
                                           const Work& w, int kt, int lane) {
  const int t0 = __builtin_amdgcn_readfirstlane(w.lo + kt * kTT);
  // wave-uniform (readfirstlane): the buffer resource must live in scalar registers
  const int valid = __builtin_amdgcn_readfirstlane(max(min(w.hi - t0, kTT), 0));
  // an empty chunk (valid == 0) reads nothing, not even its page-table entry
  int page = 0;
  if (valid > 0) page = checked_page(w.ptb[t0 >> 6], w.num_pages, w.bad);
  const bf16_t* base = w.pool + (static_cast<size_t>(page) * kPage + (t0 & (kPage - 1))) * kD;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(base), 0, valid * kRowB, kBufWord3);
#pragma unroll
  for (int j = 0; j < kLoads / 2; ++j) {
    const uint32_t off = pl[j][lane];
    st.r[j] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kSlc);
    st.r[j + kLoads / 2] =
        __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + kHalfRowsB, 0, kSlc);
  }
}

template <int NL>
__device__ __forceinline__ void store_stage(Smem& sm, const Stage<NL>& st, int lane, int kt,
                                            int first, int stride) {
  // the per-lane part of the address is formed here, at each use: a copy kept live
  // across the whole pass gets spilled, and its reload would wait on every load in flight
  int lofs = lane * 16 + first * 1024;
  asm volatile("" : "+v"(lofs));
  char* dst = &sm.ring[kt & (kNB - 1)][0] + lofs;
#pragma unroll
  for (int j = 0; j < NL; ++j)
    *reinterpret_cast<u32x4*>(dst + stride * j * 1024) = st.r[j];
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

// One score-wave slot: the 36 MFMAs of S^T for the tile at `tb` (into sacc_out) and the
// softmax of the previous tile's scores (sacc_in).  The softmax is cut into pieces of a
// few VALU instructions that sit between consecutive MFMAs, where they issue while the
// matrix core is busy (gfx950 hides about four VALU instructions behind each 32x32x16
// MFMA; larger pieces stall it).  Lane (row n32, half g) holds tokens 8 (j / 4) + 4 g +
// j % 4 of a tile; lim = visible tokens of its row there (MASK: some lane has lim < 32).
template <bool DO_MFMA, bool DO_SOFT, bool MASK, int SPF = 8>
__device__ __forceinline__ void score_slot(const char* tb, const bf16x8 (&qreg)[kKS],
                                           const int (&rb)[4], f32x16& sacc_out,
                                           const f32x16& sacc_in, int lim, float zscale,
                                           float slack, float& m_ref, float& l_run,
                                           bool& move, float& alpha, bf16_t* prow, int g) {
  // A operands run kPF K-steps ahead of the MFMA that consumes them
  constexpr int kPF = SPF;
  bf16x8 abuf[kPF];
  f32x16 acc = {};
  if (DO_MFMA) {
#pragma unroll
    for (int ks = 0; ks < kPF; ++ks)
      abuf[ks] = *reinterpret_cast<const bf16x8*>(tb + rb[ks & 3] + 128 * (ks >> 2));
  }
  float z[16], mx4[4];
  float nm = 0.f;
  bool live = false;
  uint32_t pk[2];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) {
    if (DO_MFMA) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(abuf[ks % kPF], qreg[ks], acc, 0, 0, 0);
      if (ks + kPF < kKS) {
        const int kn = ks + kPF;
        abuf[ks % kPF] = *reinterpret_cast<const bf16x8*>(tb + rb[kn & 3] + 128 * (kn >> 2));
      }
    }
    if (DO_SOFT) {
      if (ks < 4) {                       // scores out of the accumulators (masked)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * ks + i;
          z[j] = sacc_in[j];
          if (MASK && !(8 * ks + 4 * g + i < lim)) z[j] = -INFINITY;
        }
      } else if (ks < 8) {                // row maximum, four at a time
        const int q = ks - 4;
        mx4[q] = fmaxf(fmaxf(z[4 * q], z[4 * q + 1]), fmaxf(z[4 * q + 2], z[4 * q + 3]));
      } else if (ks == 8) {
        const float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
        mx4[0] = xhalf_max(mx * zscale);
      } else if (ks == 9) {
        // The first visible tile of a row fixes its reference; a later jump past the
        // slack raises it to this tile's maximum, and what was summed so far is rescaled
        // to the new reference (here the running sum, in the value waves the accumulators).
        const float mt = mx4[0];
        move = m_ref != -INFINITY && mt > m_ref + slack;
        alpha = move ? __builtin_amdgcn_exp2f(m_ref - mt) : 1.f;
        if (m_ref == -INFINITY || move) m_ref = mt;
        l_run *= alpha;
        live = m_ref != -INFINITY;
        nm = -m_ref;
      } else if (ks < 18) {               // two probabilities per step, bf16 pairs
        const int j = 2 * (ks - 10);
        float pv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          pv[i] = live ? __builtin_amdgcn_exp2f(fmaf(z[j + i], zscale, nm)) : 0.f;
          l_run += pv[i];
        }
        pk[(j >> 1) & 1] = __builtin_bit_cast(
            uint32_t, __builtin_shufflevector(
                          __builtin_bit_cast(__bf16 __attribute__((ext_vector_type(1))),
                                             static_cast<__bf16>(pv[0])),
                          __builtin_bit_cast(__bf16 __attribute__((ext_vector_type(1))),
                                             static_cast<__bf16>(pv[1])),
                          0, 1));
        if ((j & 3) == 2) {               // four tokens 8 (j / 4) + 4 g .. +3 are done
          *reinterpret_cast<uint2*>(prow + 8 * (j >> 2) + 4 * g) = make_uint2(pk[0], pk[1]);
        }
      }
    }
    // keep the read for step ks+kPF and this step's softmax piece next to MFMA ks
    __builtin_amdgcn_sched_barrier(0);
  }
  if (DO_MFMA) sacc_out = acc;
}

// Score wave QW (rows 32 QW .. 32 QW + 31).  Slot s: the MFMAs of tile s and the softmax
// (P, published to LDS) of tile s-1, so the value waves use tile s-2.
template <int NQ, int QW, int SPF = 8>
__device__ __forceinline__ void score_wave(Smem& sm, const Work& w, int lane) {
  const int n32 = lane & 31, g = lane >> 5;
  bf16x8 qreg[kKS];
  const int r = w.y * 32 * NQ + 32 * QW + n32;
  const int top_row = min(w.hi, w.T - w.s_q + r / w.H + 1);
  const bf16_t* qp = w.q_abs + (w.qrow0 + 32 * QW + n32) * kD + 8 * g;
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
  const int sw = rswz(n32);
  int rb[4];                         // byte offset of chunk 2b+g of this lane's row
#pragma unroll
  for (int b4 = 0; b4 < 4; ++b4) rb[b4] = n32 * kRowB + 16 * ((2 * b4 + g) ^ sw);
  const int n = w.n_tiles;
  float m_ref = -INFINITY, l_run = 0.f;
  f32x16 sacc[2];
  // one slot; P = parity of s (sacc[P] takes tile s, sacc[1 - P] holds tile s-1).
  // Slots run in turns of two (even, odd) and every wave leaves the loop only at the end of
  // a turn, so the value waves' loop has a single exit; a turn may run one slot past n + 1,
  // which does no work.  Returns true when the pass is over (at an odd slot).
  auto slot = [&](auto par, int s) -> bool {
    constexpr int P = decltype(par)::value;
    const bool mf = s < n, sf = s >= 1 && s <= n;
    const char* tb = &sm.ring[s & (kNB - 1)][0];
    const int lim = top_row - (w.lo + (s - 1) * kTT);
    bf16_t* prow = &sm.pbuf[(s - 1) & 1][(32 * QW + n32) * kPRow];
    bool move = false;
    float alpha = 1.f;
    const bool masked = __builtin_amdgcn_ballot_w64(lim < kTT) != 0;
    if (mf && sf && !masked)
      score_slot<true, true, false, SPF>(tb, qreg, rb, sacc[P], sacc[1 - P], lim, w.zscale,
                                    w.slack, m_ref, l_run, move, alpha, prow, g);
    else if (mf && sf)
      score_slot<true, true, true, SPF>(tb, qreg, rb, sacc[P], sacc[1 - P], lim, w.zscale,
                                   w.slack, m_ref, l_run, move, alpha, prow, g);
    else if (mf)
      score_slot<true, false, false, SPF>(tb, qreg, rb, sacc[P], sacc[1 - P], lim, w.zscale,
                                     w.slack, m_ref, l_run, move, alpha, prow, g);
    else if (sf)
      score_slot<false, true, true, SPF>(tb, qreg, rb, sacc[P], sacc[1 - P], lim, w.zscale,
                                    w.slack, m_ref, l_run, move, alpha, prow, g);
    if (sf) {   // tile s-1's rescale factors, for the value waves in slot s+1
      if (g == 0) sm.alpha[(s - 1) & 1][32 * QW + n32] = alpha;
      const bool any = __builtin_amdgcn_ballot_w64(move) != 0;
      if (n32 == 0 && g == 0) sm.moved[(s - 1) & 1][QW] = any ? 1 : 0;
    }
    __syncthreads();
    return P == 1 && s >= n + 1;
  };
  __syncthreads();   // the streaming waves have stored tile 0
  for (int s = 0;; s += 2) {
    slot(std::integral_constant<int, 0>(), s);
    if (slot(std::integral_constant<int, 1>(), s + 1)) break;
  }
  const float l_tot = xhalf_sum(l_run);
  if (g == 0) {
    sm.lfin[32 * QW + n32] = l_tot;
    const size_t orow = (w.qrow0 + 32 * QW + n32) * w.S + w.u;
    w.lse_part[orow] = (l_tot > 0.f) ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
  }
  __syncthreads();
}

// One value-wave tile from ring slot `slot`: acc (+)= C^T . P^T.  The transposed
// A-operand reads run four (mb, kt) steps ahead of their MFMA pair.
template <int NQ, bool FIRST, int KMB = 8>
__device__ __forceinline__ void value_ring_tile(Smem& sm, int slot, int pb_i,
                                                const int (&trofs)[2][2][2], int n32, int g,
                                                f32x16 (&acc)[KMB][NQ]) {
  bf16x8 pb[2][NQ];
  // per-lane offset formed at each use (see store_stage): the constant parts fold into
  // the LDS instructions' offset field
  int pofs = n32 * kPRow + 8 * g;
  asm volatile("" : "+v"(pofs));
  const bf16_t* pbase = &sm.pbuf[pb_i][0] + pofs;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int nb = 0; nb < NQ; ++nb)
      pb[kt][nb] = *reinterpret_cast<const bf16x8*>(pbase + 32 * nb * kPRow + 16 * kt);
  const char* cb = &sm.ring[slot][0];
  // the 8 base offsets, opaque per tile, so that their per-block variants are formed
  // here (one add each) rather than kept live across the loop
  int to[2][2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        to[a][b][c] = trofs[a][b][c];
      }
  auto read_a = [&](int step) -> bf16x8 {
    const int mb = step >> 1, kt = step & 1;
    const int ofs = 128 * (mb >> 1);
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(const __attribute__((address_space(3))) char*)(
            cb + to[mb & 1][kt][0] + ofs));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(const __attribute__((address_space(3))) char*)(
            cb + to[mb & 1][kt][1] + ofs));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  constexpr int kSteps = 2 * KMB, kPF = 4;
  bf16x8 abuf[kPF];
#pragma unroll
  for (int st = 0; st < kPF; ++st) abuf[st] = read_a(st);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    const int mb = st >> 1, kt = st & 1;
#pragma unroll
    for (int nb = 0; nb < NQ; ++nb) {
      if (FIRST && kt == 0) {
        const f32x16 zero = {};
        acc[mb][nb] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(abuf[st % kPF], pb[kt][nb], zero, 0, 0, 0);
      } else {
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(abuf[st % kPF], pb[kt][nb],
                                                              acc[mb][nb], 0, 0, 0);
      }
    }
    if (st + kPF < kSteps) abuf[st % kPF] = read_a(st + kPF);
    // keep the reads for step st+kPF between MFMA pairs st and st+1
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Before the value waves add tile k: if some row's reference moved in tile k, every row's
// accumulators take that row's factor (1 for rows that did not move).  Lane (n32, g) holds
// rows 32 nb + n32 of the block.
template <int KMB, int NQ>
__device__ __forceinline__ void rescale_if_moved(Smem& sm, int k, int n32,
                                                 f32x16 (&acc)[KMB][NQ]) {
  int any = sm.moved[k & 1][0];
  if (NQ > 1) any |= sm.moved[k & 1][1];
  if (__builtin_amdgcn_readfirstlane(any)) {
#pragma unroll
    for (int nb = 0; nb < NQ; ++nb) {
      const float a = sm.alpha[k & 1][32 * nb + n32];
#pragma unroll
      for (int mb = 0; mb < KMB; ++mb) acc[mb][nb] *= a;
    }
  }
}

// Value wave VW of the 32-row layout: latent columns [256 VW, 256 VW + 256) of the block's
// rows (32 NQ).  It also streams half of every tile through the ring (below) and, in slot s,
// multiplies tile s-2.
// A value wave's epilogue: its 32 NQ rows x 32 KMB latent columns of O^T, each row scaled
// by 1 / (its softmax sum), go to o_part.  In the MFMA layout a store instruction would
// write 32-byte pieces of 32 rows; the ring is free once every wave has passed the last
// barrier, so the block is staged there row-major (each of at most NVW value waves in its
// own part) and leaves in whole 1-KB row segments, which shortens the burst of partial
// writes that ends the kernel.  Same products as a direct store, so the same bits.
template <int NQ, int KMB, int NVW>
__device__ __forceinline__ void write_partials(Smem& sm, const Work& w, int vw, int lat0,
                                               const f32x16 (&acc)[KMB][NQ], int lane) {
  constexpr int kCols = 32 * KMB, kRows = 32 * NQ;
  constexpr int kStg = kCols + 4;          // floats per staged row (padded)
  constexpr int kPerRow = kCols / 4;       // float4 per row
  static_assert(NVW * kRows * kStg * 4 <= static_cast<int>(sizeof(sm.ring)),
                "staged partials exceed the ring");
  static_assert(64 % kPerRow == 0 || kPerRow % 64 == 0, "row segments and the wave");
  const int n32 = lane & 31, g = lane >> 5;
  float* stg = reinterpret_cast<float*>(&sm.ring[0][0]) + vw * kRows * kStg;
#pragma unroll
  for (int nb = 0; nb < NQ; ++nb) {
    const float l = sm.lfin[32 * nb + n32];
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    float* srow = stg + (32 * nb + n32) * kStg + 4 * g;
#pragma unroll
    for (int mb = 0; mb < KMB; ++mb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float4 v;
        v.x = acc[mb][nb][4 * a + 0] * inv;
        v.y = acc[mb][nb][4 * a + 1] * inv;
        v.z = acc[mb][nb][4 * a + 2] * inv;
        v.w = acc[mb][nb][4 * a + 3] * inv;
        *reinterpret_cast<float4*>(srow + 32 * mb + 8 * a) = v;
      }
  }
  // read back by this wave only (its LDS operations complete in order): instruction i
  // covers 256 consecutive floats of the block, row r = idx / kPerRow
  float* obase = w.o_part + (w.qrow0 * w.S + w.u) * kDC + lat0;
#pragma unroll 8
  for (int i = 0; i < kRows * kPerRow / 64; ++i) {
    const int idx = 64 * i + lane, r = idx / kPerRow, c4 = 4 * (idx - r * kPerRow);
    const float4 v = *reinterpret_cast<const float4*>(stg + r * kStg + c4);
    *reinterpret_cast<float4*>(obase + static_cast<size_t>(r) * w.S * kDC + c4) = v;
  }
}

template <int NQ, int VW>
__device__ __forceinline__ void value_wave(Smem& sm, const Work& w, int lane) {
  const int n32 = lane & 31, g = lane >> 5;
  constexpr int lat0 = VW * 256;
  const int q16 = lane >> 4, L = lane & 15;
  const int m_base = 16 * (q16 & 1), g16 = q16 >> 1;
  int trofs[2][2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h4 = 0; h4 < 2; ++h4) {
        const int col = lat0 + 32 * par + m_base + 4 * (L & 3);
        const int tok = 16 * kt + 8 * g16 + 4 * h4 + (L >> 2);
        trofs[par][kt][h4] = tok * kRowB + (((col >> 3) ^ rswz(tok)) * 16) + (col & 7) * 2;
      }
  const int n = w.n_tiles;
  // this wave streams 1-KB blocks VW, VW + 2, ... of every tile, two tiles ahead: tile
  // s+1 is loaded into registers during slot s-2 and stored into the ring at the start of
  // slot s (its ring slot held tile s-3, last read by the value waves in slot s-1), so
  // every load has two whole slots to land.  Two register buffers alternate: tile t lives
  // in stg[t & 1].  Slot s multiplies tile s-2 (its P was published in slot s-1).
  Stage<kLoads> stg[2];
  uint32_t (&plan)[kLoads / 2][64] = sm.plan[VW];
  make_plan(plan, lane, VW);
  {
    // Loads and stores are unconditional: past the last tile they repeat tile n-1 into
    // ring slot (s+1) % 4, which no wave reads in slot s and no later slot needs.
    const int last = max(n - 1, 0);
    // prologue: tile 0 in the ring, tiles 1 and 2 in registers
    load_stage(stg[0], plan, w, 0, lane);
    load_stage(stg[1], plan, w, min(1, last), lane);
    store_stage(sm, stg[0], lane, 0, VW, 2);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(stg[0], plan, w, min(2, last), lane);
    __syncthreads();
    // slots 0 and 1: the score waves start; tiles 1 and 2 go into the ring
    store_stage(sm, stg[1], lane, 1, VW, 2);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(stg[1], plan, w, min(3, last), lane);
    __syncthreads();
    store_stage(sm, stg[0], lane, 2, VW, 2);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(stg[0], plan, w, min(4, last), lane);
    __syncthreads();
    if (n == 0) {
      __syncthreads();   // the score waves have published the row sums
      float* orow0 = w.o_part + (w.qrow0 * w.S + w.u) * kDC + lat0 + 4 * g;
      for (int nb = 0; nb < NQ; ++nb)
        for (int c = 0; c < 256; c += 8)
          *reinterpret_cast<float4*>(orow0 + (32 * nb + n32) * w.S * kDC + c) =
              make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    // slot s stores tile s+1 from stg[(s+1) & 1], reloads that buffer with tile s+3 and
    // multiplies tile s-2 (none past the last tile: a turn can run one slot past n+1)
    f32x16 acc[8][NQ];
    auto vslot = [&](auto par, int s) {
      constexpr int X = decltype(par)::value;   // (s + 1) & 1
      store_stage(sm, stg[X], lane, s + 1, VW, 2);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(stg[X], plan, w, min(s + 3, last), lane);
      __builtin_amdgcn_sched_barrier(0);
      if (s - 2 < n) {
        rescale_if_moved<8, NQ>(sm, s - 2, n32, acc);
        value_ring_tile<NQ, false>(sm, (s - 2) & (kNB - 1), (s - 2) & 1, trofs, n32, g, acc);
      }
      __syncthreads();
    };
    // turn (2, 3); slot 2 is peeled so the accumulators are first written outside the loop
    store_stage(sm, stg[1], lane, 3, VW, 2);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(stg[1], plan, w, min(5, last), lane);
    __builtin_amdgcn_sched_barrier(0);
    value_ring_tile<NQ, true>(sm, 0, 0, trofs, n32, g, acc);
    __syncthreads();
    vslot(std::integral_constant<int, 0>(), 3);
    // turns (4, 5), (6, 7), ...: the pass ends after the turn holding slot n + 1
    if (n + 1 > 3) {
      for (int s = 4;; s += 2) {
        vslot(std::integral_constant<int, 1>(), s);
        vslot(std::integral_constant<int, 0>(), s + 1);
        if (s + 1 >= n + 1) break;
      }
    }
    __syncthreads();   // the score waves have published the row sums
    write_partials<NQ, 8, 2>(sm, w, VW, lat0, acc, lane);
    return;
  }
}


// Eight-wave layout (64 query rows): loader wave LW streams ring blocks LW, LW + 2, ... of
// every tile exactly as the value waves of the 32-row layout do (two tiles ahead, two
// register buffers), and does nothing else; the same slots, turns and barriers as every
// other wave.
template <int LW>
__device__ __forceinline__ void loader_wave(Smem& sm, const Work& w, int lane) {
  const int n = w.n_tiles;
  Stage<kLoads> stg[2];
  uint32_t (&plan)[kLoads / 2][64] = sm.plan[LW];
  make_plan(plan, lane, LW);
  {
    const int last = max(n - 1, 0);
    load_stage(stg[0], plan, w, 0, lane);
    load_stage(stg[1], plan, w, min(1, last), lane);
    store_stage(sm, stg[0], lane, 0, LW, 2);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(stg[0], plan, w, min(2, last), lane);
    __syncthreads();
    store_stage(sm, stg[1], lane, 1, LW, 2);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(stg[1], plan, w, min(3, last), lane);
    __syncthreads();
    store_stage(sm, stg[0], lane, 2, LW, 2);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(stg[0], plan, w, min(4, last), lane);
    __syncthreads();
    if (n == 0) {
      __syncthreads();
      return;
    }
    auto lslot = [&](auto par, int s) {
      constexpr int X = decltype(par)::value;
      store_stage(sm, stg[X], lane, s + 1, LW, 2);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(stg[X], plan, w, min(s + 3, last), lane);
      __syncthreads();
    };
    store_stage(sm, stg[1], lane, 3, LW, 2);
    __builtin_amdgcn_sched_barrier(0);
    load_stage(stg[1], plan, w, min(5, last), lane);
    __syncthreads();
    lslot(std::integral_constant<int, 0>(), 3);
    if (n + 1 > 3) {
      for (int s = 4;; s += 2) {
        lslot(std::integral_constant<int, 1>(), s);
        lslot(std::integral_constant<int, 0>(), s + 1);
        if (s + 1 >= n + 1) break;
      }
    }
    __syncthreads();
    return;
  }
}

// Eight-wave layout: value wave VW (0..3) owns latent columns [128 VW, 128 VW + 128) of the
// 64 rows (128 accumulator registers); slot s multiplies tile s-2.
template <int VW>
__device__ __forceinline__ void value_wave128(Smem& sm, const Work& w, int lane) {
  constexpr int NQ = 2, KMB = 4;
  const int n32 = lane & 31, g = lane >> 5;
  constexpr int lat0 = VW * 128;
  const int q16 = lane >> 4, L = lane & 15;
  const int m_base = 16 * (q16 & 1), g16 = q16 >> 1;
  int trofs[2][2][2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h4 = 0; h4 < 2; ++h4) {
        const int col = lat0 + 32 * par + m_base + 4 * (L & 3);
        const int tok = 16 * kt + 8 * g16 + 4 * h4 + (L >> 2);
        trofs[par][kt][h4] = tok * kRowB + (((col >> 3) ^ rswz(tok)) * 16) + (col & 7) * 2;
      }
  const int n = w.n_tiles;
  {
    __syncthreads();
    __syncthreads();
    __syncthreads();
    if (n == 0) {
      __syncthreads();
      float* orow0 = w.o_part + (w.qrow0 * w.S + w.u) * kDC + lat0 + 4 * g;
      for (int nb = 0; nb < NQ; ++nb)
        for (int c = 0; c < 128; c += 8)
          *reinterpret_cast<float4*>(orow0 + (32 * nb + n32) * w.S * kDC + c) =
              make_float4(0.f, 0.f, 0.f, 0.f);
      return;
    }
    f32x16 acc[KMB][NQ];
    auto vslot = [&](int s) {
      if (s - 2 < n) {
        rescale_if_moved<KMB, NQ>(sm, s - 2, n32, acc);
        value_ring_tile<NQ, false, KMB>(sm, (s - 2) & (kNB - 1), (s - 2) & 1, trofs, n32, g,
                                        acc);
      }
      __syncthreads();
    };
    value_ring_tile<NQ, true, KMB>(sm, 0, 0, trofs, n32, g, acc);
    __syncthreads();
    vslot(3);
    if (n + 1 > 3) {
      for (int s = 4;; s += 2) {
        vslot(s);
        vslot(s + 1);
        if (s + 1 >= n + 1) break;
      }
    }
    __syncthreads();
    write_partials<NQ, KMB, 4>(sm, w, VW, lat0, acc, lane);
    return;
  }
}

}  // namespace ring

// Workgroup -> (sequence, chunk, row block): the row blocks of one (b, u) are 8 workgroups
// apart, so they run on the same XCD.  When every workgroup of the grid has a CU at once,
// XCD x (workgroup % 8) takes the x-th contiguous range of the (b, u) units, so that an XCD
// holds the chunks of few sequences and its L2 fetches only their q_abs rows (decode at
// 16 x 4096 tokens ~0.7 us, at 4 x 131072 ~1 us faster).  In longer grids consecutive units
// go to consecutive XCDs, which spreads every sequence over all XCDs and keeps their queues
// balanced when lengths differ (contiguous ranges made the ragged MTP decode 627 -> 769 us).
// The grid's padding workgroups return (uniform for the whole workgroup, before any
// barrier).  Expanded inside each kernel: filled through a helper, the page-table reads lose
// their scalar (s_load) form, and a vector read of a page entry waits, through the in-order
// load counter, for every tile load in flight.
#define MLA_SETUP_WORK(NQ)                                                           \
  Work w;                                                                          \
  {                                                                                \
    const int wg = blockIdx.x;                                                     \
    const int rest = wg >> 3;                                                      \
    const int y = rest % n_yblk;                                                   \
    const int unit = xcd_ranges ? (wg & 7) * ((n_units + 7) >> 3) + rest / n_yblk   \
                                : (rest / n_yblk) * 8 + (wg & 7);                  \
    if (unit >= n_units) return;                                                   \
    const int b = unit / S;                                                        \
    w.u = unit - b * S;                                                            \
    w.T = checked_len(lens[b], max_pages * kPage, bad);                            \
    split_range(w.T, w.u, S, kPage, split_tokens, w.lo, w.hi);                     \
    w.n_tiles = (w.hi > w.lo) ? (w.hi - w.lo + kTT - 1) / kTT : 0;                 \
    w.q_abs = q_abs;                                                               \
    w.pool = pool;                                                                 \
    w.ptb = pt + static_cast<size_t>(b) * max_pages;                               \
    w.o_part = o_part;                                                             \
    w.lse_part = lse_part;                                                         \
    w.qrow0 = static_cast<size_t>(b) * s_q * H + static_cast<size_t>(y) * 32 * (NQ); \
    w.s_q = s_q;                                                                   \
    w.H = H;                                                                       \
    w.y = y;                                                                       \
    w.S = S;                                                                       \
    w.zscale = zscale;                                                             \
    w.slack = slack;                                                               \
    w.num_pages = num_pages;                                                       \
    w.bad = bad;                                                                   \
  }

// 32 query rows per workgroup, one wave per SIMD (the ring takes 158 KB of LDS), so the
// scheduler may use the whole register file of each SIMD for operand prefetch: wave 0
// scores, waves 1 and 2 stream the chunk and multiply.
__global__ __launch_bounds__(192, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_absorbed_mfma_r32_kernel(
    const bf16_t* __restrict__ q_abs, const bf16_t* __restrict__ pool,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens,
    float* __restrict__ o_part, float* __restrict__ lse_part, int s_q, int H, int max_pages,
    int S, int split_tokens, float zscale, float slack, int n_units, int n_yblk,
    int xcd_ranges, int num_pages, unsigned int* bad) {
  constexpr int NQ = 1;
  __shared__ __attribute__((aligned(16))) ring::Smem sm;
  MLA_SETUP_WORK(NQ)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (wave == 0)
    ring::score_wave<NQ, 0>(sm, w, lane);
  else if (wave == 1)
    ring::value_wave<NQ, 0>(sm, w, lane);
  else
    ring::value_wave<NQ, 1>(sm, w, lane);
}

// 64 query rows per workgroup, eight waves, two per SIMD (wave w runs on SIMD w % 4):
// score waves 0 and 1 share SIMDs 0 and 1 with loader waves 4 and 5; value waves 2, 6 and
// 3, 7 pair up on SIMDs 2 and 3 (36 and 32 MFMAs per SIMD per slot).  Every wave fits in
// 256 registers; the score waves prefetch 4 operand reads (the second wave on the SIMD
// covers what a deeper prefetch would).
__global__ __launch_bounds__(512, 1) void decode_absorbed_mfma_r64_kernel(
    const bf16_t* __restrict__ q_abs, const bf16_t* __restrict__ pool,
    const int32_t* __restrict__ pt, const int32_t* __restrict__ lens,
    float* __restrict__ o_part, float* __restrict__ lse_part, int s_q, int H, int max_pages,
    int S, int split_tokens, float zscale, float slack, int n_units, int n_yblk,
    int xcd_ranges, int num_pages, unsigned int* bad) {
  constexpr int NQ = 2;
  __shared__ __attribute__((aligned(16))) ring::Smem sm;
  MLA_SETUP_WORK(NQ)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  switch (wave) {
    case 0: ring::score_wave<NQ, 0, 4>(sm, w, lane); break;
    case 1: ring::score_wave<NQ, 1, 4>(sm, w, lane); break;
    case 2: ring::value_wave128<0>(sm, w, lane); break;
    case 3: ring::value_wave128<1>(sm, w, lane); break;
    case 4: ring::loader_wave<0>(sm, w, lane); break;
    case 5: ring::loader_wave<1>(sm, w, lane); break;
    case 6: ring::value_wave128<2>(sm, w, lane); break;
    default: ring::value_wave128<3>(sm, w, lane); break;
  }
}

#undef MLA_SETUP_WORK

}  // namespace

bool decode_absorbed_mfma_supported(const mla_shape_t& s) {
  return s.dtype == MLA_BF16 && s.d_c == kDC && s.d_rope == kD - kDC &&
         s.page_size == kPage && (s.s_q * s.n_heads) % 32 == 0;
}

hipError_t launch_decode_absorbed_mfma(const mla_shape_t& s, const void* q_abs,
                                       const void* pool, const int32_t* pt,
                                       const int32_t* lens, float* o_part, float* lse_part,
                                       unsigned int* bad, hipStream_t st) {
  const int rows = s.s_q * s.n_heads;
  const int nq = (rows % 64 == 0) ? 2 : 1;
  const int n_yblk = rows / (32 * nq);
  const int n_units = s.batch * s.n_splits;
  const unsigned grid = static_cast<unsigned>((n_units + 7) / 8) * 8u * n_yblk;
  constexpr unsigned kResident = 256;   // workgroups resident at once: one per CU
  const int xcd_ranges = grid <= kResident ? 1 : 0;
  const float zscale = s.softmax_scale * kLog2e;
  // Slack (log2 units) before a row's reference maximum moves; the default keeps P below
  // 2^32.  MLA_DECODE_REF_SLACK (0..64) overrides it, e.g. 0 to exercise the rescale path.
  float slack = 32.f;
  if (const char* e = getenv("MLA_DECODE_REF_SLACK")) {
    const float v = strtof(e, nullptr);
    if (v >= 0.f && v <= 64.f) slack = v;
  }
  if (nq == 2)
    hipLaunchKernelGGL(decode_absorbed_mfma_r64_kernel, dim3(grid), dim3(512), 0, st,
                       static_cast<const bf16_t*>(q_abs), static_cast<const bf16_t*>(pool), pt,
                       lens, o_part, lse_part, s.s_q, s.n_heads, s.max_pages, s.n_splits,
                       s.split_tokens, zscale, slack, n_units, n_yblk, xcd_ranges,
                       s.num_pages, bad);
  else
    hipLaunchKernelGGL(decode_absorbed_mfma_r32_kernel, dim3(grid), dim3(192), 0, st,
                       static_cast<const bf16_t*>(q_abs), static_cast<const bf16_t*>(pool), pt,
                       lens, o_part, lse_part, s.s_q, s.n_heads, s.max_pages, s.n_splits,
                       s.split_tokens, zscale, slack, n_units, n_yblk, xcd_ranges,
                       s.num_pages, bad);
  return hipGetLastError();
}

}  // namespace mla

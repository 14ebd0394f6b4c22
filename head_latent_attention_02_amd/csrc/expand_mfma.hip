// Matrix-core GQA-path cache expansion (a6) for bf16 caches with d_c = 512 and
// d_nope = d_v = 128: for every cached row [c ; k^R] and group j,
//   k[p, r, j, :] = W_UK[j] c,   v[p, r, j, :] = W_UV[j] c,   kr[p, r, :] = k^R,
// accumulated in fp32 and rounded once to bf16 (AI Radio episode on GQLA, "The paper's
// summary": per-group K and V plus the shared RoPE key, from the same weights the
// absorbed path uses).
//
// One workgroup (4 waves, one per SIMD) per (group j, range of pages).  The group's 256
// weight rows (W_UK[j] then W_UV[j], 512 wide) stay in registers for the whole range as the
// A operand of v_mfma_f32_32x32x16_bf16 (64 rows per wave); pages stream through LDS in
// halves of 32 tokens (Y^T[out][token] = W[out][:] . X^T[:][token], so both operands are read
// along the latent, the layout they have in memory), each loaded one half ahead into
// registers.  Outputs are staged through LDS and written as whole 256-byte K and V rows
// at the start of the next half, before its loads; one barrier per half page.  The G groups of a page range run on the same XCD
// (workgroups 8 apart), so each page is fetched from HBM once and shared through its L2.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLat = 512;          // latent width
constexpr int kOut = 128;          // d_nope = d_v
constexpr int kHalf = 32;          // tokens per half page
constexpr int kXRowB = kLat * 2;   // latent bytes of one token in the staged tile
constexpr int kYStride = 264;      // bf16 per staged output row (256 + 8: 16-byte aligned rows)

constexpr int kBPF = 6;           // operand reads in flight ahead of their MFMAs

struct ExpSmem {
  char x[2][kHalf * kXRowB];       // two half pages of latent rows (64 KB)
  bf16_t y[2][kHalf * kYStride];   // two half pages of outputs [token][k 0..127 | v 0..127]
};

// The 16-byte chunk ch of staged token t sits at chunk ch ^ (t & 15) of its row: the
// operand reads take one chunk from each of 16 consecutive tokens (conflict-free), the
// staging stores write whole rows.
__device__ __forceinline__ int xswz(int t, int ch) { return ch ^ (t & 15); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

__global__ __launch_bounds__(256, 1) void expand_mfma_kernel(
    const bf16_t* __restrict__ pool, const bf16_t* __restrict__ w_uk,
    const bf16_t* __restrict__ w_uv, bf16_t* __restrict__ kout, bf16_t* __restrict__ vout,
    bf16_t* __restrict__ krout, int num_pages, int G, int d_r, int n_ranges,
    int pages_per_range) {
  __shared__ __attribute__((aligned(16))) ExpSmem sm;
  // workgroup -> (range r, group j): the G groups of one range are 8 workgroups apart
  const int wg = blockIdx.x;
  const int i8 = wg >> 3;
  const int j = i8 % G;
  const int r = (i8 / G) * 8 + (wg & 7);
  if (r >= n_ranges) return;
  const int p0 = r * pages_per_range;
  const int p1 = min(p0 + pages_per_range, num_pages);
  if (p0 >= p1) return;
  const int D = kLat + d_r;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n32 = lane & 31, g = lane >> 5;

  // weight rows 64 wave + 32 ob + n32 of the group's 256 (W_UK rows, then W_UV rows)
  bf16x8 wreg[2][kLat / 16];
#pragma unroll
  for (int ob = 0; ob < 2; ++ob) {
    const int o = 64 * wave + 32 * ob + n32;
    const bf16_t* row = (o < kOut) ? w_uk + (static_cast<size_t>(j) * kOut + o) * kLat
                                   : w_uv + (static_cast<size_t>(j) * kOut + o - kOut) * kLat;
#pragma unroll
    for (int ks = 0; ks < kLat / 16; ++ks)
      wreg[ob][ks] = *reinterpret_cast<const bf16x8*>(row + 16 * ks + 8 * g);
  }
  // Wait for the weight rows here, once (s_waitcnt vmcnt(0)).  Without it the compiler's
  // wait analysis, merging the loop's first entry (weights still in flight) with its back
  // edge, keeps a descending series of vmcnt waits on them inside the MFMA loop, and in
  // every later half those waits force the next half's loads to land mid-loop, so loads
  // and MFMAs ran one after the other.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // each wave stages tokens 8 wave .. 8 wave + 7 of a half page, one 1-KB latent row per
  // load, and their RoPE keys in one more load (lane l: token l / 8, 16-byte chunk l % 8;
  // lanes past the key's width re-read its last chunk, and with no key the row's first).
  // One register buffer: the loads of half h + 1 are in flight while half h runs (a second
  // buffer would leave no registers for the operand prefetch).  The key load is
  // unconditional, so the compiler counts the loads in flight exactly; group 0 alone stores
  // the keys.
  u32x4 stg[9];
  const int n_half = 2 * (p1 - p0);
  const int per = d_r / 8;
  const int kr_tok = lane >> 3;
  const int kr_ch = min(lane & 7, max(per - 1, 0));
  const int kr_ofs = per > 0 ? kLat + 8 * kr_ch : 0;
  const bool kr_lane = j == 0 && (lane & 7) < per;
  auto load_half = [&](int h) {
    if (h >= n_half) return;
    const size_t tok0 = static_cast<size_t>(p0 + (h >> 1)) * 64 + 32 * (h & 1) + 8 * wave;
    // ordinary (cached) loads: the G workgroups of this range read the same rows, and the
    // second to seventh reads must find them in L2 (non-temporal loads measured 5.6 ms at
    // the GQLA shape, every group refetching from HBM)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      stg[i] = *(reinterpret_cast<const u32x4*>(pool + (tok0 + i) * D) + lane);
    stg[8] = *reinterpret_cast<const u32x4*>(pool + (tok0 + kr_tok) * D + kr_ofs);
  };
  // the outputs of half h - 1 (staged in y[(h - 1) & 1]) leave in four steps at the start
  // of half h: 64 rows of 256 bytes (token t: its K row, then its V row), 16 lanes per row,
  // one 16-byte store per lane and step
  auto store_step = [&](int hprev, int it) {
    const size_t tok0 = static_cast<size_t>(p0 + (hprev >> 1)) * 64 + 32 * (hprev & 1);
    const int row = 16 * it + (threadIdx.x >> 4);
    const int t = row >> 1, kv = row & 1, col = 8 * (threadIdx.x & 15);
    const u32x4 val = *reinterpret_cast<const u32x4*>(sm.y[hprev & 1] + t * kYStride +
                                                      kOut * kv + col);
    bf16_t* dst = (kv ? vout : kout) + ((tok0 + t) * G + j) * kOut + col;
    __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(dst));
  };
  load_half(0);
  // one half page; P = h & 1 as a constant, so both register buffers keep fixed registers.
  // Returns true after the last half's outputs have left (h == n_half).
  auto half = [&](auto par, int h) -> bool {
    constexpr int P = decltype(par)::value;
    if (h < n_half) {
      char* xb = sm.x[P];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = 8 * wave + i;
        *reinterpret_cast<u32x4*>(xb + t * kXRowB + 16 * xswz(t, lane)) = stg[i];
      }
      if (kr_lane) {   // the shared RoPE key, copied once per token (group 0)
        const size_t tok = static_cast<size_t>(p0 + (h >> 1)) * 64 + 32 * P + 8 * wave + kr_tok;
        __builtin_nontemporal_store(stg[8],
                                    reinterpret_cast<u32x4*>(krout + tok * d_r + 8 * kr_ch));
      }
    }
    // half h is staged; the outputs of half h - 1 are staged, and nobody still reads the
    // buffers that this half overwrites (x of half h - 2 was read before the previous
    // barrier, and y of half h - 2 was written out there too)
    __syncthreads();
    if (h == n_half) {   // the last half's outputs
#pragma unroll
      for (int it = 0; it < 4; ++it) store_step(h - 1, it);
      return true;
    }
    // the outputs of half h - 1 leave before the loads of half h + 1 are issued: the memory
    // counter retires in issue order, so the staging of half h + 1 (which waits for its
    // loads) then never waits for these stores, which have the whole MFMA loop to complete
    if (h > 0) {
#pragma unroll
      for (int it = 0; it < 4; ++it) store_step(h - 1, it);
    }
    load_half(h + 1);
    f32x16 acc[2] = {};
    const char* bt = sm.x[P] + n32 * kXRowB;
    auto read_b = [&](int ks) {
      return *reinterpret_cast<const bf16x8*>(bt + 16 * xswz(n32, 2 * ks + g));
    };
    bf16x8 bbuf[kBPF];
#pragma unroll
    for (int ks = 0; ks < kBPF; ++ks) bbuf[ks] = read_b(ks);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kLat / 16; ++ks) {
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wreg[0][ks], bbuf[ks % kBPF], acc[0],
                                                       0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wreg[1][ks], bbuf[ks % kBPF], acc[1],
                                                       0, 0, 0);
      if (ks + kBPF < kLat / 16) bbuf[ks % kBPF] = read_b(ks + kBPF);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane (n32, g) holds token n32, outputs 32 ob + 8 q + 4 g + 0..3 of the wave's 64
    bf16_t* yrow = sm.y[P] + n32 * kYStride + 64 * wave + 4 * g;
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<uint2*>(yrow + 32 * ob + 8 * q) =
            make_uint2(pack_bf16x2(acc[ob][4 * q], acc[ob][4 * q + 1]),
                       pack_bf16x2(acc[ob][4 * q + 2], acc[ob][4 * q + 3]));
    return false;
  };
  for (int h = 0;; h += 2) {
    if (half(std::integral_constant<int, 0>(), h)) break;
    if (half(std::integral_constant<int, 1>(), h + 1)) break;
  }
}

}  // namespace

bool expand_cache_mfma_supported(const mla_shape_t& s) {
  return s.dtype == MLA_BF16 && s.d_c == kLat && s.d_nope == kOut && s.d_v == kOut &&
         s.page_size == 64 && s.d_rope <= 64;
}

hipError_t launch_expand_cache_mfma(const mla_shape_t& s, const void* pool, const void* w_uk,
                                    const void* w_uv, void* k, void* v, void* kr,
                                    hipStream_t st) {
  const int G = s.n_wheads;
  // page ranges: a multiple of 8 (one per XCD slot), about 256 workgroups in all
  const int n_ranges = max(8, (256 / G) / 8 * 8);
  const int per = (s.num_pages + n_ranges - 1) / n_ranges;
  hipLaunchKernelGGL(expand_mfma_kernel, dim3(n_ranges * G), dim3(256), 0, st,
                     static_cast<const bf16_t*>(pool), static_cast<const bf16_t*>(w_uk),
                     static_cast<const bf16_t*>(w_uv), static_cast<bf16_t*>(k),
                     static_cast<bf16_t*>(v), static_cast<bf16_t*>(kr), s.num_pages, G,
                     s.d_rope, n_ranges, per);
  return hipGetLastError();
}

}  // namespace mla

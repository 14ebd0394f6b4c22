// Matrix-core GQA-path cache expansion (a6) for bf16 caches with d_c = 512 and
// d_nope = d_v = 128: for every cached row [c ; k^R] and group j,
//   k[p, r, j, :] = W_UK[j] c,   v[p, r, j, :] = W_UV[j] c,   kr[p, r, :] = k^R,
// accumulated in fp32 and rounded once to bf16 (AI Radio episode on GQLA, "The paper's
// summary": per-group K and V plus the shared RoPE key, from the same weights the
// absorbed path uses).
//
// One workgroup (8 waves, two per SIMD) per (group j, range of pages).  The group's 256
// weight rows (W_UK[j] then W_UV[j], 512 wide) stay in registers for the whole range as the
// A operand of v_mfma_f32_32x32x16_bf16 (32 rows per wave); pages stream through LDS in
// halves of 32 tokens (Y^T[out][token] = W[out][:] . X^T[:][token], so both operands are read
// along the latent, the layout they have in memory).  The latent rows go from global memory
// straight into LDS (global_load_lds_dwordx4: no staging registers), two halves ahead,
// through a ring of three half buffers; each wave waits for its own loads of the next half
// with an explicit vmcnt before the half's barrier, which is a bare s_barrier: the
// workgroup fence of __syncthreads would also wait for the loads issued after them.
// Outputs are staged through LDS and written as whole 256-byte K and V rows at the start
// of the next half, before its loads.  The G groups of a page range run on the same XCD
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

constexpr int kKrRowB = 128;       // RoPE-key bytes of one staged token (d_rope <= 64)
constexpr int kXBuf = 3;           // half buffers in the latent ring
constexpr int kBPF = 4;            // operand reads in flight ahead of their MFMAs

struct ExpSmem {
  char x[kXBuf][kHalf * kXRowB];   // latent rows of three half pages (96 KB)
  char kr[kXBuf][kHalf * kKrRowB]; // their RoPE keys (12 KB)
  bf16_t y[2][kHalf * kYStride];   // two half pages of outputs [token][k 0..127 | v 0..127]
};

// One wave-wide load straight into LDS: lane l's 16 bytes at src land at LDS byte address
// lds + 16 l (lds is wave-uniform, in m0).  Written as inline asm so that the compiler does
// not track these LDS writes: it cannot tell the ring slots apart and would wait for every
// load in flight before any LDS access.  The kernel waits for them itself (explicit vmcnt
// before the barrier that publishes a half).  The instruction has no register results.
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) void*)(p)));
}

// s_waitcnt: vector-memory count n (0..63), lgkmcnt(0), expcnt left alone
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70);
}

// Ring layout: the 16-byte chunk ch of staged token t sits at chunk ch ^ (t & 15) of its
// row, so the operand reads, one chunk from each of 16 consecutive tokens, are
// conflict-free, and each load instruction still writes one whole row.

// two floats to a pair of bf16, rounded to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// With two waves per SIMD, a wave whose vector-memory instructions (4 latent rows and one
// RoPE-key block loaded per half, 2 output stores) stall leaves the matrix core to the other
// wave on its SIMD; the price is that every B operand read from LDS feeds one MFMA (32 rows)
// instead of two (4.35 against 4.48-4.51 ms for one wave per SIMD with 64 rows each, at
// 32 x 65536 tokens).  Waves 4-7 load the same RoPE-key blocks as waves 0-3 (the same bytes
// to the same LDS addresses), so that every wave issues the same number of loads.
__global__ __launch_bounds__(512, 1) void expand_mfma_kernel(
    const bf16_t* __restrict__ pool, const bf16_t* __restrict__ w_uk,
    const bf16_t* __restrict__ w_uv, bf16_t* __restrict__ kout, bf16_t* __restrict__ vout,
    bf16_t* __restrict__ krout, int num_pages, int G, int d_r, int n_ranges,
    int pages_per_range) {
  __shared__ __attribute__((aligned(16))) ExpSmem sm;
  const int wg = blockIdx.x;
  const int i8 = wg >> 3;
  const int j = i8 % G;
  const int r = (i8 / G) * 8 + (wg & 7);
  if (r >= n_ranges) return;
  const int p0 = r * pages_per_range;
  const int p1 = min(p0 + pages_per_range, num_pages);
  if (p0 >= p1) return;
  const int D = kLat + d_r;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n32 = lane & 31, g = lane >> 5;

  // weight rows 32 wave + n32 of the group's 256 (W_UK rows, then W_UV rows)
  bf16x8 wreg[kLat / 16];
  {
    const int o = 32 * wave + n32;
    const bf16_t* row = (o < kOut) ? w_uk + (static_cast<size_t>(j) * kOut + o) * kLat
                                   : w_uv + (static_cast<size_t>(j) * kOut + o - kOut) * kLat;
#pragma unroll
    for (int ks = 0; ks < kLat / 16; ++ks)
      wreg[ks] = *reinterpret_cast<const bf16x8*>(row + 16 * ks + 8 * g);
  }
  // Wait for the weight rows here, once (s_waitcnt vmcnt(0)).  Without it the compiler's
  // wait analysis, merging the loop's first entry (weights still in flight) with its back
  // edge, keeps a descending series of vmcnt waits on them inside the MFMA loop, and in
  // every later half those waits force the next half's loads to land mid-loop.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // each wave loads the latent rows of tokens 4 wave .. 4 wave + 3 of a half page (one 1-KB
  // row per instruction, lane l bringing 16-byte chunk l ^ (t & 15) of token t) and the RoPE
  // keys of tokens 8 (wave % 4) .. +7 (lane l: token l / 8, chunk l % 8)
  const int n_half = 2 * (p1 - p0);
  const int per = d_r / 8;
  const int kb = wave & 3;
  const int kr_tok = 8 * kb + (lane >> 3);
  const int kr_ch = min(lane & 7, max(per - 1, 0));
  const int kr_ofs = per > 0 ? kLat + 8 * kr_ch : 0;
  const bool kr_lane = j == 0 && wave < 4 && (lane & 7) < per;
  auto half_tok0 = [&](int h) { return static_cast<size_t>(p0 + (h >> 1)) * 64 + 32 * (h & 1); };
  // load i (0..4) of half h into ring slot h % 3
  // the per-lane parts of the addresses are formed at each use from an opaque copy of the
  // lane index: kept live across the loop they would not leave the registers the weights need
  auto load_one = [&](int h, int i) {
    const int b = h % kXBuf;
    const char* rows = reinterpret_cast<const char*>(pool + half_tok0(h) * D);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (i < 4) {
      const int t = 4 * wave + i;
      load_lds16(rows + (t * 2 * D + 16 * (ln ^ (t & 15))), lds_addr(&sm.x[b][0]) + t * kXRowB);
    } else {
      const int kt = 8 * kb + (ln >> 3);
      const int kc = min(ln & 7, max(per - 1, 0));
      const int ko = per > 0 ? kLat + 8 * kc : 0;
      load_lds16(rows + 2 * (kt * D + ko), lds_addr(&sm.kr[b][0]) + 8 * kb * kKrRowB);
    }
  };
  // outputs of half hprev leave in two steps: 32 rows of 256 bytes per step (token t: its K
  // row, then its V row), 16 lanes per row, one 16-byte store per lane and step
  const size_t ostep = static_cast<size_t>(16) * G * kOut;
  auto read_outputs = [&](const bf16_t* ys, u32x4 (&val)[2]) {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const bf16_t* src = ys + (t >> 5) * kYStride + kOut * ((t >> 4) & 1) + 8 * (t & 15);
#pragma unroll
    for (int it = 0; it < 2; ++it)
      val[it] = *reinterpret_cast<const u32x4*>(src + 16 * it * kYStride);
  };
  auto output_dst = [&](int hprev) {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const size_t tok = half_tok0(hprev) + (t >> 5);
    return (((t >> 4) & 1) ? vout : kout) + (tok * G + j) * kOut + 8 * (t & 15);
  };
  // the end of half h: this wave's loads of half h + 1 have landed (issued after them: the 2
  // output stores of half h - 1 when h > 0, group 0's key store, the 5 loads of half h + 2
  // when there is one; the key store is left out of the count, which only makes the wait
  // cover it too), its output staging too; then the barrier.  The kernel uses no scratch.
  auto end_half = [&](int h) {
    if (h + 1 >= n_half)
      wait_vm_lgkm0<63>();
    else if (h + 2 < n_half)
      h > 0 ? wait_vm_lgkm0<7>() : wait_vm_lgkm0<5>();
    else
      h > 0 ? wait_vm_lgkm0<2>() : wait_vm_lgkm0<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
#pragma unroll
  for (int i = 0; i < 5; ++i) load_one(0, i);
#pragma unroll
  for (int i = 0; i < 5; ++i) load_one(1, i);
  wait_vm_lgkm0<5>();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // The vector-memory work of half h: the outputs of half h - 1 (staged in LDS before the
  // last barrier), group 0's RoPE keys of half h, the loads of half h + 2 into the ring slot
  // that half h - 1 used.  Waves 0-3 issue it when the half starts; waves 4-7, which share
  // SIMDs with them, half-way through their MFMA loop, so that on each SIMD one wave's memory
  // issue overlaps the other's matrix work (issued together, every wave's issue stalled on
  // the CU's vector-memory path while the matrix cores idled).  Either way it is issued
  // before the half's end, so end_half's counts hold for both.
  const bool late = wave >= 4;
  auto issue = [&](auto par, int h) {
    constexpr int P = decltype(par)::value;
    const int b = h % kXBuf;
    if (h > 0) {
      u32x4 oval[2];
      read_outputs(sm.y[1 - P], oval);
      bf16_t* odst = output_dst(h - 1);
#pragma unroll
      for (int it = 0; it < 2; ++it)
        __builtin_nontemporal_store(oval[it], reinterpret_cast<u32x4*>(odst + it * ostep));
    }
    if (kr_lane) {
      const u32x4 key = *reinterpret_cast<const u32x4*>(&sm.kr[b][0] + 8 * kb * kKrRowB +
                                                        16 * lane);
      __builtin_nontemporal_store(
          key, reinterpret_cast<u32x4*>(krout + (half_tok0(h) + kr_tok) * d_r + 8 * kr_ch));
    }
    if (h + 2 < n_half) {
#pragma unroll
      for (int i = 0; i < 5; ++i) load_one(h + 2, i);
    }
  };
  auto half = [&](auto par, int h) {
    constexpr int P = decltype(par)::value;
    const int b = h % kXBuf;
    if (!late) issue(par, h);
    f32x16 acc = {};
    // chunk 2 ks + g of token n32 sits at (2 ks + g) ^ (n32 & 15): 8 per-lane offsets for
    // ks % 8, the rest (256 bytes per 8 K-steps) an immediate
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int tn = ln & 31, tg = ln >> 5;
    const char* bt = &sm.x[b][0] + tn * kXRowB;
    int bo[8];
#pragma unroll
    for (int k8 = 0; k8 < 8; ++k8) bo[k8] = 16 * ((2 * k8 + tg) ^ (tn & 15));
    auto read_b = [&](int ks) {
      return *reinterpret_cast<const bf16x8*>(bt + bo[ks & 7] + 256 * (ks >> 3));
    };
    bf16x8 bbuf[kBPF];
#pragma unroll
    for (int ks = 0; ks < kBPF; ++ks) bbuf[ks] = read_b(ks);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kLat / 16; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wreg[ks], bbuf[ks % kBPF], acc, 0, 0, 0);
      if (ks + kBPF < kLat / 16) bbuf[ks % kBPF] = read_b(ks + kBPF);
      __builtin_amdgcn_sched_barrier(0);
      if (ks == kLat / 32 - 1) {
        if (late) issue(par, h);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // lane (n32, g) holds token n32, outputs 8 q + 4 g + 0..3 of the wave's 32
    bf16_t* yrow = sm.y[P] + n32 * kYStride + 32 * wave + 4 * g;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint2*>(yrow + 8 * q) =
          make_uint2(pack_bf16x2(acc[4 * q], acc[4 * q + 1]),
                     pack_bf16x2(acc[4 * q + 2], acc[4 * q + 3]));
    end_half(h);
  };
  for (int h = 0;; h += 2) {   // n_half is even
    half(std::integral_constant<int, 0>(), h);
    half(std::integral_constant<int, 1>(), h + 1);
    if (h + 2 >= n_half) break;
  }
  {
    u32x4 oval[2];
    read_outputs(sm.y[(n_half - 1) & 1], oval);
    bf16_t* odst = output_dst(n_half - 1);
#pragma unroll
    for (int it = 0; it < 2; ++it)
      __builtin_nontemporal_store(oval[it], reinterpret_cast<u32x4*>(odst + it * ostep));
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
  hipLaunchKernelGGL(expand_mfma_kernel, dim3(n_ranges * G), dim3(512), 0, st,
                     static_cast<const bf16_t*>(pool), static_cast<const bf16_t*>(w_uk),
                     static_cast<const bf16_t*>(w_uv), static_cast<bf16_t*>(k),
                     static_cast<bf16_t*>(v), static_cast<bf16_t*>(kr), s.num_pages, G,
                     s.d_rope, n_ranges, per);
  return hipGetLastError();
}

}  // namespace mla

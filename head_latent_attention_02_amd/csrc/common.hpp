// Shared device helpers for libmla (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

typedef uint16_t bf16_t;  // bf16 storage: the upper half of an IEEE binary32

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Checked builds (compiled with MLA_CHECKED) bounds-check every device-resident page-table
// entry before it is used as an address: an entry outside [0, num_pages) is replaced by page
// 0, so nothing outside the pool is read, and sets the library's bad-page flag (*bad = 1),
// which mla_checked_bad_pages reports.  Unchecked builds compile the check out.
#ifdef MLA_CHECKED
constexpr bool kChecked = true;
#else
constexpr bool kChecked = false;
#endif
__device__ __forceinline__ int checked_page(int page, int num_pages, unsigned int* bad) {
  if constexpr (kChecked) {
    if (page < 0 || page >= num_pages) {
      if (bad) *bad = 1u;
      return 0;
    }
  }
  return page;
}

// Checked builds also bound each device-resident context length T_b to [0, max_tokens]
// (max_tokens = max_pages * page_size, the tokens one page-table row can map) before it
// becomes a page-table index, and raise the same flag when they have to clamp it, so a
// length past the table row never reads beyond that row.  Unchecked builds use T_b as is.
__device__ __forceinline__ int checked_len(int T, int max_tokens, unsigned int* bad) {
  if constexpr (kChecked) {
    if (T < 0 || T > max_tokens) {
      if (bad) *bad = 1u;
      return T < 0 ? 0 : max_tokens;
    }
  }
  return T;
}

__device__ __forceinline__ float ldf(const float* p) { return *p; }
__device__ __forceinline__ float ldf(const bf16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 with round-to-nearest-even; NaN maps to the canonical quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}
__device__ __forceinline__ void stf(float* p, float v) { *p = v; }
__device__ __forceinline__ void stf(bf16_t* p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Token range [lo, hi) of split u (page-aligned even chunks, or fixed chunks).
__device__ __forceinline__ void split_range(int T, int u, int S, int P, int split_tokens,
                                            int& lo, int& hi) {
  long L;
  if (split_tokens > 0) {
    L = split_tokens;
  } else {
    long per = (static_cast<long>(T) + S - 1) / S;
    L = ((per + P - 1) / P) * P;
  }
  long a = static_cast<long>(u) * L;
  lo = static_cast<int>(a < T ? a : T);
  long e = a + L;
  hi = static_cast<int>(e < T ? e : T);
}

}  // namespace mla

// Calibration microbenchmarks for the roofline denominators (libmla_calib.so).
//
// calib_hbm_read: the read bandwidth this part reaches for a pure stream in the access
// pattern the decode kernels use (every workgroup streams its own contiguous span in
// 36 KB tiles of 1 KB per load instruction, non-temporal, four waves with four tiles in
// flight each), timed by the caller around the launch.
// calib_mfma_bf16: the dense bf16 matrix-core rate for v_mfma_f32_32x32x16_bf16 with four
// independent accumulators per wave and two waves per SIMD, 32768 FLOP per instruction.
// Neither touches the method's data or arithmetic; they only measure the machine.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileB = 36864;    // bytes per tile (36 x 1 KB)
constexpr int kWaves = 4;
constexpr int kLoads = 36 / kWaves;
constexpr int kDepth = 4;        // tiles in flight per wave
constexpr int kBufWord3 = 0x00020000;
constexpr int kNonTemporal = 2;

__global__ __launch_bounds__(256, 1) void hbm_read_kernel(const char* __restrict__ buf,
                                                          int tiles, unsigned* sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const char* base0 = buf + static_cast<size_t>(blockIdx.x) * tiles * kTileB;
  uint32_t off[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) off[j] = (wave + kWaves * j) * 1024 + lane * 16;
  u32x4 b[kDepth][kLoads];
  u32x4 acc = {0u, 0u, 0u, 0u};
  auto load = [&](int i, int t) {
    if (t >= tiles) return;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base0 + static_cast<size_t>(t) * kTileB), 0, kTileB, kBufWord3);
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      b[i][j] = __builtin_amdgcn_raw_buffer_load_b128(r, off[j], 0, kNonTemporal);
  };
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) load(i, i);
  for (int t = 0; t < tiles; t += kDepth) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      load((i + kDepth - 1) % kDepth, t + i + kDepth - 1);
      if (t + i < tiles) {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) acc ^= b[i][j] + static_cast<unsigned>(j);
      }
    }
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(256, 2) void mfma_bf16_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(static_cast<float>((lane + i) & 7) * 0.125f);
    b[i] = static_cast<__bf16>(static_cast<float>((lane * 3 + i) & 7) * 0.0625f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Bytes one call of calib_hbm_read streams: n_wg workgroups x tiles x 36864.
int64_t calib_hbm_read_bytes(int32_t n_wg, int32_t tiles) {
  return static_cast<int64_t>(n_wg) * tiles * kTileB;
}

// Streams calib_hbm_read_bytes(n_wg, tiles) bytes of `buf` (device, caller-owned) once;
// `sink` (device, n_wg * 256 uint32) receives a checksum so the loads are not elided.
// Returns 0, or the HIP error code of the launch.
int32_t calib_hbm_read(const void* buf, int32_t n_wg, int32_t tiles, unsigned* sink,
                       hipStream_t stream) {
  if (!buf || !sink || n_wg <= 0 || tiles <= 0) return -1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(n_wg), dim3(256), 0, stream,
                     static_cast<const char*>(buf), tiles, sink);
  return static_cast<int32_t>(hipGetLastError());
}

// FLOPs one call of calib_mfma_bf16 performs: n_wg x 4 waves x iters x 4 x 32768.
int64_t calib_mfma_bf16_flops(int32_t n_wg, int32_t iters) {
  return static_cast<int64_t>(n_wg) * 4 * iters * 4 * 32768;
}

// Runs the bf16 matrix-core loop; `sink` (device, n_wg * 256 floats) takes the sums.
int32_t calib_mfma_bf16(int32_t n_wg, int32_t iters, float* sink, hipStream_t stream) {
  if (!sink || n_wg <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(n_wg), dim3(256), 0, stream, iters, sink);
  return static_cast<int32_t>(hipGetLastError());
}

}  // extern "C"

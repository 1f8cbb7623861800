// Matrix-core rate microbenchmark for gfx950 (measurement only, not part of
// the vsmooth C ABI; built into libvsmooth_peak.so and used by bench.py
// --peaks).
//
// Each wave issues `iters` rounds of eight independent products on register
// operands -- FP8 v_mfma_scale_f32_32x32x64_f8f6f4 (unit E8M0 scales) or
// bf16 v_mfma_f32_32x32x16_bf16 -- so the matrix core never waits on memory
// or on a dependency, and records its s_memtime ticks (shader clock) around
// the loop.  Flops per product: 2 * 32 * 32 * 64 (FP8), 2 * 32 * 32 * 16
// (bf16).  The caller converts ticks and its own event time into the clock
// and the rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256, 2) void mfma_loop(int iters, long long* ticks, float* sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v16f acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
  // small E4M3 / bf16 operands that keep the sums finite
  v8i a8, b8;
  v8bf a16, b16;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a8[e] = 0x30303030 + ((lane + e) & 7);
    b8[e] = 0x28282828 + ((lane * 3 + e) & 7);
    a16[e] = static_cast<__bf16>(0.001f * (lane + e));
    b16[e] = static_cast<__bf16>(0.002f * (lane - e));
  }
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i], 0, 0, 0, 127, 0, 127);
      else
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16, b16, acc[i], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += acc[i][0];
  const long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    const int w = blockIdx.x * (blockDim.x >> 6) + wave;
    ticks[w] = t1 - t0;
    sink[w] = s;
  }
}

}  // namespace

// kind 0: FP8, 1: bf16.  ticks and sink hold one entry per wave
// (blocks * threads / 64); threads is a multiple of 64 up to 256.
// Returns 0, or 1 for bad arguments, 2 for a launch error.
extern "C" int vs_peak_mfma_loop(int kind, int blocks, int threads, int iters, long long* ticks,
                                 float* sink, void* stream) {
  if (kind < 0 || kind > 1 || blocks < 1 || threads < 64 || threads > 256 || threads % 64 ||
      iters < 1 || !ticks || !sink)
    return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(mfma_loop<0>, dim3(blocks), dim3(threads), 0, st, iters, ticks, sink);
  else
    hipLaunchKernelGGL(mfma_loop<1>, dim3(blocks), dim3(threads), 0, st, iters, ticks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

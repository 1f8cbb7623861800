// Matrix-core rate microbenchmark for gfx950 (measurement only, not part of
// the vsmooth C ABI; built into libvsmooth_peak.so and used by bench.py
// --peaks).
//
// Each wave issues `iters` rounds of eight independent products on register
// operands -- FP8 v_mfma_scale_f32_32x32x64_f8f6f4 (unit E8M0 scales) or
// bf16 v_mfma_f32_32x32x16_bf16 -- so the matrix core never waits on memory
// or on a dependency, and records its s_memtime ticks (shader clock) around
// the loop.  Each of the eight products has its own random A operand, so
// consecutive products see different bytes.  Flops per product: 2 * 32 *
// 32 * 64 (FP8), 2 * 32 * 32 * 16 (bf16).  The caller converts ticks and its
// own event time into the clock and the rate.  mix_loop (below) runs the
// attention kernel's two phase mixes for the clock each holds.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

// A 32-bit mix of x (an integer hash; operand bytes that change from one
// product to the next, as random FP8 codes do, draw more power than repeated
// patterns).
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// Four random E4M3 bytes of moderate size: random sign and mantissa, the
// exponent field in 4-7 (magnitudes 1/8 to 15/8), so the sums stay finite.
__device__ __forceinline__ uint32_t rand_e4m3x4(uint32_t x) {
  return (hash32(x) & 0x9F9F9F9Fu) | 0x20202020u;
}

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
  // a different random A per accumulator, so consecutive products see
  // different operand bytes
  v8i a8[8], b8;
  v8bf a16[8], b16;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    b8[e] = static_cast<int>(rand_e4m3x4(lane * 8 + e + 4096));
    b16[e] = static_cast<__bf16>(0.002f * (lane - e));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a8[i][e] = static_cast<int>(rand_e4m3x4((i * 64 + lane) * 8 + e));
      a16[i][e] = static_cast<__bf16>(static_cast<float>(static_cast<int>(hash32((i * 64 + lane) * 8 + e) & 255) - 128) * 1e-3f);
    }
  }
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0)
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[i], b8, acc[i], 0, 0, 0, 127, 0, 127);
      else
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a16[i], b16, acc[i], 0, 0, 0);
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

// Mixes of the attention kernel's two phases, for the clock each holds under
// sustained load (eight waves per CU, two per SIMD, as in the kernel).  Each
// wave records s_memtime (shader clock) and s_memrealtime (100 MHz) ticks
// around its loop, so its own clock is the ratio.
//   role 0: FP8 products (32x32x64, unit E8M0 scales) whose A operand is read
//           from a 16 KB LDS tile, 32 bytes per lane per product (2 KB per
//           wave), eight independent accumulators: the matrix-core phase's
//           operand traffic;
//   role 1: the vector phase's mix on 64 register values per lane: a chain
//           of 32 max3, 64 exp2, 32 E4M3 packs and 64 adds (the row sum),
//           without the growth branch (this file is built without NaN
//           handling, so the maxima need no quieting of their inputs);
//   role 2: the same products with register operands.
template <int ROLE>
__device__ __forceinline__ void mix_role(int iters, int lane, const uint4* lds, long long& tk,
                                         long long& rt, float& out) {
  if constexpr (ROLE == 0 || ROLE == 2) {
    v16f acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    v8i b8, a8r[ROLE == 2 ? 8 : 1];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b8[e] = static_cast<int>(rand_e4m3x4(lane * 8 + e + 4096));
#pragma unroll
      for (int i = 0; i < (ROLE == 2 ? 8 : 1); ++i)
        a8r[i][e] = static_cast<int>(rand_e4m3x4((i * 64 + lane) * 8 + e));
    }
    const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v8i a8 = a8r[ROLE == 2 ? i : 0];
        if constexpr (ROLE == 0) {
          // 1 KB of consecutive 16-byte chunks per read: no bank conflicts;
          // the offset moves every turn so the reads stay in the loop
          const int c = ((it * 8 + i) * 136 + lane) & 1023;
          const uint4 x = lds[c], y = lds[c ^ 512];
          a8 = v8i{static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z),
                   static_cast<int>(x.w), static_cast<int>(y.x), static_cast<int>(y.y),
                   static_cast<int>(y.z), static_cast<int>(y.w)};
        }
        acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[i], 0, 0, 0, 127, 0, 127);
      }
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += acc[i][0];
    tk = __builtin_amdgcn_s_memtime() - t0;
    rt = __builtin_amdgcn_s_memrealtime() - r0;
    out = sum;
  } else {
    float x[64];
#pragma unroll
    for (int r = 0; r < 64; ++r) x[r] = -0.05f * ((r + lane) & 31) - 1.0f;   // all < 8
    uint32_t xo = 0;
    float ls = 0.0f;
    const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
      // new scores every turn, as the products deliver them (no instruction)
#pragma unroll
      for (int r = 0; r < 64; ++r) asm volatile("" : "+v"(x[r]));
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 64; ++r) mx = __builtin_fmaxf(mx, x[r]);
      ls += mx;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float e0 = __builtin_amdgcn_exp2f(x[4 * q]), e1 = __builtin_amdgcn_exp2f(x[4 * q + 1]);
        const float e2 = __builtin_amdgcn_exp2f(x[4 * q + 2]), e3 = __builtin_amdgcn_exp2f(x[4 * q + 3]);
        ls += (e0 + e1) + (e2 + e3);
        uint32_t pk = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false));
        pk = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, static_cast<int>(pk), true));
        xo ^= pk;
      }
    }
    tk = __builtin_amdgcn_s_memtime() - t0;
    rt = __builtin_amdgcn_s_memrealtime() - r0;
    out = ls + static_cast<float>(xo & 1u);
  }
}

// kind 0: every wave role 0; 1: every wave role 1; 2: waves 0-3 role 0 and
// waves 4-7 role 1 (each SIMD runs one of each, as the ping-pong does);
// 3: every wave role 2.  One workgroup of 512 threads per CU.
template <int KIND>
__global__ __launch_bounds__(512, 1) void mix_loop(int iters_p, int iters_v, long long* ticks,
                                                   long long* rticks, float* sink) {
  __shared__ uint4 lds[1024];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < 1024; i += 512)
    lds[i] = uint4{rand_e4m3x4(4 * i), rand_e4m3x4(4 * i + 1), rand_e4m3x4(4 * i + 2),
                   rand_e4m3x4(4 * i + 3)};
  __syncthreads();
  long long tk = 0, rt = 0;
  float out = 0.0f;
  if (KIND == 0 || (KIND == 2 && wave < 4)) mix_role<0>(iters_p, lane, lds, tk, rt, out);
  else if (KIND == 3) mix_role<2>(iters_p, lane, lds, tk, rt, out);
  else mix_role<1>(iters_v, lane, lds, tk, rt, out);
  if (lane == 0) {
    const int w = blockIdx.x * 8 + wave;
    ticks[w] = tk;
    rticks[w] = rt;
    sink[w] = out;
  }
}

}  // namespace

// Phase mixes (see mix_loop): kind 0-3, `blocks` workgroups of 512 threads,
// product loops of iters_p turns (8 products each), vector loops of iters_v
// turns (one tile's mix each).  ticks, rticks and sink hold blocks * 8
// entries.  Returns 0, or 1 for bad arguments, 2 for a launch error.
extern "C" int vs_peak_mix_loop(int kind, int blocks, int iters_p, int iters_v, long long* ticks,
                                long long* rticks, float* sink, void* stream) {
  if (kind < 0 || kind > 3 || blocks < 1 || iters_p < 1 || iters_v < 1 || !ticks || !rticks || !sink)
    return 1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(blocks), block(512);
  if (kind == 0) hipLaunchKernelGGL(mix_loop<0>, grid, block, 0, st, iters_p, iters_v, ticks, rticks, sink);
  else if (kind == 1) hipLaunchKernelGGL(mix_loop<1>, grid, block, 0, st, iters_p, iters_v, ticks, rticks, sink);
  else if (kind == 2) hipLaunchKernelGGL(mix_loop<2>, grid, block, 0, st, iters_p, iters_v, ticks, rticks, sink);
  else hipLaunchKernelGGL(mix_loop<3>, grid, block, 0, st, iters_p, iters_v, ticks, rticks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

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

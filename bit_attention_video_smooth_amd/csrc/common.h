// Internal helpers shared by the libvsmooth HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "vsmooth.h"

namespace vs {

constexpr int kBlock = 128;            // tokens per quantization block / KV tile

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef double v2d __attribute__((ext_vector_type(2)));

inline int n_blocks(int S) { return (S + kBlock - 1) / kBlock; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Status of the most recent launch on this thread.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? VS_OK : VS_ERR_HIP;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Element offset of (b, s, h, d=0) in a [B,S,H,D] or [B,H,S,D] tensor.
__device__ __forceinline__ size_t token_offset(int layout, int b, int s, int h,
                                               int S, int H, int D) {
  return layout == VS_LAYOUT_BSHD
             ? ((static_cast<size_t>(b) * S + s) * H + h) * D
             : ((static_cast<size_t>(b) * H + h) * S + s) * D;
}

// Two float32 values -> two E4M3 bytes written into byte lanes [2*hi, 2*hi+1]
// of `old` (hardware conversion: round to nearest even; inputs must already
// lie in [-448, 448]).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, static_cast<int>(old), HI));
}

// Two float32 values -> two bf16 (round to nearest even) packed low, high.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
  const v2bf16 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  uint32_t r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}

// float32 -> nearest bf16 (ties to the even mantissa), returned as float32
// (finite inputs).
__device__ __forceinline__ float round_bf16(float y) {
  const uint32_t b = __float_as_uint(y);
  return __uint_as_float((b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u);
}

// Rotary embedding of 8 consecutive channels (4 interleaved pairs) of one
// token, with the 4 pairs' cosines and sines: y0 = f32(f32(a cos) - f32(b sin)),
// y1 = f32(f32(a sin) + f32(b cos)), each rounded to bf16 (what a model's own
// rotation of its bf16 activations gives).  No contraction to FMA: every
// product and sum is rounded on its own, in this order.
__device__ __forceinline__ void rope8(float (&x)[8], const float4& cs, const float4& sn) {
#pragma clang fp contract(off)
  const float c[4] = {cs.x, cs.y, cs.z, cs.w}, s[4] = {sn.x, sn.y, sn.z, sn.w};
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float a = x[2 * p], b = x[2 * p + 1];
    const float ac = a * c[p], bs = b * s[p], as = a * s[p], bc = b * c[p];
    x[2 * p] = round_bf16(ac - bs);
    x[2 * p + 1] = round_bf16(as + bc);
  }
}

__device__ __forceinline__ float clamp448(float x) {
  return __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
}

// Wave-wide (64 lanes) reductions through DPP/ds_swizzle-based shuffles.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

}  // namespace vs

// vs_quantize_residual: per-128-token-block E4M3 quantizers.
//
// TeleFuser PR #40 ("Changes"): K is centred by its sequence mean in FP32
// before E4M3 quantization.  VC-Attention summary (Key Contribution 1): each
// hardware block subtracts its V mean and only the residual is quantized.
// The block's scale is set by its largest entry (VC-Attention abstract): the
// power of two 2^e, e the smallest integer with amax <= 448 * 2^e (e >= -126),
// codes = E4M3(x * 2^-e), for Q, centred K and the V residual alike -- an
// E8M0 block scale that the FP8 matrix core applies itself in QK^T and PV.
// Q is multiplied by c = softmax_scale * log2(e) in FP32 first, so the QK^T
// product is the score in log2 units.
//
// One workgroup per (block, head, batch).  The block (128 tokens x D) is read
// once from HBM into registers (64 values per thread at D = 128), reduced to
// its amax, encoded with the hardware E4M3 conversion (round to nearest even
// after clamping to +-448, i.e. saturating), and written once:
//   Q, K  -> [B,H,S_pad,D], one row of D codes per token;
//   V     -> [B,H,nb,D,128], per block one row of 128 token codes per
//            channel, tokens in the order the attention kernel's MFMA B/A
//            operand layout consumes (transposed through LDS).
// The Q pass also emits q_mu[s] = c * (q_s . mu_K) from the bf16 q.
#include <float.h>

#include "common.h"

namespace vs {
namespace {

// Position inside a V block row of token tau (inverse of the order documented
// in vsmooth.h): the 32x32x64 MFMA consumes tokens 64kk + 32c + 8a + 4h + i
// at byte 64kk + 32h + 16c + 4a + i.
__device__ __forceinline__ int v_pos(int tau) {
  return (tau & ~63) | (((tau >> 2) & 1) << 5) | (((tau >> 5) & 1) << 4) |
         (((tau >> 3) & 3) << 2) | (tau & 3);
}

// Block amax over the workgroup (4 waves): wave max, then across waves.
__device__ __forceinline__ float block_amax(float a, float* red4) {
  a = wave_max(a);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red4[w] = a;
  __syncthreads();
  a = __builtin_fmaxf(__builtin_fmaxf(red4[0], red4[1]), __builtin_fmaxf(red4[2], red4[3]));
  return a;
}

// Load TPT tokens x 8 channels of one block into float32 registers, with an
// optional per-channel mean subtracted (one float32 subtraction).  Invalid
// (padding) tokens are +0.
template <int D>
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int layout, int b,
                                           int h, int j, int S, int H,
                                           const float* __restrict__ mean8,
                                           float (&val)[kBlock / (256 / (D / 8))][8]) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = mean8 ? mean8[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    if (tok < S) {
      const uint4 w = *reinterpret_cast<const uint4*>(x + token_offset(layout, b, tok, h, S, H, D) + 8 * c);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        val[i][2 * e] = mean8 ? bf16_to_f32(ww[e] & 0xFFFFu) - mu[2 * e] : bf16_to_f32(ww[e] & 0xFFFFu);
        val[i][2 * e + 1] = mean8 ? bf16_to_f32(ww[e] >> 16) - mu[2 * e + 1] : bf16_to_f32(ww[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) val[i][e] = 0.0f;
    }
  }
}

// Smallest e >= -126 with amax <= 448 * 2^e (0 when amax == 0).
__device__ __forceinline__ int pow2_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = ilogbf(amax) - 8;
  while (amax > ldexpf(448.0f, e)) ++e;
  while (e > -126 && amax <= ldexpf(448.0f, e - 1)) --e;
  return e < -126 ? -126 : e;
}

// Q (mean == nullptr, scaled by pre = c) or centred K (pre = 1): codes as
// token rows.  With q_mu != nullptr also q_mu[s] = c * (q_s . k_mean) from
// the bf16 q.
template <int D>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int layout, int S, int H, int nb,
    const float* __restrict__ mean, float pre, uint8_t* __restrict__ codes,
    float* __restrict__ scale_out, const float* __restrict__ k_mean,
    float* __restrict__ q_mu, float c_log2) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  __shared__ float red4[4];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const float* mean8 = mean ? mean + bh * D + 8 * c : nullptr;

  float val[TPT][8];
  load_block<D>(x, layout, b, h, j, S, H, mean8, val);

  if (q_mu) {
    float km[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) km[e] = k_mean[bh * D + 8 * c + e];
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(val[i][e], km[e], dot);
#pragma unroll
      for (int o = CH / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
      const int tok = j * kBlock + r + ROWS * i;
      if (c == 0 && tok < S) q_mu[bh * S + tok] = dot * c_log2;
    }
  }

  if (pre != 1.0f) {
#pragma unroll
    for (int i = 0; i < TPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) val[i][e] *= pre;
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(val[i][e]));
  const float amax = block_amax(a, red4);
  const int ex = pow2_exponent(amax);
  const float inv = ldexpf(1.0f, -ex);
  if (threadIdx.x == 0) scale_out[bh * nb + j] = ldexpf(1.0f, ex);

  const size_t S_pad = static_cast<size_t>(nb) * kBlock;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    uint32_t w0 = 0, w1 = 0;
    w0 = cvt_pk_e4m3<false>(clamp448(val[i][0] * inv), clamp448(val[i][1] * inv), w0);
    w0 = cvt_pk_e4m3<true>(clamp448(val[i][2] * inv), clamp448(val[i][3] * inv), w0);
    w1 = cvt_pk_e4m3<false>(clamp448(val[i][4] * inv), clamp448(val[i][5] * inv), w1);
    w1 = cvt_pk_e4m3<true>(clamp448(val[i][6] * inv), clamp448(val[i][7] * inv), w1);
    *reinterpret_cast<uint2*>(codes + (bh * S_pad + tok) * D + 8 * c) = make_uint2(w0, w1);
  }
}

// Residual V: codes transposed per block, [D][128] in the MFMA token order,
// power-of-two scale.
template <int D>
__global__ __launch_bounds__(256) void quant_vt_kernel(
    const uint16_t* __restrict__ x, int layout, int S, int H, int nb,
    const float* __restrict__ v_mean, int vmean_mode, uint8_t* __restrict__ codes,
    float* __restrict__ scale_out) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  __shared__ float red4[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * kBlock];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const float* mean8 = nullptr;
  if (vmean_mode == VS_VMEAN_BLOCK) mean8 = v_mean + (bh * nb + j) * D + 8 * c;
  else if (vmean_mode == VS_VMEAN_SEQ) mean8 = v_mean + bh * D + 8 * c;

  float val[TPT][8];
  load_block<D>(x, layout, b, h, j, S, H, mean8, val);
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    if (tok < S) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(val[i][e]));
    }
  }
  const float amax = block_amax(a, red4);
  const int e = pow2_exponent(amax);
  const float inv = ldexpf(1.0f, -e);
  if (threadIdx.x == 0) scale_out[bh * nb + j] = ldexpf(1.0f, e);

#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tau = r + ROWS * i;            // token inside the block
    const int tok = j * kBlock + tau;
    uint32_t w0 = 0, w1 = 0;
    if (tok < S) {
      w0 = cvt_pk_e4m3<false>(clamp448(val[i][0] * inv), clamp448(val[i][1] * inv), w0);
      w0 = cvt_pk_e4m3<true>(clamp448(val[i][2] * inv), clamp448(val[i][3] * inv), w0);
      w1 = cvt_pk_e4m3<false>(clamp448(val[i][4] * inv), clamp448(val[i][5] * inv), w1);
      w1 = cvt_pk_e4m3<true>(clamp448(val[i][6] * inv), clamp448(val[i][7] * inv), w1);
    }
    const int p = v_pos(tau);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[(8 * c + e) * kBlock + p] = static_cast<uint8_t>(w0 >> (8 * e));
      tile[(8 * c + 4 + e) * kBlock + p] = static_cast<uint8_t>(w1 >> (8 * e));
    }
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(codes + (bh * nb + j) * static_cast<size_t>(D) * kBlock);
  const uint4* src = reinterpret_cast<const uint4*>(tile);
#pragma unroll
  for (int i = 0; i < D * kBlock / 16 / 256; ++i) dst[threadIdx.x + 256 * i] = src[threadIdx.x + 256 * i];
}

}  // namespace
}  // namespace vs

extern "C" int vs_quantize_residual(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    int kv_layout, int B, int S, int H, int D,
                                    float softmax_scale, const float* k_mean,
                                    const float* v_mean, int vmean_mode, uint8_t* q8,
                                    float* q_scale, uint8_t* k8, float* k_scale, uint8_t* v8,
                                    float* v_scale, float* q_mu, void* stream) {
  using namespace vs;
  if (B < 0 || S < 0 || H < 0) return VS_ERR_INVALID_ARG;
  if (kv_layout != VS_LAYOUT_BSHD && kv_layout != VS_LAYOUT_BHSD) return VS_ERR_INVALID_ARG;
  if (vmean_mode != VS_VMEAN_NONE && vmean_mode != VS_VMEAN_BLOCK && vmean_mode != VS_VMEAN_SEQ)
    return VS_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !(softmax_scale <= FLT_MAX)) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (B == 0 || S == 0 || H == 0) return VS_OK;
  if ((vmean_mode == VS_VMEAN_NONE) != (v_mean == nullptr)) return VS_ERR_INVALID_ARG;
  if (k_mean && !q_mu) return VS_ERR_INVALID_ARG;
  if (!q || !k || !v || !q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale)
    return VS_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, k_mean, v_mean, q8, q_scale, k8, k_scale, v8, v_scale, q_mu};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VS_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535) return VS_ERR_UNSUPPORTED;

  const int nb = n_blocks(S);
  const float c_log2 = softmax_scale * 1.44269504088896341f;
  hipStream_t st = as_stream(stream);
  const dim3 grid(nb, H, B), block(256);
  if (D == 128) {
    hipLaunchKernelGGL(quant_rows_kernel<128>, grid, block, 0, st, q, VS_LAYOUT_BSHD, S, H, nb,
                       nullptr, c_log2, q8, q_scale, k_mean, k_mean ? q_mu : nullptr, c_log2);
    hipLaunchKernelGGL(quant_rows_kernel<128>, grid, block, 0, st, k, kv_layout, S, H, nb, k_mean,
                       1.0f, k8, k_scale, nullptr, nullptr, c_log2);
    hipLaunchKernelGGL(quant_vt_kernel<128>, grid, block, 0, st, v, kv_layout, S, H, nb, v_mean,
                       vmean_mode, v8, v_scale);
  } else {
    hipLaunchKernelGGL(quant_rows_kernel<64>, grid, block, 0, st, q, VS_LAYOUT_BSHD, S, H, nb,
                       nullptr, c_log2, q8, q_scale, k_mean, k_mean ? q_mu : nullptr, c_log2);
    hipLaunchKernelGGL(quant_rows_kernel<64>, grid, block, 0, st, k, kv_layout, S, H, nb, k_mean,
                       1.0f, k8, k_scale, nullptr, nullptr, c_log2);
    hipLaunchKernelGGL(quant_vt_kernel<64>, grid, block, 0, st, v, kv_layout, S, H, nb, v_mean,
                       vmean_mode, v8, v_scale);
  }
  return launch_status();
}

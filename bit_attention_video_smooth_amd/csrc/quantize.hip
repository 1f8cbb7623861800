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
//
// Gather fused in (vs_quantize_residual_perm): with a permutation, row i of
// head h's K and V blocks is read from token perm[b, h, i] of the caller's
// [B,S,H,D] tensors, so the permuted K and V are never written to HBM
// (VC-Attention summary, Key Contribution 3: the grouping's gather is part of
// the fused prologue).
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

// Grid of one (block, head) per workgroup.  With token-major input (BSHD)
// the head is the fastest index (hfast), so workgroups that run together
// read neighbouring 256-byte pieces of the same token rows instead of rows
// 128 tokens apart; with head-major input (BHSD) the block is.  gridDim.y
// caps the slower index at 65535.
struct BlockGrid {
  dim3 grid;
  int hfast;
};
inline BlockGrid block_grid(int layout, int nb, int H, int B) {
  if (layout == VS_LAYOUT_BSHD && nb <= 65535) return {dim3(H, nb, B), 1};
  return {dim3(nb, H, B), 0};
}

// Source token of block row `tok`: perm[b, h, tok] (BSHD input; entries
// outside [0, S) are clamped, so a bad permutation cannot read out of
// bounds), or tok itself without a permutation.
template <bool PERM>
__device__ __forceinline__ int src_token(const int32_t* __restrict__ perm, size_t bh, int S,
                                         int tok) {
  if (!PERM) return tok;
  const int s = perm[bh * S + tok];
  return s < 0 ? 0 : (s >= S ? S - 1 : s);
}

// Load TPT tokens x 8 channels of one block into float32 registers, rotated
// by the rotary tables first (ROPE: row src of cos / sin, [S, D/2], pairs
// 4c .. 4c + 3 for the thread's channels 8c .. 8c + 7), with an optional
// per-channel mean subtracted (one float32 subtraction).  Invalid (padding)
// tokens are +0.
template <int D, bool PERM, bool ROPE>
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int layout, int b,
                                           int h, int j, int S, int H,
                                           const float* __restrict__ mean8,
                                           const int32_t* __restrict__ perm,
                                           const float* __restrict__ rope_cos,
                                           const float* __restrict__ rope_sin,
                                           float (&val)[kBlock / (256 / (D / 8))][8]) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = mean8 ? mean8[e] : 0.0f;
  // permuted rows: all source indices first, so their loads overlap
  int srcs[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    srcs[i] = PERM ? src_token<PERM>(perm, static_cast<size_t>(b) * H + h, S, tok < S ? tok : S - 1)
                   : tok;
  }
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    if (tok < S) {
      const int src = srcs[i];
      const uint4 w = *reinterpret_cast<const uint4*>(x + token_offset(layout, b, src, h, S, H, D) + 8 * c);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        val[i][2 * e] = bf16_to_f32(ww[e] & 0xFFFFu);
        val[i][2 * e + 1] = bf16_to_f32(ww[e] >> 16);
      }
      if (ROPE) {
        const size_t t = static_cast<size_t>(src) * (D / 2) + 4 * c;
        rope8(val[i], *reinterpret_cast<const float4*>(rope_cos + t),
              *reinterpret_cast<const float4*>(rope_sin + t));
      }
      if (mean8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) val[i][e] -= mu[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) val[i][e] = 0.0f;
    }
  }
}

// x of lane (lane ^ J), J in {1, 2, 4, 8}: DPP quad permutations for 1 and
// 2, the swizzle unit's bit-mask mode (xor within 32 lanes) for 4 and 8 --
// no LDS address round trip.
__device__ __forceinline__ float lane_xor(float x, int j) {
  const int v = __float_as_int(x);
  int r;
  switch (j) {
    case 1: r = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); break;  // quad [1,0,3,2]
    case 2: r = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false); break;  // quad [2,3,0,1]
    case 4: r = __builtin_amdgcn_ds_swizzle(v, 0x101F); break;              // and 0x1F, xor 4
    default: r = __builtin_amdgcn_ds_swizzle(v, 0x201F); break;             // and 0x1F, xor 8
  }
  return __int_as_float(r);
}

// Rows of a block times the Sylvester Hadamard matrix H_D (entries +-1),
// in float32: the butterfly (a, b) -> (a + b, a - b) over channel bit 0,
// then bit 1, and so on -- channel bits 0-2 inside a thread's 8 channels,
// the higher bits across the CH lanes of a token row (lane bit j holds
// channel bit 3 + j), where the lane with the bit set keeps its partner's
// value minus its own.  Each sum and difference is rounded once, in this
// order (it decides the codes).  (VC-Attention summary, Key Contribution 3:
// the QK Hadamard rotation belongs to the fused quantizer prologue.)
template <int D>
__device__ __forceinline__ void hadamard_rows(float (&val)[kBlock / (256 / (D / 8))][8]) {
  constexpr int CH = D / 8, TPT = kBlock / (256 / CH);
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & h)) {
          const float a = val[i][e], b = val[i][e + h];
          val[i][e] = a + b;
          val[i][e + h] = a - b;
        }
  }
  const int c = threadIdx.x % CH;
#pragma unroll
  for (int j = 1; j < CH; j <<= 1) {
    const bool hi = (c & j) != 0;
#pragma unroll
    for (int i = 0; i < TPT; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = val[i][e];
        const float y = lane_xor(x, j);
        val[i][e] = hi ? y - x : x + y;
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
// the bf16 q.  PERM: rows gathered through perm (K only).  HAD: rows
// rotated by H_D after the centring and before the scaling by pre (the
// caller folds Q's 1/D into pre).  ROPE: rows rotated by the rotary
// tables first (before the centring; q_mu from the rotated q).  B16:
// instead of the E4M3 bytes, each
// code's value times the block scale as bf16 (2 bytes per element, same
// row layout): E4M3 values carry 4 significant bits, so the bf16 is exact
// whenever the smallest code times the scale is a bf16 number
// (scale >= 2^-124).
template <int D, bool PERM, bool HAD, bool B16, bool ROPE>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int layout, int S, int H, int nb,
    const float* __restrict__ mean, float pre, uint8_t* __restrict__ codes,
    float* __restrict__ scale_out, const float* __restrict__ k_mean,
    float* __restrict__ q_mu, float c_log2, int hfast, const int32_t* __restrict__ perm,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  __shared__ float red4[4];
  const int j = hfast ? blockIdx.y : blockIdx.x, h = hfast ? blockIdx.x : blockIdx.y,
            b = blockIdx.z;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const float* mean8 = mean ? mean + bh * D + 8 * c : nullptr;

  float val[TPT][8];
  load_block<D, PERM, ROPE>(x, layout, b, h, j, S, H, mean8, perm, rope_cos, rope_sin, val);

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

  if (HAD) hadamard_rows<D>(val);
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
  const float sc = ldexpf(1.0f, ex);
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    uint32_t w0 = 0, w1 = 0;
    w0 = cvt_pk_e4m3<false>(clamp448(val[i][0] * inv), clamp448(val[i][1] * inv), w0);
    w0 = cvt_pk_e4m3<true>(clamp448(val[i][2] * inv), clamp448(val[i][3] * inv), w0);
    w1 = cvt_pk_e4m3<false>(clamp448(val[i][4] * inv), clamp448(val[i][5] * inv), w1);
    w1 = cvt_pk_e4m3<true>(clamp448(val[i][6] * inv), clamp448(val[i][7] * inv), w1);
    if (B16) {
      // decoded values (hardware E4M3 -> f32, exact), times the power-of-two
      // scale (exact), rounded to bf16 (nearest even; exact here)
      const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), false);
      const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w0), true);
      const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), false);
      const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w1), true);
      const uint32_t o[4] = {f32x2_to_bf16x2(f0[0] * sc, f0[1] * sc),
                             f32x2_to_bf16x2(f1[0] * sc, f1[1] * sc),
                             f32x2_to_bf16x2(f2[0] * sc, f2[1] * sc),
                             f32x2_to_bf16x2(f3[0] * sc, f3[1] * sc)};
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(codes) + (bh * S_pad + tok) * D + 8 * c) =
          make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      *reinterpret_cast<uint2*>(codes + (bh * S_pad + tok) * D + 8 * c) = make_uint2(w0, w1);
    }
  }
}

// OCP MX FP4 (E2M1) nibble of x: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6,
// ties to the even code (mantissa bit 0), saturating at 6, sign kept.
// Below 1 the codes 0, 1, 2 step by 0.5: rint(2 |x|) (round half to even).
// From 1 up a code is 2 + 2 e + m for |x| = 2^e (1 + m / 2): the float's
// bits rounded to one mantissa bit, ties to even (add 2^21 - 1 plus the
// kept bit, carry into the exponent), then exponent and bit read together.
__device__ __forceinline__ uint32_t fp4_code(float x) {
  const float m = __builtin_fabsf(x);
  const uint32_t b = __float_as_uint(m);
  const uint32_t r = (b + 0x1FFFFFu + ((b >> 22) & 1u)) >> 22;
  const uint32_t hi = min(r - 252u, 7u);
  const uint32_t lo = static_cast<uint32_t>(__builtin_rintf(2.0f * m));
  return (m < 1.0f ? lo : hi) | (__float_as_uint(x) >> 31 << 3);
}

// Value of an E2M1 nibble (sign in bit 3): 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float fp4_value(uint32_t code) {
  const uint32_t m = code & 7u;
  const float mag = m < 2u ? 0.5f * static_cast<float>(m)
                           : ldexpf(1.0f + 0.5f * static_cast<float>(m & 1u), static_cast<int>(m >> 1) - 1);
  return (code & 8u) ? -mag : mag;
}

// The bf16 V tile in LDS: channel row d of 128 tokens, 8-byte units (4
// tokens) XOR-swizzled by d / 8 so that the 16 channel groups of a wave's
// stores fall on different banks.  Token tau sits at position p16(tau):
// bits 2 and 3 of tau swapped (the bf16 PV product's k order); the four
// tokens 4a .. 4a + 3 of a quad stay together in unit
// 4 (a / 4) + ((a / 2) % 2) + 2 (a % 2).
__device__ __forceinline__ int quad_unit16(int a) { return 4 * (a >> 2) + ((a >> 1) & 1) + 2 * (a & 1); }

__device__ __forceinline__ void store_quad16(uint16_t* tile16, int d, int a, const float (&x)[4]) {
  const int u = quad_unit16(a) ^ ((d >> 3) & 31);
  *reinterpret_cast<uint2*>(tile16 + d * kBlock + 4 * u) =
      make_uint2(f32x2_to_bf16x2(x[0], x[1]), f32x2_to_bf16x2(x[2], x[3]));
}

// The LDS tile, unswizzled, to its global [D][128] bf16 place.
template <int D>
__device__ __forceinline__ void copy_out16(const uint16_t* tile16, uint16_t* dst) {
  for (int g = threadIdx.x; g < D * kBlock / 4; g += 256) {
    const int d = g >> 5, u = g & 31;
    *reinterpret_cast<uint2*>(dst + 4 * g) =
        *reinterpret_cast<const uint2*>(tile16 + d * kBlock + 4 * (u ^ ((d >> 3) & 31)));
  }
}

// Smallest e >= -127 with amax <= 6 * 2^e (0 when amax == 0).
__device__ __forceinline__ int fp4_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = ilogbf(amax) - 2;
  while (amax > ldexpf(6.0f, e)) ++e;
  while (e > -127 && amax <= ldexpf(6.0f, e - 1)) --e;
  return e < -127 ? -127 : e;
}

// Columns k of the 4x4 byte matrix whose rows are w[0..3]: byte k of the
// result e is byte e of w[k] (two rounds of v_perm_b32).
__device__ __forceinline__ void transpose4x4(const uint32_t (&w)[4], uint32_t (&col)[4]) {
  const uint32_t x0 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
  const uint32_t x1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
  const uint32_t y0 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const uint32_t y1 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  col[0] = __builtin_amdgcn_perm(y0, x0, 0x05040100u);
  col[1] = __builtin_amdgcn_perm(y0, x0, 0x07060302u);
  col[2] = __builtin_amdgcn_perm(y1, x1, 0x05040100u);
  col[3] = __builtin_amdgcn_perm(y1, x1, 0x07060302u);
}

// Residual V: codes transposed per block, [D][128] in the MFMA token order,
// power-of-two scale.  Thread t owns channels 8 (t % CH) .. + 7 and whole
// token quads 4a .. 4a + 3: v_pos keeps a quad's four tokens in one aligned
// dword, so a byte transpose in registers yields one dword per channel and
// quad.  The LDS tile is XOR-swizzled by 16-byte chunk (chunk ^ (d / 8) % 8
// in row d) so the dword writes of a wave, whose rows d are 1 KB apart,
// spread over the banks; the copy-out reads it back in row order.
//
// OWN_MEAN (mode VS_VMEAN_BLOCK_OUT): the block mean is formed here from the
// values already in registers -- float64 sums of the bf16 values (exact),
// per thread, then over the threads of a channel group in a fixed order, one
// division, one rounding to float32, as vs_smooth_stats forms it -- written
// to v_mean and subtracted.
//
// FP4 (VS_V_MXFP4): the residual as OCP MX FP4 (E2M1) codes with one E8M0
// scale per channel and 32 consecutive tokens (group g = tokens 32g..32g+31
// of the block), the smallest power of two 2^e (e >= -127) with
// amax <= 6 * 2^e; codes round to nearest even (fp4_code).  Per block a
// D x 64-byte tile: channel row d holds group g in bytes 16g..16g+15, in
// the k order of the 4-bit A operand of the FP8/FP4 matrix core -- nibble
// q (low nibble first) is token 8 ((q % 16) / 4) + 4 (q / 16) + q % 4 of
// the group -- and scale_out is u8 [B,H,nb,D,4], byte g = e + 127.
//
// nat (VS_P_MXFP4, E4M3 codes only): position p of a channel row holds
// token p with bits 4 and 5 swapped -- the k order in which the attention
// kernel's 4-bit probability tile (lane half h: k positions 16 h .. + 15
// and 32 + 16 h .. + 15) meets V, so that each lane's 32 probabilities are
// 32 consecutive keys.
//
// B16 (VS_BF16_MMA): instead of the codes, each quantized residual's value
// (the E4M3 or E2M1 code's value times its scale, exact in bf16) as bf16,
// per block a D x 128 tile with token tau of a channel row at position
// p16(tau) (bits 2 and 3 of tau swapped: the k order of the bf16 matrix
// core's PV product); scale_out as without it.
template <int D, bool OWN_MEAN, bool PERM, bool FP4, bool B16>
__global__ __launch_bounds__(256) void quant_vt_kernel(
    const uint16_t* __restrict__ x, int layout, int S, int H, int nb,
    float* __restrict__ v_mean, int vmean_mode, uint8_t* __restrict__ codes,
    float* __restrict__ scale_out, int hfast, const int32_t* __restrict__ perm, int nat) {
  constexpr int CH = D / 8;              // 8-channel groups
  constexpr int QR = 256 / CH;           // quads in flight per pass
  constexpr int NQ = kBlock / 4 / QR;    // quads per thread
  __shared__ float red4[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[B16 ? 16 : D * kBlock];
  __shared__ __attribute__((aligned(16))) uint16_t tile16[B16 ? D * kBlock : 8];
  __shared__ double part[OWN_MEAN ? QR : 1][OWN_MEAN ? D : 1];
  __shared__ float smean[OWN_MEAN ? D : 1];
  const int j = hfast ? blockIdx.y : blockIdx.x, h = hfast ? blockIdx.x : blockIdx.y,
            b = blockIdx.z;
  const int c = threadIdx.x % CH, a0 = threadIdx.x / CH;
  const size_t bh = static_cast<size_t>(b) * H + h;
  float mu[8];
  {
    const float* mean8 = nullptr;
    if (!OWN_MEAN && vmean_mode == VS_VMEAN_BLOCK) mean8 = v_mean + (bh * nb + j) * D + 8 * c;
    else if (vmean_mode == VS_VMEAN_SEQ) mean8 = v_mean + bh * D + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) mu[e] = mean8 ? mean8[e] : 0.0f;
  }

  // residuals in float32; padding tokens are +0
  // permuted rows: all source indices first, so their loads overlap
  int srcs[NQ][4];
#pragma unroll
  for (int n = 0; n < NQ; ++n)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tok = j * kBlock + 4 * (a0 + QR * n) + q;
      srcs[n][q] = PERM ? src_token<PERM>(perm, bh, S, tok < S ? tok : S - 1) : tok;
    }
  float val[NQ][4][8];
#pragma unroll
  for (int n = 0; n < NQ; ++n)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tok = j * kBlock + 4 * (a0 + QR * n) + q;
      if (tok < S) {
        const int src = srcs[n][q];
        const uint4 w = *reinterpret_cast<const uint4*>(x + token_offset(layout, b, src, h, S, H, D) + 8 * c);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          val[n][q][2 * e] = bf16_to_f32(ww[e] & 0xFFFFu) - mu[2 * e];
          val[n][q][2 * e + 1] = bf16_to_f32(ww[e] >> 16) - mu[2 * e + 1];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) val[n][q][e] = 0.0f;
      }
    }
  if (OWN_MEAN) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      double sum = 0.0;
#pragma unroll
      for (int n = 0; n < NQ; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) sum += static_cast<double>(val[n][q][e]);
      part[a0][8 * c + e] = sum;
    }
    __syncthreads();
    if (threadIdx.x < D) {
      double sum = 0.0;
      for (int r = 0; r < QR; ++r) sum += part[r][threadIdx.x];
      const float m = static_cast<float>(sum / static_cast<double>(min(kBlock, S - j * kBlock)));
      smean[threadIdx.x] = m;
      v_mean[(bh * nb + j) * D + threadIdx.x] = m;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float m = smean[8 * c + e];
#pragma unroll
      for (int n = 0; n < NQ; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (j * kBlock + 4 * (a0 + QR * n) + q < S) val[n][q][e] -= m;
    }
  }
  if constexpr (FP4) {
    // group maxima (float bits of non-negative values order as integers);
    // a quad of tokens 4a..4a+3 lies in group a / 8
    __shared__ unsigned gmax[4][D];
    __shared__ int gexp[4][D];
    uint8_t* tile4 = tile;                       // D x 64 bytes of the tile
    for (int i = threadIdx.x; i < 4 * D; i += 256) (&gmax[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      const int g = (a0 + QR * n) >> 3;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) m = __builtin_fmaxf(m, __builtin_fabsf(val[n][q][e]));
        atomicMax(&gmax[g][8 * c + e], __float_as_uint(m));
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 4 * D; i += 256) {
      const int g = i / D, d = i % D;
      const int ex = fp4_exponent(__uint_as_float(gmax[g][d]));
      gexp[g][d] = ex;
      reinterpret_cast<uint8_t*>(scale_out)[((bh * nb + j) * D + d) * 4 + g] =
          static_cast<uint8_t>(ex + 127);
    }
    __syncthreads();
    if constexpr (B16) {
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const int a = a0 + QR * n, g = a >> 3;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int ex = gexp[g][8 * c + e];
          const float inv = ldexpf(1.0f, -ex), sc = ldexpf(1.0f, ex);
          float x[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) x[q] = fp4_value(fp4_code(val[n][q][e] * inv)) * sc;
          store_quad16(tile16, 8 * c + e, a, x);
        }
      }
      __syncthreads();
      copy_out16<D>(tile16, reinterpret_cast<uint16_t*>(codes) + (bh * nb + j) * static_cast<size_t>(D) * kBlock);
    } else {
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        const int a = a0 + QR * n, g = a >> 3;
        // the quad's four nibbles: bytes 8 (a % 2) + 2 ((a % 8) / 2) of the group
        const int off = 16 * g + 8 * (a & 1) + 2 * ((a & 7) >> 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float inv = ldexpf(1.0f, -gexp[g][8 * c + e]);
          uint32_t w = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) w |= fp4_code(val[n][q][e] * inv) << (4 * q);
          *reinterpret_cast<uint16_t*>(tile4 + (8 * c + e) * 64 + off) = static_cast<uint16_t>(w);
        }
      }
      __syncthreads();
      uint4* dst = reinterpret_cast<uint4*>(codes + (bh * nb + j) * static_cast<size_t>(D) * 64);
      for (int idx = threadIdx.x; idx < D * 64 / 16; idx += 256)
        dst[idx] = *reinterpret_cast<const uint4*>(tile4 + 16 * idx);
    }
    return;
  }
  float a = 0.0f;
#pragma unroll
  for (int n = 0; n < NQ; ++n)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(val[n][q][e]));
  const float amax = block_amax(a, red4);
  const int e = pow2_exponent(amax);
  const float inv = ldexpf(1.0f, -e);
  if (threadIdx.x == 0) scale_out[bh * nb + j] = ldexpf(1.0f, e);

  if constexpr (B16) {
    const float sc = ldexpf(1.0f, e);
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
      float x[8][4];                       // channel e2, token q of the quad
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float* v = val[n][q];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint32_t w = cvt_pk_e4m3<false>(clamp448(v[4 * h2] * inv), clamp448(v[4 * h2 + 1] * inv), 0u);
          w = cvt_pk_e4m3<true>(clamp448(v[4 * h2 + 2] * inv), clamp448(v[4 * h2 + 3] * inv), w);
          const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
          const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
          x[4 * h2 + 0][q] = f0[0] * sc;
          x[4 * h2 + 1][q] = f0[1] * sc;
          x[4 * h2 + 2][q] = f1[0] * sc;
          x[4 * h2 + 3][q] = f1[1] * sc;
        }
      }
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) store_quad16(tile16, 8 * c + e2, a0 + QR * n, x[e2]);
    }
    __syncthreads();
    copy_out16<D>(tile16, reinterpret_cast<uint16_t*>(codes) + (bh * nb + j) * static_cast<size_t>(D) * kBlock);
  } else {
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    uint32_t lo[4], hi[4];                 // token q: channels 0-3, 4-7
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* v = val[n][q];
      lo[q] = cvt_pk_e4m3<false>(clamp448(v[0] * inv), clamp448(v[1] * inv), 0u);
      lo[q] = cvt_pk_e4m3<true>(clamp448(v[2] * inv), clamp448(v[3] * inv), lo[q]);
      hi[q] = cvt_pk_e4m3<false>(clamp448(v[4] * inv), clamp448(v[5] * inv), 0u);
      hi[q] = cvt_pk_e4m3<true>(clamp448(v[6] * inv), clamp448(v[7] * inv), hi[q]);
    }
    uint32_t col[8];                       // channel e: the quad's 4 tokens
    transpose4x4(lo, *reinterpret_cast<uint32_t(*)[4]>(col));
    transpose4x4(hi, *reinterpret_cast<uint32_t(*)[4]>(col + 4));
    // byte of token 4a (a multiple of 4): the FP8 MFMA token order, or (nat)
    // the token order with bits 4 and 5 swapped
    const int t4 = 4 * (a0 + QR * n);
    const int p = nat ? (t4 & ~48) | (((t4 >> 4) & 1) << 5) | (((t4 >> 5) & 1) << 4) : v_pos(t4);
    const int swz = ((p >> 4) ^ (c & 7)) << 4 | (p & 15);
#pragma unroll
    for (int e2 = 0; e2 < 8; ++e2)
      *reinterpret_cast<uint32_t*>(tile + (8 * c + e2) * kBlock + swz) = col[e2];
  }
  __syncthreads();
  uint4* dst = reinterpret_cast<uint4*>(codes + (bh * nb + j) * static_cast<size_t>(D) * kBlock);
#pragma unroll
  for (int i = 0; i < D * kBlock / 16 / 256; ++i) {
    const int idx = threadIdx.x + 256 * i;   // 16-byte chunk of the row-major tile
    const int row = idx >> 3, ch = idx & 7;
    dst[idx] = *reinterpret_cast<const uint4*>(tile + row * kBlock + ((ch ^ ((row >> 3) & 7)) << 4));
  }
  }
}

}  // namespace
}  // namespace vs

namespace vs {
namespace {

template <int D, bool PERM, bool HAD, bool FP4, bool B16>
void launch_quant(const BlockGrid& gq, const BlockGrid& gkv, hipStream_t st, const uint16_t* q,
                  const uint16_t* k, const uint16_t* v, int kv_layout, int S, int H, int nb,
                  float c_log2, const float* k_mean, float* v_mean, int vmean_mode, uint8_t* q8,
                  float* q_scale, uint8_t* k8, float* k_scale, uint8_t* v8, float* v_scale,
                  float* q_mu, const int32_t* perm, const float* rope_cos,
                  const float* rope_sin, int nat) {
  const dim3 block(256);
  // with the rotation Q carries its 1/D (a power of two: exact)
  const float q_pre = HAD ? c_log2 * (1.0f / D) : c_log2;
  if (rope_cos) {
    hipLaunchKernelGGL((quant_rows_kernel<D, false, HAD, B16, true>), gq.grid, block, 0, st, q,
                       VS_LAYOUT_BSHD, S, H, nb, nullptr, q_pre, q8, q_scale, k_mean,
                       k_mean ? q_mu : nullptr, c_log2, gq.hfast, nullptr, rope_cos, rope_sin);
    hipLaunchKernelGGL((quant_rows_kernel<D, PERM, HAD, B16, true>), gkv.grid, block, 0, st, k,
                       kv_layout, S, H, nb, k_mean, 1.0f, k8, k_scale, nullptr, nullptr, c_log2,
                       gkv.hfast, perm, rope_cos, rope_sin);
  } else {
    hipLaunchKernelGGL((quant_rows_kernel<D, false, HAD, B16, false>), gq.grid, block, 0, st, q,
                       VS_LAYOUT_BSHD, S, H, nb, nullptr, q_pre, q8, q_scale, k_mean,
                       k_mean ? q_mu : nullptr, c_log2, gq.hfast, nullptr, nullptr, nullptr);
    hipLaunchKernelGGL((quant_rows_kernel<D, PERM, HAD, B16, false>), gkv.grid, block, 0, st, k,
                       kv_layout, S, H, nb, k_mean, 1.0f, k8, k_scale, nullptr, nullptr, c_log2,
                       gkv.hfast, perm, nullptr, nullptr);
  }
  if (vmean_mode == VS_VMEAN_BLOCK_OUT)
    hipLaunchKernelGGL((quant_vt_kernel<D, true, PERM, FP4, B16>), gkv.grid, block, 0, st, v,
                       kv_layout, S, H, nb, v_mean, vmean_mode, v8, v_scale, gkv.hfast, perm,
                       nat);
  else
    hipLaunchKernelGGL((quant_vt_kernel<D, false, PERM, FP4, B16>), gkv.grid, block, 0, st, v,
                       kv_layout, S, H, nb, v_mean, vmean_mode, v8, v_scale, gkv.hfast, perm,
                       nat);
}

int quantize_residual(const uint16_t* q, const uint16_t* k, const uint16_t* v, int kv_layout,
                      const int32_t* perm, unsigned flags, int B, int S, int H, int D,
                      float softmax_scale,
                      const float* k_mean, float* v_mean, int vmean_mode, uint8_t* q8,
                      float* q_scale, uint8_t* k8, float* k_scale, uint8_t* v8, float* v_scale,
                      float* q_mu, const float* rope_cos, const float* rope_sin, void* stream) {
  if (B < 0 || S < 0 || H < 0) return VS_ERR_INVALID_ARG;
  if (kv_layout != VS_LAYOUT_BSHD && kv_layout != VS_LAYOUT_BHSD) return VS_ERR_INVALID_ARG;
  if (perm && kv_layout != VS_LAYOUT_BSHD) return VS_ERR_INVALID_ARG;
  if (flags & ~(VS_QK_HADAMARD | VS_V_MXFP4 | VS_BF16_MMA | VS_P_MXFP4)) return VS_ERR_INVALID_ARG;
  // the 4-bit probability tile meets E4M3 V codes
  if ((flags & VS_P_MXFP4) && (flags & (VS_V_MXFP4 | VS_BF16_MMA))) return VS_ERR_INVALID_ARG;
  if (vmean_mode != VS_VMEAN_NONE && vmean_mode != VS_VMEAN_BLOCK && vmean_mode != VS_VMEAN_SEQ &&
      vmean_mode != VS_VMEAN_BLOCK_OUT)
    return VS_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !(softmax_scale <= FLT_MAX)) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (B == 0 || S == 0 || H == 0) return VS_OK;
  if ((vmean_mode == VS_VMEAN_NONE) != (v_mean == nullptr)) return VS_ERR_INVALID_ARG;
  if (k_mean && !q_mu) return VS_ERR_INVALID_ARG;
  if (!q || !k || !v || !q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale)
    return VS_ERR_INVALID_ARG;
  if (!rope_cos != !rope_sin) return VS_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, k_mean, v_mean, q8, q_scale, k8, k_scale, v8, v_scale, q_mu, perm,
                        rope_cos, rope_sin};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VS_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535) return VS_ERR_UNSUPPORTED;

  const int nb = n_blocks(S);
  const float c_log2 = softmax_scale * 1.44269504088896341f;
  hipStream_t st = as_stream(stream);
  const BlockGrid gq = block_grid(VS_LAYOUT_BSHD, nb, H, B), gkv = block_grid(kv_layout, nb, H, B);
#define VS_QUANT_ARGS gq, gkv, st, q, k, v, kv_layout, S, H, nb, c_log2, k_mean, v_mean, \
    vmean_mode, q8, q_scale, k8, k_scale, v8, v_scale, q_mu, perm, rope_cos, rope_sin, nat
  const bool had = (flags & VS_QK_HADAMARD) != 0, fp4 = (flags & VS_V_MXFP4) != 0;
  const bool b16 = (flags & VS_BF16_MMA) != 0;
  const int nat = (flags & VS_P_MXFP4) != 0;
  // (D, permutation, rotation, FP4 V, bf16 Q/K) -> one instantiation
  const int sel = (D == 128 ? 16 : 0) | (b16 ? 8 : 0) | (perm ? 4 : 0) | (had ? 2 : 0) | (fp4 ? 1 : 0);
  switch (sel) {
#define VS_Q(n, d, b, p, h, f) case n: launch_quant<d, p, h, f, b>(VS_QUANT_ARGS); break;
    VS_Q(0, 64, false, false, false, false) VS_Q(1, 64, false, false, false, true)
    VS_Q(2, 64, false, false, true, false) VS_Q(3, 64, false, false, true, true)
    VS_Q(4, 64, false, true, false, false) VS_Q(5, 64, false, true, false, true)
    VS_Q(6, 64, false, true, true, false) VS_Q(7, 64, false, true, true, true)
    VS_Q(8, 64, true, false, false, false) VS_Q(9, 64, true, false, false, true)
    VS_Q(10, 64, true, false, true, false) VS_Q(11, 64, true, false, true, true)
    VS_Q(12, 64, true, true, false, false) VS_Q(13, 64, true, true, false, true)
    VS_Q(14, 64, true, true, true, false) VS_Q(15, 64, true, true, true, true)
    VS_Q(16, 128, false, false, false, false) VS_Q(17, 128, false, false, false, true)
    VS_Q(18, 128, false, false, true, false) VS_Q(19, 128, false, false, true, true)
    VS_Q(20, 128, false, true, false, false) VS_Q(21, 128, false, true, false, true)
    VS_Q(22, 128, false, true, true, false) VS_Q(23, 128, false, true, true, true)
    VS_Q(24, 128, true, false, false, false) VS_Q(25, 128, true, false, false, true)
    VS_Q(26, 128, true, false, true, false) VS_Q(27, 128, true, false, true, true)
    VS_Q(28, 128, true, true, false, false) VS_Q(29, 128, true, true, false, true)
    VS_Q(30, 128, true, true, true, false)
    default: launch_quant<128, true, true, true, true>(VS_QUANT_ARGS); break;
#undef VS_Q
  }
#undef VS_QUANT_ARGS
  return launch_status();
}

}  // namespace
}  // namespace vs

extern "C" int vs_quantize_residual(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                    int kv_layout, int B, int S, int H, int D,
                                    float softmax_scale, const float* k_mean,
                                    float* v_mean, int vmean_mode, uint8_t* q8,
                                    float* q_scale, uint8_t* k8, float* k_scale, uint8_t* v8,
                                    float* v_scale, float* q_mu, void* stream) {
  return vs::quantize_residual(q, k, v, kv_layout, nullptr, 0u, B, S, H, D, softmax_scale, k_mean,
                               v_mean, vmean_mode, q8, q_scale, k8, k_scale, v8, v_scale, q_mu,
                               nullptr, nullptr, stream);
}

extern "C" int vs_quantize_residual_perm(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         const int32_t* perm, int B, int S, int H, int D,
                                         float softmax_scale, const float* k_mean,
                                         float* v_mean, int vmean_mode, uint8_t* q8,
                                         float* q_scale, uint8_t* k8, float* k_scale,
                                         uint8_t* v8, float* v_scale, float* q_mu,
                                         void* stream) {
  if (!perm && B > 0 && S > 0 && H > 0) return VS_ERR_INVALID_ARG;
  return vs::quantize_residual(q, k, v, VS_LAYOUT_BSHD, perm, 0u, B, S, H, D, softmax_scale, k_mean,
                               v_mean, vmean_mode, q8, q_scale, k8, k_scale, v8, v_scale, q_mu,
                               nullptr, nullptr, stream);
}

extern "C" int vs_quantize_residual_ex(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       int kv_layout, const int32_t* perm, unsigned flags, int B,
                                       int S, int H, int D, float softmax_scale,
                                       const float* rope_cos, const float* rope_sin,
                                       const float* k_mean, float* v_mean, int vmean_mode,
                                       uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                                       uint8_t* v8, float* v_scale, float* q_mu, void* stream) {
  return vs::quantize_residual(q, k, v, kv_layout, perm, flags, B, S, H, D, softmax_scale, k_mean,
                               v_mean, vmean_mode, q8, q_scale, k8, k_scale, v8, v_scale, q_mu,
                               rope_cos, rope_sin, stream);
}

// vs_fp8_attn_fwd: FP8 (E4M3) attention forward with the in-recurrence V-mean
// restore and the optional ExpCast-FP8 probability cast.
//
// Method (VC-Attention summary, Key Contributions 1-2 and "Methodology in
// Plain English"; abstract): QK^T and PV run on the low-bit matrix cores,
// the online softmax between them keeps a running row max and row sum, and
// each block's V mean is added back as a rank-one term from the tile row
// sum.  Output O and log2-LSE as in FastVideo PR #2048 ("Test Results").
//
// gfx950 mapping
//   1-D grid over (batch, head, 128-query block), ordered so that each XCD
//   (workgroup id mod 8) walks a contiguous range of heads: the K/V of a head
//   then streams through one XCD's L2 for all its query blocks.
//   256 threads = 4 waves; a workgroup owns 128 queries (one Q quantization
//   block, so s_Q is uniform), each wave 32.  Per 128-key tile j:
//     S^T = K_j Q^T on v_mfma_f32_32x32x64_f8f6f4 (A = 32 keys x 64 channels
//       from LDS, B = the wave's 32 queries, held in registers for the whole
//       loop).  A lane owns one query (lane % 32) and 16 keys per 32-key
//       sub-tile, so the tile max / row sum need one cross-half exchange.
//     P is formed in registers and packed to E4M3 straight into the B operand
//       of PV: the accumulator layout of two key sub-tiles is exactly one
//       64-token k-step of the PV MFMA, given that V is stored in the matching
//       token order (vs_quantize_residual).
//     O^T: acc = alpha acc (only when some row's max moved), then
//       acc += 2^e_j 2^-8 V_j^T P^T on v_mfma_scale_f32_32x32x64_f8f6f4 (A =
//       32 channels x 64 tokens): the power-of-two V block scale and P's 2^8
//       are E8M0 operand scales, so the product accumulates straight into acc;
//       then the rank-one restore acc += mu_j (x) l_j as
//       v_mfma_f32_32x32x1_2b_f32 outer products (one per pair of channel
//       tiles) instead of D FMAs per lane.
//   K and V tiles (16 KB each at D = 128) are double-buffered in LDS and
//   filled with global_load_lds_dwordx4 (no staging registers): each lane's
//   16-byte source is chosen so the LDS image is the XOR-swizzled tile, and
//   the 128-bit operand reads of 16 consecutive rows hit distinct banks
//   (gfx950's LDS serves a 128-bit read over 64 banks: rows of 128 B need the
//   chunk index XORed with (row >> 1) & 7).  The ragged last tile's mask sits
//   behind a uniform branch.
#include <float.h>

#include "common.h"

namespace vs {
namespace {

typedef float v32f __attribute__((ext_vector_type(32)));

constexpr float kExpcastK0 = 119.66015f;   // 120 - 4 (log2(1.5) - 1/2)

__device__ __forceinline__ v8i make_v8i(const uint4& a, const uint4& b) {
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Same product with E8M0 operand scales (byte b means 2^(b - 127)).
__device__ __forceinline__ v16f mfma_fp8_scaled(const v8i& a, const v8i& b, const v16f& c,
                                                int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

__device__ __forceinline__ uint4 lds_read16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte asynchronous global -> LDS copy; lane i of the wave writes
// dst + 16 i (dst is wave-uniform).
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// XOR swizzle of a row's 16-byte chunk index: rows of 8 chunks (128 B) use
// (row >> 1) & 7, rows of 4 chunks (64 B) use (row >> 1) & 3.
template <int ROWCHUNKS>
__device__ __forceinline__ int row_swz(int row) {
  return ROWCHUNKS == 8 ? ((row >> 1) & 7) : ((row >> 1) & 3);
}

// Source chunk, inside one 64-chunk (1 KB) DMA block `blk` of a tile, for the
// LDS chunk position `lane`: that position holds logical chunk
// (position ^ swizzle(row)) of its row.  Only the parity of the block index
// matters for 8-chunk rows (8 rows per block); none for 4-chunk rows.
template <int ROWCHUNKS>
__device__ __forceinline__ int dma_src_chunk(int lane, int blk) {
  if (ROWCHUNKS == 8) {
    const int row = 8 * blk + (lane >> 3);
    return (lane & ~7) | ((lane & 7) ^ row_swz<8>(row));
  }
  const int row = 16 * blk + (lane >> 2);
  return (lane & ~3) | ((lane & 3) ^ row_swz<4>(row));
}

template <int D, bool EXPCAST, int VMEAN>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ v8, const float* __restrict__ v_scale,
    const float* __restrict__ v_mean, const float* __restrict__ q_mu, int S, int H,
    int nb, int total, float c_log2, float* __restrict__ out, float* __restrict__ lse2) {
  constexpr int KD = D / 64;                 // k-steps of the QK product
  constexpr int DT = D / 32;                 // 32-channel tiles of O^T
  constexpr int TB = kBlock * D;             // bytes of one K (or V) tile
  constexpr int KRC = D / 16;                // 16-byte chunks per K row
  constexpr int NDMA = TB / 16 / 64 / 4;     // DMA instructions per wave, tile and tensor
  __shared__ __attribute__((aligned(1024))) uint8_t sk[2][TB];
  __shared__ __attribute__((aligned(1024))) uint8_t sv[2][TB];
  __shared__ __attribute__((aligned(16))) float smu[2][D];

  // ---- workgroup -> (b, h, query block), XCD-contiguous ----
  int qb, h, b;
  {
    const int L = blockIdx.x;
    const int xcd = L & 7, idx = L >> 3;
    const int per = total >> 3, rem = total & 7;
    const int logical = xcd < rem ? xcd * (per + 1) + idx
                                  : rem * (per + 1) + (xcd - rem) * per + idx;
    qb = logical % nb;
    const int bh_l = logical / nb;
    h = bh_l % H;
    b = bh_l / H;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const size_t S_pad = static_cast<size_t>(nb) * kBlock;

  // this lane's query and its B operand (32 bytes per k-step)
  const int qrow = qb * kBlock + wave * 32 + l32;
  v8i qa[KD];
  {
    const uint8_t* qp = q8 + (bh * S_pad + qrow) * D + 32 * hh;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      qa[kd] = make_v8i(*reinterpret_cast<const uint4*>(qp + 64 * kd),
                        *reinterpret_cast<const uint4*>(qp + 64 * kd + 16));
  }
  const float sq = q_scale[bh * nb + qb];

  const uint8_t* kbase = k8 + bh * S_pad * D;
  const uint8_t* vbase = v8 + bh * nb * static_cast<size_t>(TB);
  const float* mubase = (VMEAN == VS_VMEAN_BLOCK) ? v_mean + bh * nb * D : nullptr;
  const float* ksc = k_scale + bh * nb;
  const float* vsc = v_scale + bh * nb;

  // per-lane DMA source offsets (bytes inside a 1 KB block; even and odd
  // blocks) and operand read bases
  const int k_src[2] = {dma_src_chunk<KRC>(lane, 0) * 16, dma_src_chunk<KRC>(lane, 1) * 16};
  const int v_src[2] = {dma_src_chunk<8>(lane, 0) * 16, dma_src_chunk<8>(lane, 1) * 16};
  int k_rd[KD][2], v_rd[2][2];
#pragma unroll
  for (int kd = 0; kd < KD; ++kd)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      k_rd[kd][e] = l32 * D + (((4 * kd + 2 * hh + e) ^ row_swz<KRC>(l32)) << 4);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      v_rd[kk][e] = l32 * kBlock + (((4 * kk + 2 * hh + e) ^ row_swz<8>(l32)) << 4);

  float m = -INFINITY, l = 0.0f;
  v16f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

#define VS_ISSUE_TILE(J, BUF)                                                          \
  do {                                                                                 \
    const uint8_t* kg_ = kbase + static_cast<size_t>(J) * TB;                          \
    const uint8_t* vg_ = vbase + static_cast<size_t>(J) * TB;                          \
    _Pragma("unroll") for (int i_ = 0; i_ < NDMA; ++i_) {                              \
      const int base_ = (wave * NDMA + i_) * 1024;                                     \
      dma16(kg_ + base_ + k_src[i_ & 1], &sk[(BUF)][base_]);                           \
      dma16(vg_ + base_ + v_src[i_ & 1], &sv[(BUF)][base_]);                           \
    }                                                                                  \
    if (VMEAN == VS_VMEAN_BLOCK && wave == 0 && lane < D / 4)                          \
      dma16(mubase + static_cast<size_t>(J) * D + 4 * lane, &smu[(BUF)][0]);           \
  } while (0)

  VS_ISSUE_TILE(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int j = 0; j < nb; ++j) {
    const int buf = j & 1;
    const bool last = j == nb - 1;
    if (!last) VS_ISSUE_TILE(j + 1, buf ^ 1);
    const uint8_t* skb = sk[buf];
    const uint8_t* svb = sv[buf];

    // ---- S^T = K_j Q^T : 4 sub-tiles of 32 keys ----
    v16f s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint8_t* kr = skb + t * 32 * D;
      s[t] = mfma_fp8(make_v8i(lds_read16(kr + k_rd[0][0]), lds_read16(kr + k_rd[0][1])), qa[0],
                      v16f{});
#pragma unroll
      for (int kd = 1; kd < KD; ++kd)
        s[t] = mfma_fp8(make_v8i(lds_read16(kr + k_rd[kd][0]), lds_read16(kr + k_rd[kd][1])),
                        qa[kd], s[t]);
    }
    // keys past S (ragged last tile only): -inf drops them from the max and
    // gives p = 0 / code 0
    if (last && (S & (kBlock - 1))) {
      const int valid = S - j * kBlock;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * t + 8 * (r >> 2) + 4 * hh + (r & 3) >= valid) s[t][r] = -INFINITY;
    }

    // ---- running max, once per tile ----
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[t][r]);
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float cj = (sq * ksc[j]) * c_log2;
    const float m_new = __builtin_fmaxf(m, mx * cj);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);

    // ---- P tile -> E4M3 B operand; tile row sum ----
    v8i pb[2];
    float ell = 0.0f;
    if (!EXPCAST) {
      const float bias = 8.0f - m_new;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][4 * w + 0], cj, bias));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][4 * w + 1], cj, bias));
          const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][4 * w + 2], cj, bias));
          const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][4 * w + 3], cj, bias));
          ell += (p0 + p1) + (p2 + p3);
          uint32_t pk = cvt_pk_e4m3<false>(p0, p1, 0u);
          pk = cvt_pk_e4m3<true>(p2, p3, pk);
          pb[t >> 1][4 * (t & 1) + w] = static_cast<int>(pk);
        }
      }
    } else {
      const float c8 = 8.0f * cj;
      const float bias = kExpcastK0 - 8.0f * m_new;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t pk = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float code = __builtin_rintf(__builtin_fmaf(s[t][4 * w + e], c8, bias));
            code = code < 8.0f ? 0.0f : __builtin_fminf(code, 126.0f);
            pk |= static_cast<uint32_t>(code) << (8 * e);
          }
          ell += (__builtin_amdgcn_cvt_f32_fp8(static_cast<int>(pk), 0) +
                  __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(pk), 1)) +
                 (__builtin_amdgcn_cvt_f32_fp8(static_cast<int>(pk), 2) +
                  __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(pk), 3));
          pb[t >> 1][4 * (t & 1) + w] = static_cast<int>(pk);
        }
      }
    }
    ell += __shfl_xor(ell, 32, 64);
    ell *= (1.0f / 256.0f);
    l = alpha * l + ell;

    // ---- O^T = alpha O^T + 2^e_j 2^-8 (V^T P^T) + mu (x) l ----
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] *= alpha;
    }
    // E8M0 byte of the V block scale 2^e_j (a normal float: its exponent
    // field), and 2^-8 for P's prescale
    const int sv_e8 = (__float_as_int(vsc[j]) >> 23) & 0xFF;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const uint8_t* vr = svb + t * 32 * kBlock;
      acc[t] = mfma_fp8_scaled(make_v8i(lds_read16(vr + v_rd[0][0]), lds_read16(vr + v_rd[0][1])),
                               pb[0], acc[t], sv_e8, 127 - 8);
      acc[t] = mfma_fp8_scaled(make_v8i(lds_read16(vr + v_rd[1][0]), lds_read16(vr + v_rd[1][1])),
                               pb[1], acc[t], sv_e8, 127 - 8);
    }
    if (VMEAN == VS_VMEAN_BLOCK) {
#pragma unroll
      for (int pr = 0; pr < DT / 2; ++pr) {
        // lanes 0-31 carry mu of channel tile 2pr, lanes 32-63 of tile 2pr+1
        const float mu = smu[buf][64 * pr + lane];
        v32f c2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          c2[r] = acc[2 * pr][r];
          c2[16 + r] = acc[2 * pr + 1][r];
        }
        c2 = __builtin_amdgcn_mfma_f32_32x32x1f32(mu, ell, c2, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[2 * pr][r] = c2[r];
          acc[2 * pr + 1][r] = c2[16 + r];
        }
      }
    }
    m = m_new;

    if (!last) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }
#undef VS_ISSUE_TILE

  // ---- epilogue: O = acc / l (+ sequence mean), lse2 = m + log2 l + q_mu ----
  if (qrow < S) {
    const float inv_l = 1.0f / l;
    float* orow = out + ((static_cast<size_t>(b) * S + qrow) * H + h) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * t + 8 * a + 4 * hh;
        float4 o;
        o.x = acc[t][4 * a + 0] * inv_l;
        o.y = acc[t][4 * a + 1] * inv_l;
        o.z = acc[t][4 * a + 2] * inv_l;
        o.w = acc[t][4 * a + 3] * inv_l;
        if (VMEAN == VS_VMEAN_SEQ) {
          const float* mu = v_mean + bh * D + d0;
          o.x += mu[0]; o.y += mu[1]; o.z += mu[2]; o.w += mu[3];
        }
        *reinterpret_cast<float4*>(orow + d0) = o;
      }
    if (hh == 0)
      lse2[bh * S + qrow] = m + __builtin_amdgcn_logf(l) + (q_mu ? q_mu[bh * S + qrow] : 0.0f);
  }
}

template <int D, bool EXPCAST>
void launch_vm(int vmean_mode, int total, hipStream_t st, const uint8_t* q8, const float* qs,
               const uint8_t* k8, const float* ks, const uint8_t* v8, const float* vs,
               const float* vm, const float* qmu, int S, int H, int nb, float c, float* out,
               float* lse2) {
  const dim3 grid(total), block(256);
  if (vmean_mode == VS_VMEAN_BLOCK)
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_BLOCK>), grid, block, 0, st, q8, qs, k8,
                       ks, v8, vs, vm, qmu, S, H, nb, total, c, out, lse2);
  else if (vmean_mode == VS_VMEAN_SEQ)
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_SEQ>), grid, block, 0, st, q8, qs, k8,
                       ks, v8, vs, vm, qmu, S, H, nb, total, c, out, lse2);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_NONE>), grid, block, 0, st, q8, qs, k8,
                       ks, v8, vs, vm, qmu, S, H, nb, total, c, out, lse2);
}

}  // namespace
}  // namespace vs

extern "C" int vs_fp8_attn_fwd(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                               const float* k_scale, const uint8_t* v8, const float* v_scale,
                               const float* v_mean, int vmean_mode, const float* q_mu, int B,
                               int S, int H, int D, float softmax_scale, unsigned flags,
                               float* out, float* lse2, void* stream) {
  using namespace vs;
  if (B < 0 || S < 0 || H < 0) return VS_ERR_INVALID_ARG;
  if (vmean_mode != VS_VMEAN_NONE && vmean_mode != VS_VMEAN_BLOCK && vmean_mode != VS_VMEAN_SEQ)
    return VS_ERR_INVALID_ARG;
  if (flags & ~VS_EXPCAST) return VS_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || !(softmax_scale <= FLT_MAX)) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (B == 0 || S == 0 || H == 0) return VS_OK;
  if ((vmean_mode == VS_VMEAN_NONE) != (v_mean == nullptr)) return VS_ERR_INVALID_ARG;
  if (!q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale || !out || !lse2)
    return VS_ERR_INVALID_ARG;
  const void* ptrs[] = {q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, out, lse2};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VS_ERR_UNSUPPORTED;
  const int nb = n_blocks(S);
  const long long total = static_cast<long long>(B) * H * nb;
  if (total > 0x7FFFFFFFLL) return VS_ERR_UNSUPPORTED;

  const float c = softmax_scale * 1.44269504088896341f;
  hipStream_t st = as_stream(stream);
  const bool ec = (flags & VS_EXPCAST) != 0;
  const int tot = static_cast<int>(total);
  if (D == 128) {
    if (ec) launch_vm<128, true>(vmean_mode, tot, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, H, nb, c, out, lse2);
    else launch_vm<128, false>(vmean_mode, tot, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, H, nb, c, out, lse2);
  } else {
    if (ec) launch_vm<64, true>(vmean_mode, tot, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, H, nb, c, out, lse2);
    else launch_vm<64, false>(vmean_mode, tot, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, H, nb, c, out, lse2);
  }
  return launch_status();
}

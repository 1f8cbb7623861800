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
//   grid (ceil(S/128), H, B); 256 threads = 4 waves; one workgroup owns 128
//   queries (one Q quantization block, so s_Q is uniform), each wave 32.
//   Per 128-key tile j:
//     S^T = K_j Q^T on v_mfma_f32_32x32x64_f8f6f4 (A = 32 keys x 64 channels
//       from LDS, B = the wave's 32 queries held in registers), 4 key
//       sub-tiles x D/64 k-steps.  In the accumulator a lane holds one query
//       (lane % 32) and 16 keys per sub-tile, so the row max / row sum need
//       one exchange with the other half-wave only.
//     P is formed in registers and packed to E4M3 straight into the B operand
//       of the PV product: the accumulator layout of two key sub-tiles is
//       exactly the 64-token k-step the PV MFMA consumes, given that V is
//       stored with the matching token order (vs_quantize_residual).
//     O^T += V_j^T P^T on the same MFMA (A = 32 channels x 64 tokens, LDS).
//   K and V tiles (16 KB each at D = 128) are double-buffered in LDS through
//   registers; 16-byte chunks are XOR-swizzled by row so the 128-bit operand
//   reads of 8 consecutive rows hit distinct banks.  The block means of V for
//   the tile ride along in LDS.
#include <float.h>

#include "common.h"

namespace vs {
namespace {

constexpr float kExpcastK0 = 119.66015f;   // 120 - 4 (log2(1.5) - 1/2)

template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return D == 128 ? (row & 7) : ((row >> 1) & 3);
}
__device__ __forceinline__ int v_swz(int row) { return row & 7; }

__device__ __forceinline__ v8i make_v8i(const uint4& a, const uint4& b) {
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int D, bool EXPCAST, int VMEAN>
__global__ __launch_bounds__(256) void attn_fwd_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ v8, const float* __restrict__ v_scale,
    const float* __restrict__ v_mean, const float* __restrict__ q_mu, int S, int H,
    int nb, float c_log2, float* __restrict__ out, float* __restrict__ lse2) {
  constexpr int KD = D / 64;                 // k-steps of the QK product
  constexpr int DT = D / 32;                 // 32-channel tiles of O^T
  constexpr int TB = kBlock * D;             // bytes of one K (or V) tile
  constexpr int CPT = TB / 16 / 256;         // 16-byte chunks per thread per tile
  constexpr int KCH = D / 16;                // 16-byte chunks per K row
  __shared__ __attribute__((aligned(16))) uint8_t sk[2][TB];
  __shared__ __attribute__((aligned(16))) uint8_t sv[2][TB];
  __shared__ __attribute__((aligned(16))) float smu[2][D];

  const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const size_t S_pad = static_cast<size_t>(nb) * kBlock;

  // this lane's query and its B operand (32 bytes per k-step)
  const int qrow = qb * kBlock + wave * 32 + l32;
  v8i qa[KD];
  {
    const uint8_t* qp = q8 + (bh * S_pad + qrow) * D + 32 * hh;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const uint4 a = *reinterpret_cast<const uint4*>(qp + 64 * kd);
      const uint4 c = *reinterpret_cast<const uint4*>(qp + 64 * kd + 16);
      qa[kd] = make_v8i(a, c);
    }
  }
  const float sq = q_scale[bh * nb + qb];

  const uint8_t* kbase = k8 + bh * S_pad * D;
  const uint8_t* vbase = v8 + bh * nb * static_cast<size_t>(D) * kBlock;
  const float* mubase = (VMEAN == VS_VMEAN_BLOCK) ? v_mean + bh * nb * D : nullptr;

  uint4 kst[CPT], vst[CPT];
  float must = 0.0f;
  auto load_tile = [&](int j) {
    const uint4* kg = reinterpret_cast<const uint4*>(kbase + static_cast<size_t>(j) * TB);
    const uint4* vg = reinterpret_cast<const uint4*>(vbase + static_cast<size_t>(j) * TB);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      kst[i] = kg[tid + 256 * i];
      vst[i] = vg[tid + 256 * i];
    }
    if (VMEAN == VS_VMEAN_BLOCK && tid < D) must = mubase[static_cast<size_t>(j) * D + tid];
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int g = tid + 256 * i;
      const int kr = g / KCH, kc = g % KCH;
      *reinterpret_cast<uint4*>(&sk[buf][kr * D + ((kc ^ k_swz<D>(kr)) << 4)]) = kst[i];
      const int vr = g >> 3, vc = g & 7;
      *reinterpret_cast<uint4*>(&sv[buf][vr * kBlock + ((vc ^ v_swz(vr)) << 4)]) = vst[i];
    }
    if (VMEAN == VS_VMEAN_BLOCK && tid < D) smu[buf][tid] = must;
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  float m = -INFINITY, l = 0.0f;
  v16f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;

  for (int j = 0; j < nb; ++j) {
    const int buf = j & 1;
    if (j + 1 < nb) load_tile(j + 1);

    // ---- S^T = K_j Q^T : 4 sub-tiles of 32 keys ----
    v16f s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
      const int kr = 32 * t + l32;
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) {
        const int c0 = 4 * kd + 2 * hh;
        const uint4 a0 = *reinterpret_cast<const uint4*>(&sk[buf][kr * D + ((c0 ^ k_swz<D>(kr)) << 4)]);
        const uint4 a1 = *reinterpret_cast<const uint4*>(&sk[buf][kr * D + (((c0 + 1) ^ k_swz<D>(kr)) << 4)]);
        s[t] = mfma_fp8(make_v8i(a0, a1), qa[kd], s[t]);
      }
    }
    // keys past S (last tile only): -inf, so they drop out of the max and
    // give p = 0 / code 0
    if (j == nb - 1 && (S & (kBlock - 1))) {
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
    const float cj = (sq * k_scale[bh * nb + j]) * c_log2;
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

    // ---- O^T = alpha O^T + s_V (V^T P^T) + ell mu_j ----
    const float svj = v_scale[bh * nb + j] * (1.0f / 256.0f);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      v16f tmp;
#pragma unroll
      for (int r = 0; r < 16; ++r) tmp[r] = 0.0f;
      const int vr = 32 * t + l32;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c0 = 4 * kk + 2 * hh;
        const uint4 a0 = *reinterpret_cast<const uint4*>(&sv[buf][vr * kBlock + ((c0 ^ v_swz(vr)) << 4)]);
        const uint4 a1 = *reinterpret_cast<const uint4*>(&sv[buf][vr * kBlock + (((c0 + 1) ^ v_swz(vr)) << 4)]);
        tmp = mfma_fp8(make_v8i(a0, a1), pb[kk], tmp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float o = __builtin_fmaf(tmp[r], svj, acc[t][r] * alpha);
        if (VMEAN == VS_VMEAN_BLOCK)
          o = __builtin_fmaf(ell, smu[buf][32 * t + 8 * (r >> 2) + 4 * hh + (r & 3)], o);
        acc[t][r] = o;
      }
    }
    m = m_new;

    if (j + 1 < nb) {
      store_tile(buf ^ 1);
      __syncthreads();
    }
  }

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
void launch_vm(int vmean_mode, dim3 grid, hipStream_t st, const uint8_t* q8, const float* qs,
               const uint8_t* k8, const float* ks, const uint8_t* v8, const float* vs,
               const float* vm, const float* qmu, int S, int H, int nb, float c, float* out,
               float* lse2) {
  if (vmean_mode == VS_VMEAN_BLOCK)
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_BLOCK>), grid, dim3(256), 0, st, q8,
                       qs, k8, ks, v8, vs, vm, qmu, S, H, nb, c, out, lse2);
  else if (vmean_mode == VS_VMEAN_SEQ)
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_SEQ>), grid, dim3(256), 0, st, q8,
                       qs, k8, ks, v8, vs, vm, qmu, S, H, nb, c, out, lse2);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_NONE>), grid, dim3(256), 0, st, q8,
                       qs, k8, ks, v8, vs, vm, qmu, S, H, nb, c, out, lse2);
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
  if (B > 65535 || H > 65535) return VS_ERR_UNSUPPORTED;

  const int nb = n_blocks(S);
  const float c = softmax_scale * 1.44269504088896341f;
  const dim3 grid(nb, H, B);
  hipStream_t st = as_stream(stream);
  const bool ec = (flags & VS_EXPCAST) != 0;
  if (D == 128) {
    if (ec) launch_vm<128, true>(vmean_mode, grid, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, H, nb, c, out, lse2);
    else launch_vm<128, false>(vmean_mode, grid, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, H, nb, c, out, lse2);
  } else {
    if (ec) launch_vm<64, true>(vmean_mode, grid, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, H, nb, c, out, lse2);
    else launch_vm<64, false>(vmean_mode, grid, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, H, nb, c, out, lse2);
  }
  return launch_status();
}

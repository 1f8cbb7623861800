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
//   1-D grid over (batch, head, pair of 128-query blocks), ordered so that
//   each XCD (workgroup id mod 8) walks a contiguous range of heads: the K/V
//   of a head then streams through one XCD's L2 for all its query blocks.
//   512 threads = 8 waves in two groups of four; group g owns query block
//   2 pair + g (one Q quantization block, so s_Q is uniform), each wave 32
//   queries.  Waves w and w + 4 share a SIMD (round-robin placement), and the
//   groups run a ping-pong one phase apart, separated by workgroup barriers:
//   while one wave issues its matrix-core phase, the other wave on the SIMD
//   runs its vector phase.
//     M(j): S^T = K_j Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (A = 32 keys x
//       64 channels from LDS, B = the wave's 32 queries, held in registers
//       for the whole loop; a lane owns one query (lane % 32) and 16 keys per
//       32-key sub-tile; the power-of-two K and Q block scales are the E8M0
//       operand scales, and Q carries softmax_scale * log2 e, so the product
//       is the score in log2 units), then for tile j - 1: the row sum of its E4M3
//       probabilities (P codes as the B operand of two 16x16x128 products
//       against a 0/1 A operand that keeps a lane's two queries apart), O^T +=
//       2^e 2^-8 V^T P^T on v_mfma_scale_f32_32x32x64_f8f6f4 (the
//       power-of-two V block scale and P's 2^8 are E8M0 operand scales, so
//       the product accumulates straight into acc), and the rank-one restore
//       acc += mu (x) l as v_mfma_f32_32x32x1_2b_f32 outer products.
//     V(j): tile max (one cross-half exchange), integer running max, O^T
//       rescale by an exact power of two (only when some row's max moved),
//       and P = E4M3(2^s / 2^(m - 8)) -- exp2 of the score and the scaled
//       FP8 pack, whose power-of-two scale applies the offset -- packed straight into
//       the B operand of PV: the accumulator layout of two key sub-tiles is
//       exactly one 64-token k-step of the PV MFMA, given that V is stored in
//       the matching token order (vs_quantize_residual).
//   K and V tiles (16 KB each at D = 128) are double-buffered in LDS, shared
//   by all eight waves, and filled by the first group with buffer_load ...
//   lds (no staging registers, no per-lane address arithmetic): each lane's
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

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8i make_v8i(const uint4& a, const uint4& b) {
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

// 16x16x128 FP8 product without operand scales.
__device__ __forceinline__ v4f mfma_fp8_16(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// E8M0 byte of a power-of-two float scale (its biased exponent).
__device__ __forceinline__ int e8m0_of(float pow2) { return (__float_as_int(pow2) >> 23) & 0xFF; }

// Same product with E8M0 operand scales (byte b means 2^(b - 127)).
__device__ __forceinline__ v16f mfma_fp8_scaled(const v8i& a, const v8i& b, const v16f& c,
                                                int scale_a, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

__device__ __forceinline__ uint4 lds_read16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
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

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over `bytes` bytes at `base` (stride 0, gfx9 data format).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// 16-byte asynchronous buffer -> LDS copy: lane i reads base + soff + voff
// and writes dst + 16 i (dst and soff wave-uniform).
__device__ __forceinline__ void dma16(rsrc_t rs, int voff, int soff, void* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, 0);
}

// Uniform values and per-lane constants of one wave.
template <int D>
struct Ctx {
  rsrc_t krs, vrs, murs, scrs;           // K codes, V codes, V block means, V group scales
  const float* ksc;                      // K block scales of this head
  const float* vsc;                      // V block scales of this head
  int q_e8;                              // E8M0 byte of this query block's scale
  int nb, S, dma_wave, hh, lane;         // dma_wave: 0-3 in the DMA group, else -1
  int k_src[2], v_src[2];                // DMA source offsets (even / odd 1 KB block)
  int k_rd[D / 64][2], v_rd[2][2];       // swizzled operand read offsets
  int v4_rd[2];                          // MXFP4 V: read offset of k-step kk
  v8i qa[D / 64];                        // this lane's query, B operand of QK
  v8i ones;                              // E4M3 ones or zeros, A operand of the row sums
};

// Recurrence state of one wave: log2-domain scores s of the current key
// tile, its E4M3 probabilities pb, the integer running max m, the factor
// alpha of the last tile (applied to O^T already, to l when that tile's row
// sum is known), O^T and l.
template <int D>
struct State {
  v16f s[4];
  v8i pb[2];
  v16f acc[D / 32];
  float m, alpha, l;
  // block scales one tile ahead of their use (scalar loads complete while a
  // whole phase runs): K scale of the next M phase's QK tile, V scale of the
  // next M phase's PV tile
  float ks, vs;
};

// K of tile j into dst: 16 KB (D = 128) as 1 KB DMA blocks, a quarter per
// wave of the DMA group.
template <int D>
__device__ __forceinline__ void issue_k(const Ctx<D>& c, int j, uint8_t* dst) {
  constexpr int TB = kBlock * D, NDMA = TB / 16 / 64 / 4;
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int base = (c.dma_wave * NDMA + i) * 1024;
    dma16(c.krs, c.k_src[i & 1], j * TB + base, dst + base);
  }
}

// V of tile j (E4M3: 16 KB at D = 128; MXFP4: 8 KB of codes plus the
// D x 4 group scale bytes), and its block mean.
template <int D, int VMEAN, bool V4>
__device__ __forceinline__ void issue_v(const Ctx<D>& c, int j, uint8_t* dst, float* mu_dst,
                                        uint8_t* sc_dst) {
  constexpr int TB = kBlock * D / (V4 ? 2 : 1), NDMA = TB / 16 / 64 / 4;
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int base = (c.dma_wave * NDMA + i) * 1024;
    dma16(c.vrs, c.v_src[i & 1], j * TB + base, dst + base);
  }
  if (VMEAN == VS_VMEAN_BLOCK && c.dma_wave == 0 && c.lane < D / 4)
    dma16(c.murs, 16 * c.lane, j * D * 4, mu_dst);
  if (V4 && c.dma_wave == 1 && c.lane < D / 4)
    dma16(c.scrs, 16 * c.lane, j * D * 4, sc_dst);
}

// Keys at or past `valid` (ragged last tile) -> -inf: dropped from the max,
// probability 0 / code 0.  Written without compares: a key offset K of the
// lane is masked iff (valid - 4 hh - 1/2 - K) < 0, and min(s, that * inf) is
// -inf then and s otherwise (the factor is never 0).  Compare masks would
// each take a 64-bit scalar register pair.
__device__ __forceinline__ void mask_tile(v16f (&s)[4], int valid, int hh) {
  float lim = static_cast<float>(valid - 4 * hh) - 0.5f;
  // opaque to the optimizer: the bound is loop-invariant where this runs
  // once, and hoisting its 64 products would only occupy registers
  asm volatile("" : "+v"(lim));
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float key = static_cast<float>(32 * t + 8 * (r >> 2) + (r & 3));
      s[t][r] = __builtin_fminf(s[t][r], (lim - key) * INFINITY);
    }
}

// Max of x over lanes l and l ^ 32 without an LDS round trip:
// v_permlane32_swap of two copies of x leaves the other half's value of
// every lane in one of the two results (lanes 0-31 in the second, lanes
// 32-63 in the first), and x itself in the other.
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __builtin_fmaxf(x, __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

__device__ __forceinline__ float tile_max(const v16f (&s)[4]) {
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[t][r]);
  return max_with_other_half(mx);
}

// E4M3 probability codes of 4 scores of one lane (the dword w of sub-tile t
// of the B operand of PV), |m| <= 64: 2^s is finite and normal down to where
// its code is 0, and the pack divides it by 2^(m - 8) exactly before
// rounding to nearest even.
__device__ __forceinline__ int p_codes4_fast(const v16f& s, int w, float sc) {
  const float e0 = __builtin_amdgcn_exp2f(s[4 * w + 0]);
  const float e1 = __builtin_amdgcn_exp2f(s[4 * w + 1]);
  const float e2 = __builtin_amdgcn_exp2f(s[4 * w + 2]);
  const float e3 = __builtin_amdgcn_exp2f(s[4 * w + 3]);
  // the high half is written next, so the low write may keep any upper
  // bits: reuse e0's register instead of a zeroed one
  v2s o;
  __builtin_memcpy(&o, &e0, 4);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, e0, e1, sc, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, e2, e3, sc, true);
  int pk;
  __builtin_memcpy(&pk, &o, 4);
  return pk;
}

// The same codes for any m (exp2 of s + 8 - m, rounded to float32 first),
// or the ExpCast codes.
template <bool EXPCAST, bool CAP>
__device__ __forceinline__ int p_codes4(const v16f& s, int w, float bias) {
  if (!EXPCAST) {
    const float p0 = __builtin_amdgcn_exp2f(s[4 * w + 0] + bias);
    const float p1 = __builtin_amdgcn_exp2f(s[4 * w + 1] + bias);
    const float p2 = __builtin_amdgcn_exp2f(s[4 * w + 2] + bias);
    const float p3 = __builtin_amdgcn_exp2f(s[4 * w + 3] + bias);
    // the high half is written next, so the low write may keep any upper
    // bits: reuse p0's register instead of a zeroed one
    uint32_t pk = cvt_pk_e4m3<false>(p0, p1, __float_as_uint(p0));
    return static_cast<int>(cvt_pk_e4m3<true>(p2, p3, pk));
  }
  // ExpCast: code = rint(8 (s - m') + K0), capped at 126, codes below 8 -> 0.
  // v_cvt_pk_u8_f32 rounds half to even and saturates at 0 (so negative
  // pre-codes and -inf of masked keys give 0) while packing the byte.  The
  // cap only binds when |m'| is huge (CAP, a uniform slow path); otherwise
  // every byte is <= 121, so b + 0x78 carries into bit 7 exactly when b >= 8,
  // and the mask 0x80 - 0x01 = 0x7F keeps those bytes and clears the rest.
  uint32_t pk = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float x = __builtin_fmaf(s[4 * w + e], 8.0f, bias);
    if (CAP) x = __builtin_fminf(x, 126.0f);
    pk = __builtin_amdgcn_cvt_pk_u8_f32(x, e, pk);
  }
  const uint32_t m = (pk + 0x78787878u) & 0x80808080u;
  return static_cast<int>(pk & (m - (m >> 7)));
}

// Matrix-core phase M(j) of one wave: S^T of key tile j (if j < nb), then
// for tile j - 1 (if j >= 1) the row sums of its E4M3 probabilities, PV and
// the rank-one mean restore, and l's update.
//   kb: K of tile j      vb, mub: V and V mean of tile j - 1
template <int D, int VMEAN, bool V4>
__device__ __forceinline__ void phase_mfma(const int j, const Ctx<D>& c, State<D>& st,
                                           const uint8_t* kb, const uint8_t* vb,
                                           const float* mub, const uint8_t* scb) {
  constexpr int KD = D / 64, DT = D / 32;
  // the matrix-core phase issues first when both waves of the SIMD are ready
  __builtin_amdgcn_s_setprio(1);
  if (j < c.nb) {
    const int ks_e8 = e8m0_of(st.ks);
    // sub-tile major is fine here: the products of other waves fill the gap
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint8_t* kr = kb + t * 32 * D;
        const v8i a = make_v8i(lds_read16(kr + c.k_rd[kd][0]), lds_read16(kr + c.k_rd[kd][1]));
        st.s[t] = mfma_fp8_scaled(a, c.qa[kd], kd == 0 ? v16f{} : st.s[t], ks_e8, c.q_e8);
      }
  }
  if (j >= 1) {
    // row sums on the 16x16x128 product, half the cost of a 32x32x64 one.
    // Read as that shape, the P operand of one PV k-step holds in lane l
    // column l % 16 and the 32 k values of lane group l / 16; those lanes
    // carry query l % 32, i.e. column n pairs query n (groups 0 and 2)
    // with query n + 16 (groups 1 and 3).  A row m of ones over the groups
    // of parity (m / 4) % 2 only then sums one query, and the output row
    // of lane l (4 (l / 16) + r) has that parity of l / 16: every lane's
    // accumulator holds its own query's sum over the tile's 128 keys.
    v4f rs = mfma_fp8_16(c.ones, st.pb[0], v4f{});
    rs = mfma_fp8_16(c.ones, st.pb[1], rs);
    // O^T += 2^e 2^-8 V^T P^T: the E8M0 byte of the V block scale (a normal
    // power of two: its exponent field) and 2^-8 for P's prescale
    const int sv_e8 = (__float_as_int(st.vs) >> 23) & 0xFF;
    // V fragments read one product ahead (the fence keeps each read above
    // the product before it)
    auto vfrag = [&](int i) {
      const uint8_t* vr = vb + (i % DT) * 32 * kBlock;
      return make_v8i(lds_read16(vr + c.v_rd[i / DT][0]), lds_read16(vr + c.v_rd[i / DT][1]));
    };
    if (V4) {
      // MXFP4 V^T: lane (channel 32 dt + lane % 32, half hh) holds k-step
      // kk's tokens 64 kk + 32 hh .. + 31 in 16 bytes, and passes its own
      // E8M0 group scale (byte 2 kk + hh of its channel's scale word)
      uint32_t sw[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        sw[dt] = reinterpret_cast<const uint32_t*>(scb)[32 * dt + (c.lane & 31)] >> (8 * c.hh);
      auto vfrag4 = [&](int i) {
        const uint4 x = lds_read16(vb + (i % DT) * 32 * 64 + c.v4_rd[i / DT]);
        return v8i{static_cast<int>(x.x), static_cast<int>(x.y), static_cast<int>(x.z),
                   static_cast<int>(x.w), 0, 0, 0, 0};
      };
      v8i vf = vfrag4(0);
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        const v8i a = vf;
        if (i + 1 < 2 * DT) vf = vfrag4(i + 1);
        __builtin_amdgcn_sched_barrier(0);
        const int sa = static_cast<int>((sw[i % DT] >> (16 * (i / DT))) & 0xFF);
        st.acc[i % DT] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a, st.pb[i / DT], st.acc[i % DT], 4, 0, 0, sa, 0, 127 - 8);
      }
    } else {
      v8i vf = vfrag(0);
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        const v8i a = vf;
        if (i + 1 < 2 * DT) vf = vfrag(i + 1);
        __builtin_amdgcn_sched_barrier(0);
        st.acc[i % DT] = mfma_fp8_scaled(a, st.pb[i / DT], st.acc[i % DT], sv_e8, 127 - 8);
      }
    }
    const float ell = rs[0] * (1.0f / 256.0f);
    if (VMEAN == VS_VMEAN_BLOCK) {
      // + mu (x) l, one outer product per pair of channel tiles: lanes 0-31
      // carry mu of tile 2pr, lanes 32-63 of tile 2pr + 1
#pragma unroll
      for (int pr = 0; pr < DT / 2; ++pr) {
        const float mu = mub[64 * pr + c.lane];
        v32f c2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          c2[r] = st.acc[2 * pr][r];
          c2[16 + r] = st.acc[2 * pr + 1][r];
        }
        c2 = __builtin_amdgcn_mfma_f32_32x32x1f32(mu, ell, c2, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          st.acc[2 * pr][r] = c2[r];
          st.acc[2 * pr + 1][r] = c2[16 + r];
        }
      }
    }
    st.l = st.alpha * st.l + ell;
    // keep the products in this phase: left to itself the compiler may sink
    // them past the barrier, up to the vector phase's rescale, which then
    // reads their results a few instructions after issue (seen to give wrong
    // O without the mean restore, which otherwise pins them)
#pragma unroll
    for (int t = 0; t < DT; ++t) asm volatile("" : "+v"(st.acc[t]));
    // after the last LDS read of the phase, so no wait joins the two
    if (!V4) st.vs = c.vsc[j < c.nb ? j : c.nb - 1];
  }
  __builtin_amdgcn_s_setprio(0);
}

// Vector phase V(j) of one wave, j < nb: mask (ragged last tile), tile max,
// integer running max, O^T rescale, E4M3 probabilities of key tile j.
template <int D, bool EXPCAST>
__device__ __forceinline__ void phase_valu(const int j, const Ctx<D>& c, State<D>& st) {
  constexpr int DT = D / 32;
  if (j == c.nb - 1 && (c.S & (kBlock - 1))) mask_tile(st.s, c.S - j * kBlock, c.hh);
  const float m_new = __builtin_fmaxf(st.m, __builtin_ceilf(tile_max(st.s)));
  st.alpha = __builtin_amdgcn_exp2f(st.m - m_new);   // a power of two (0 on tile 0)
  if (__ballot(st.alpha != 1.0f)) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[t][r] *= st.alpha;
  }
  st.m = m_new;
  if (EXPCAST) {
    const float bias = kExpcastK0 - 8.0f * m_new;
    // ExpCast pre-codes stay below 126.5 unless rounding of 8 m is coarse
    // (|m| >= 2^20 log2 units): only then is the cap applied per element
    if (__ballot(__builtin_fabsf(m_new) >= 1048576.0f)) {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        st.pb[q >> 3][q & 7] = p_codes4<true, true>(st.s[q >> 2], q & 3, bias);
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        st.pb[q >> 3][q & 7] = p_codes4<true, false>(st.s[q >> 2], q & 3, bias);
    }
  } else if (!__ballot(__builtin_fabsf(m_new) > 64.0f)) {
    const float sc = __builtin_amdgcn_ldexpf(1.0f, static_cast<int>(m_new) - 8);
#pragma unroll
    for (int q = 0; q < 16; ++q) st.pb[q >> 3][q & 7] = p_codes4_fast(st.s[q >> 2], q & 3, sc);
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      st.pb[q >> 3][q & 7] = p_codes4<false, false>(st.s[q >> 2], q & 3, 8.0f - m_new);
  }
  st.ks = c.ksc[j + 1 < c.nb ? j + 1 : j];
}

// One trip of the ping-pong: M(j), barrier, V(j), barrier.  The two wave
// groups run it one phase apart, so on every SIMD one wave's matrix-core
// phase overlaps the other wave's vector phase.  The DMA group issues the
// copies of K tile j + 1 and V tile j at the start of its M(j) and waits for
// them before the barrier that ends its V(j); the buffers it overwrites were
// last read in the other group's M(j - 1), which ended at the barrier before.
//   kb: K_j (read)     kw: K_{j+1} (filled)
//   vb: V_{j-1} (read) vw: V_j (filled)
template <int D, bool EXPCAST, int VMEAN, bool V4>
__device__ __forceinline__ void pingpong_trip(const int j, const Ctx<D>& c, State<D>& st,
                                              const uint8_t* kb, uint8_t* kw,
                                              const uint8_t* vb, uint8_t* vw,
                                              const float* mub, float* muw,
                                              const uint8_t* scb, uint8_t* scw) {
  if (c.dma_wave >= 0 && j < c.nb) {
    if (j + 1 < c.nb) issue_k<D>(c, j + 1, kw);
    issue_v<D, VMEAN, V4>(c, j, vw, muw, scw);
  }
  phase_mfma<D, VMEAN, V4>(j, c, st, kb, vb, mub, scb);
  __syncthreads();
  if (j < c.nb) phase_valu<D, EXPCAST>(j, c, st);
  if (c.dma_wave >= 0) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

template <int D, bool EXPCAST, int VMEAN, bool V4>
__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ v8, const float* __restrict__ v_scale,
    const float* __restrict__ v_mean, const float* __restrict__ q_mu, int S, int H,
    int nb, int npairs, int total, void* __restrict__ out, int out_bf16,
    float* __restrict__ lse2) {
  constexpr int KD = D / 64;                 // k-steps of the QK product
  constexpr int DT = D / 32;                 // 32-channel tiles of O^T
  constexpr int TB = kBlock * D;             // bytes of one K (or V) tile
  constexpr int KRC = D / 16;                // 16-byte chunks per K row
  // separate variables per buffer: the compiler then knows a DMA into one
  // buffer does not alias reads of the other and does not wait for it
  __shared__ __attribute__((aligned(1024))) uint8_t sk0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t sk1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t sv0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t sv1[TB];
  __shared__ __attribute__((aligned(16))) float smu0[D];
  __shared__ __attribute__((aligned(16))) float smu1[D];
  // MXFP4 V: the tile's E8M0 group scales, 4 bytes per channel
  __shared__ __attribute__((aligned(16))) uint8_t ssc0[V4 ? D * 4 : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ssc1[V4 ? D * 4 : 16];

  // ---- workgroup -> (b, h, pair of query blocks), XCD-contiguous ----
  int qp, h, b;
  {
    const int L = blockIdx.x;
    const int xcd = L & 7, idx = L >> 3;
    const int per = total >> 3, rem = total & 7;
    const int logical = xcd < rem ? xcd * (per + 1) + idx
                                  : rem * (per + 1) + (xcd - rem) * per + idx;
    qp = logical % npairs;
    const int bh_l = logical / npairs;
    h = bh_l % H;
    b = bh_l / H;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;               // waves w and w + 4 share a SIMD
  const size_t bh = static_cast<size_t>(b) * H + h;
  const size_t S_pad = static_cast<size_t>(nb) * kBlock;
  // group g owns query block 2 qp + g; past the last block (odd nb) it runs
  // on a copy of the last block and writes nothing
  const int qb_raw = 2 * qp + group;
  const int qb = qb_raw < nb ? qb_raw : nb - 1;

  Ctx<D> c;
  c.dma_wave = group == 0 ? wave : -1;
  c.lane = lane;
  c.hh = hh;
  c.nb = nb;
  c.S = S;
  const int qrow = qb * kBlock + (wave & 3) * 32 + l32;
  {
    const uint8_t* qptr = q8 + (bh * S_pad + qrow) * D + 32 * hh;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      c.qa[kd] = make_v8i(*reinterpret_cast<const uint4*>(qptr + 64 * kd),
                          *reinterpret_cast<const uint4*>(qptr + 64 * kd + 16));
  }
  c.q_e8 = e8m0_of(q_scale[bh * nb + qb]);
  c.krs = make_rsrc(k8 + bh * S_pad * D, S_pad * D);
  c.vrs = V4 ? make_rsrc(v8 + bh * S_pad * D / 2, S_pad * D / 2)
             : make_rsrc(v8 + bh * S_pad * D, S_pad * D);
  c.scrs = make_rsrc(V4 ? reinterpret_cast<const uint8_t*>(v_scale) + bh * nb * D * 4
                        : reinterpret_cast<const uint8_t*>(v_scale),
                     V4 ? nb * D * 4 : 0);
  c.murs = make_rsrc(VMEAN == VS_VMEAN_BLOCK ? v_mean + bh * nb * D : v_mean,
                     VMEAN == VS_VMEAN_BLOCK ? nb * D * sizeof(float) : 0);
  c.ksc = k_scale + bh * nb;
  c.vsc = v_scale + bh * nb;
  c.k_src[0] = dma_src_chunk<KRC>(lane, 0) * 16;
  c.k_src[1] = dma_src_chunk<KRC>(lane, 1) * 16;
  c.v_src[0] = dma_src_chunk<V4 ? 4 : 8>(lane, 0) * 16;
  c.v_src[1] = dma_src_chunk<V4 ? 4 : 8>(lane, 1) * 16;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    c.v4_rd[kk] = l32 * 64 + (((2 * kk + hh) ^ row_swz<4>(l32)) << 4);
#pragma unroll
  for (int kd = 0; kd < KD; ++kd)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      c.k_rd[kd][e] = l32 * D + (((4 * kd + 2 * hh + e) ^ row_swz<KRC>(l32)) << 4);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      c.v_rd[kk][e] = l32 * kBlock + (((4 * kk + 2 * hh + e) ^ row_swz<8>(l32)) << 4);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    c.ones[i] = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1) ? 0x38383838 : 0;

  State<D> st;
  st.ks = c.ksc[0];
  st.vs = V4 ? 1.0f : c.vsc[0];
  st.m = -INFINITY;
  st.l = 0.0f;
  st.alpha = 1.0f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[t][r] = 0.0f;

  // ---- prologue: K of tile 0; group 1 runs one phase behind group 0 ----
  if (c.dma_wave >= 0) {
    issue_k<D>(c, 0, sk0);
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  if (group == 1) __syncthreads();

  // ---- nb + 1 trips, two per loop iteration (static buffer roles) ----
  for (int j = 0; j <= nb; j += 2) {
    pingpong_trip<D, EXPCAST, VMEAN, V4>(j, c, st, sk0, sk1, sv1, sv0, smu1, smu0, ssc1, ssc0);
    if (j + 1 <= nb)
      pingpong_trip<D, EXPCAST, VMEAN, V4>(j + 1, c, st, sk1, sk0, sv0, sv1, smu0, smu1, ssc0,
                                           ssc1);
  }
  if (group == 0) __syncthreads();

  // ---- epilogue: O = acc / l (+ sequence mean), lse2 = m + log2 l + q_mu ----
  if (qb_raw < nb && qrow < S) {
    const float inv_l = 1.0f / st.l;
    const size_t orow = ((static_cast<size_t>(b) * S + qrow) * H + h) * D;
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * t + 8 * a + 4 * hh;
        float4 o;
        o.x = st.acc[t][4 * a + 0] * inv_l;
        o.y = st.acc[t][4 * a + 1] * inv_l;
        o.z = st.acc[t][4 * a + 2] * inv_l;
        o.w = st.acc[t][4 * a + 3] * inv_l;
        if (VMEAN == VS_VMEAN_SEQ) {
          const float* mu = v_mean + bh * D + d0;
          o.x += mu[0]; o.y += mu[1]; o.z += mu[2]; o.w += mu[3];
        }
        if (out_bf16) {
          // the float32 result rounded to bf16 (nearest even), 8 bytes
          const v2bf lo = {static_cast<__bf16>(o.x), static_cast<__bf16>(o.y)};
          const v2bf hi = {static_cast<__bf16>(o.z), static_cast<__bf16>(o.w)};
          uint2 w;
          __builtin_memcpy(&w.x, &lo, 4);
          __builtin_memcpy(&w.y, &hi, 4);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + orow + d0) = w;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(out) + orow + d0) = o;
        }
      }
    if (hh == 0)
      lse2[bh * S + qrow] =
          st.m + __builtin_amdgcn_logf(st.l) + (q_mu ? q_mu[bh * S + qrow] : 0.0f);
  }
}

template <int D, bool EXPCAST, bool V4>
void launch_vm(int vmean_mode, int total, hipStream_t st, const uint8_t* q8, const float* qs,
               const uint8_t* k8, const float* ks, const uint8_t* v8, const float* vs,
               const float* vm, const float* qmu, int S, int H, int nb, int npairs,
               void* out, int out_bf16, float* lse2) {
  const dim3 grid(total), block(512);
  if (vmean_mode == VS_VMEAN_BLOCK)
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_BLOCK, V4>), grid, block, 0, st, q8,
                       qs, k8, ks, v8, vs, vm, qmu, S, H, nb, npairs, total, out, out_bf16, lse2);
  else if (vmean_mode == VS_VMEAN_SEQ)
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_SEQ, V4>), grid, block, 0, st, q8,
                       qs, k8, ks, v8, vs, vm, qmu, S, H, nb, npairs, total, out, out_bf16, lse2);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, EXPCAST, VS_VMEAN_NONE, V4>), grid, block, 0, st, q8,
                       qs, k8, ks, v8, vs, vm, qmu, S, H, nb, npairs, total, out, out_bf16, lse2);
}

}  // namespace
}  // namespace vs

extern "C" int vs_fp8_attn_fwd(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                               const float* k_scale, const uint8_t* v8, const float* v_scale,
                               const float* v_mean, int vmean_mode, const float* q_mu, int B,
                               int S, int H, int D, unsigned flags, void* out, float* lse2,
                               void* stream) {
  using namespace vs;
  if (B < 0 || S < 0 || H < 0) return VS_ERR_INVALID_ARG;
  if (vmean_mode != VS_VMEAN_NONE && vmean_mode != VS_VMEAN_BLOCK && vmean_mode != VS_VMEAN_SEQ)
    return VS_ERR_INVALID_ARG;
  if (flags & ~(VS_EXPCAST | VS_V_MXFP4 | VS_OUT_BF16)) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (B == 0 || S == 0 || H == 0) return VS_OK;
  if ((vmean_mode == VS_VMEAN_NONE) != (v_mean == nullptr)) return VS_ERR_INVALID_ARG;
  if (!q8 || !q_scale || !k8 || !k_scale || !v8 || !v_scale || !out || !lse2)
    return VS_ERR_INVALID_ARG;
  const void* ptrs[] = {q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, out, lse2};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VS_ERR_UNSUPPORTED;
  const int nb = n_blocks(S);
  // one workgroup per (batch, head, pair of 128-query blocks)
  const int npairs = (nb + 1) / 2;
  const long long total = static_cast<long long>(B) * H * npairs;
  if (total > 0x7FFFFFFFLL) return VS_ERR_UNSUPPORTED;
  // one head's codes are addressed through a 32-bit buffer range
  if (static_cast<long long>(nb) * kBlock * D > 0x7FFFFFFFLL) return VS_ERR_UNSUPPORTED;

  hipStream_t st = as_stream(stream);
  const bool ec = (flags & VS_EXPCAST) != 0, v4 = (flags & VS_V_MXFP4) != 0;
  const int tot = static_cast<int>(total);
  const int out_bf16 = (flags & VS_OUT_BF16) != 0;
#define VS_ATTN_ARGS vmean_mode, tot, st, q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, S, \
    H, nb, npairs, out, out_bf16, lse2
  switch ((D == 128 ? 4 : 0) | (ec ? 2 : 0) | (v4 ? 1 : 0)) {
    case 0: launch_vm<64, false, false>(VS_ATTN_ARGS); break;
    case 1: launch_vm<64, false, true>(VS_ATTN_ARGS); break;
    case 2: launch_vm<64, true, false>(VS_ATTN_ARGS); break;
    case 3: launch_vm<64, true, true>(VS_ATTN_ARGS); break;
    case 4: launch_vm<128, false, false>(VS_ATTN_ARGS); break;
    case 5: launch_vm<128, false, true>(VS_ATTN_ARGS); break;
    case 6: launch_vm<128, true, false>(VS_ATTN_ARGS); break;
    default: launch_vm<128, true, true>(VS_ATTN_ARGS); break;
  }
#undef VS_ATTN_ARGS
  return launch_status();
}

// vs_fp8_attn_fwd: FP8 (E4M3) attention forward with the in-recurrence V-mean
// restore and the optional ExpCast-FP8 probability cast.
//
// Method (VC-Attention summary, Key Contributions 1-2 and "Methodology in
// Plain English"; abstract): QK^T and PV run on the low-bit matrix cores,
// the online softmax between them keeps the running row maximum and the row
// sum of the probabilities, and each block's V mean is added back as a
// rank-one term from that tile row sum.  Output O and log2-LSE as in
// FastVideo PR #2048 ("Test Results").
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
//     M(j): S^T = K_j Q^T, A = 32 keys from LDS, B = the wave's 32 queries
//       held in registers for the whole loop (a lane owns one query, lane %
//       32, and 16 keys per 32-key sub-tile).  Two forms:
//         FP8: v_mfma_scale_f32_32x32x64_f8f6f4 on the E4M3 codes, the
//           power-of-two K and Q block scales as E8M0 operand scales;
//         bf16 (VS_BF16_MMA): v_mfma_f32_32x32x16_bf16 on the decoded codes
//           with the block scales folded in (the FP8 matrix core truncates
//           small products inside each group of 8 to about 13 bits below the
//           group's largest; the bf16 one keeps float32 accuracy at half
//           the rate).
//       Q carries softmax_scale * log2 e, so the product is the score in
//       log2 units, and the first product of each sub-tile takes as its
//       accumulator the per-row bias 8 - m (m the running max): the matrix
//       core returns x = s - m + 8 directly.  Then for tile j - 1:
//       O^T += 2^e 2^-8 V^T P^T on v_mfma_scale_f32_32x32x64_f8f6f4 (the
//       power-of-two V block scale and P's 2^8 are E8M0 operand scales) and
//       the rank-one restore acc += mu (x) l_tile as
//       v_mfma_f32_32x32x1_2b_f32 outer products.
//     V(j): tile max of x (one cross-half exchange); where some row's max
//       grew (a uniform branch), x, O^T and l are shifted by the growth and
//       the bias moves; then p8 = 2^x, the E4M3 codes E4M3(p8) packed
//       straight into the B operand of PV (the accumulator layout of two
//       key sub-tiles is one 64-token k-step of PV, given V stored in the
//       matching token order), and the tile row sum of the float32 p.
//   K and V tiles are double-buffered in LDS, shared by all eight waves, and
//   filled by the first group with buffer_load ... lds (no staging
//   registers, no per-lane address arithmetic): each lane's 16-byte source
//   is chosen so the LDS image is the XOR-swizzled tile, and the 128-bit
//   operand reads of 16 consecutive rows hit distinct banks (gfx950's LDS
//   serves a 128-bit read over 64 banks).  The ragged last tile's mask sits
//   behind a uniform branch.
#include <float.h>

#include "common.h"

namespace vs {
namespace {

typedef float v32f __attribute__((ext_vector_type(32)));

constexpr float kExpcastK0 = 119.66015f;   // 120 - 4 (log2(1.5) - 1/2)

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8i make_v8i(const uint4& a, const uint4& b) {
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

__device__ __forceinline__ v8bf as_v8bf(const uint4& x) {
  v8bf r;
  __builtin_memcpy(&r, &x, 16);
  return r;
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

// XOR swizzle of a row's 16-byte chunk index, so that 16 lanes reading one
// chunk column of 16 consecutive rows touch 64 distinct banks: rows of 16
// chunks (256 B) use row & 15, rows of 8 chunks (128 B) (row >> 1) & 7,
// rows of 4 chunks (64 B) (row >> 1) & 3.
template <int ROWCHUNKS>
__device__ __forceinline__ int row_swz(int row) {
  return ROWCHUNKS == 16 ? (row & 15) : ROWCHUNKS == 8 ? ((row >> 1) & 7) : ((row >> 1) & 3);
}

// Source chunk, inside one 64-chunk (1 KB) DMA block `blk` of a tile, for the
// LDS chunk position `lane`: that position holds logical chunk
// (position ^ swizzle(row)) of its row.  The block index matters modulo 4
// for 16-chunk rows (4 rows per block), modulo 2 for 8-chunk rows (8 rows
// per block), not at all for 4-chunk rows.
template <int ROWCHUNKS>
__device__ __forceinline__ int dma_src_chunk(int lane, int blk) {
  if (ROWCHUNKS == 16) {
    const int row = 4 * blk + (lane >> 4);
    return (lane & ~15) | ((lane & 15) ^ row_swz<16>(row));
  }
  if (ROWCHUNKS == 8) {
    const int row = 8 * blk + (lane >> 3);
    return (lane & ~7) | ((lane & 7) ^ row_swz<8>(row));
  }
  const int row = 16 * blk + (lane >> 2);
  return (lane & ~3) | ((lane & 3) ^ row_swz<4>(row));
}

// a[i] for a runtime i without indexing a private array (which would live
// in scratch memory): a chain of selects.
template <int N>
__device__ __forceinline__ int pick(const int (&a)[N], int i) {
  int r = a[0];
#pragma unroll
  for (int k = 1; k < N; ++k) r = i == k ? a[k] : r;
  return r;
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

// Probability casts (template parameter PC): E4M3 of 2^8 p, ExpCast-FP8,
// or the 4-bit tile (MXFP4: E2M1 codes, one E8M0 exponent per 32 keys).
constexpr int kPcE4m3 = 0, kPcExpcast = 1, kPcMxfp4 = 2;

// First K row of QK^T sub-tile t.  With the 4-bit probability tile, A-row i
// of sub-tile t loads key 64 (t / 2) + 16 (t % 2) + krow4(i), so that
// register r of lane half hh holds key 64 (t / 2) + 32 hh + 16 (t % 2) + r:
// each lane then owns 32 consecutive keys per PV k-step, one MX group.
template <bool P4>
constexpr int k_sub_row(int t) { return P4 ? 64 * (t >> 1) + 16 * (t & 1) : 32 * t; }

__device__ __forceinline__ int krow4(int i) { return 32 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// XOR swizzle of a K row with 8 chunks under the 4-bit tile's row mapping:
// the 16 lanes of one read then fetch rows {0-3, 4-7} + 32 {0, 1} (+ 16 or
// 64 per sub-tile), so bit 5 of the row also enters the swizzle to keep
// them on distinct banks.
__device__ __forceinline__ int row_swz8_p4(int row) { return ((row >> 1) & 7) ^ (((row >> 5) & 1) << 2); }

// Bytes of one K row in LDS and HBM: D codes, or D bf16 values.
template <int D, bool BF>
constexpr int k_row_bytes() { return BF ? 2 * D : D; }

// Uniform values and per-lane constants of one wave.
template <int D, bool BF>
struct Ctx {
  static constexpr int KRC = k_row_bytes<D, BF>() / 16;   // 16-byte chunks per K row
  static constexpr int NKS = BF ? D / 16 : D / 64;        // k-steps of the QK product
  rsrc_t krs, vrs, murs, scrs;           // K codes, V codes, V block means, V group scales
  const float* ksc;                      // K block scales of this head
  const float* vsc;                      // V block scales of this head
  int q_e8;                              // E8M0 byte of this query block's scale
  int nb, S, dma_wave, hh, lane;         // dma_wave: 0-3 in the DMA group, else -1
  int k_src[KRC == 16 ? 4 : 2];          // K DMA source offsets (1 KB block mod 4 or 2)
  int v_src[BF ? 4 : 2];                 // V DMA source offsets
  int k_rd[NKS][BF ? 1 : 2];             // swizzled K operand read offsets
  int v_rd[BF ? 8 : 2][BF ? 1 : 2];      // swizzled V operand read offsets
  int v4_rd[2];                          // MXFP4 V: read offset of k-step kk
  v8i qa[BF ? 1 : D / 64];             // this lane's query codes, B operand of QK (FP8)
  v8bf qb[BF ? D / 16 : 1];            // this lane's query as bf16, B operand (bf16)
};

// Recurrence state of one wave: x = s - m + 8 of the current key tile (s
// the log2-domain score, m the running row max), its E4M3 probabilities pb
// (as the bf16 values pbf for the bf16 PV), O^T, the bias 8 - m as the first
// QK product's accumulator, l (the row sum of p8 = 2^8 p = 2^x) and the
// last tile's row sum for its mean restore.  O^T, l and the row sums are in
// units of 2^8 p: O = acc / l is unchanged and lse2 = m + log2(l) - 8.
template <int D, bool BF>
struct State {
  v16f s[4];
  v8i pb[BF ? 1 : 2];
  int ps4[2];          // 4-bit tile: E8M0 byte of the lane's group per k-step
  v8bf pbf[BF ? 8 : 1];
  v16f acc[D / 32];
  v16f bias;
  float b, l, ell;
  // block scales one tile ahead of their use (scalar loads complete while a
  // whole phase runs): K scale of the next M phase's QK tile, V scale of the
  // next M phase's PV tile
  float ks, vs;
};

// K of tile j into dst (16 KB of codes at D = 128, 32 KB as bf16) as 1 KB
// DMA blocks, a quarter per wave of the DMA group.
template <int D, bool BF>
__device__ __forceinline__ void issue_k(const Ctx<D, BF>& c, int j, uint8_t* dst) {
  constexpr int TB = kBlock * k_row_bytes<D, BF>(), NDMA = TB / 16 / 64 / 4;
  constexpr int NSRC = Ctx<D, BF>::KRC == 16 ? 4 : 2;
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int blk = c.dma_wave * NDMA + i;
    dma16(c.krs, pick(c.k_src, blk % NSRC), j * TB + blk * 1024, dst + blk * 1024);
  }
}

// Bytes of one V tile: D channel rows of 128 tokens, as E4M3 codes, MXFP4
// nibbles or bf16 values.
template <int D, bool BF, bool V4>
constexpr int v_tile_bytes() { return BF ? kBlock * D * 2 : V4 ? kBlock * D / 2 : kBlock * D; }

// V of tile j (E4M3: 16 KB at D = 128; MXFP4: 8 KB of codes plus the
// D x 4 group scale bytes; bf16: 32 KB), and its block mean.
template <int D, bool BF, int VMEAN, bool V4>
__device__ __forceinline__ void issue_v(const Ctx<D, BF>& c, int j, uint8_t* dst, float* mu_dst,
                                        uint8_t* sc_dst) {
  constexpr int TB = v_tile_bytes<D, BF, V4>(), NDMA = TB / 16 / 64 / 4;
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int blk = c.dma_wave * NDMA + i;
    dma16(c.vrs, pick(c.v_src, blk % (BF ? 4 : 2)), j * TB + blk * 1024, dst + blk * 1024);
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
template <bool P4>
__device__ __forceinline__ void mask_tile(v16f (&s)[4], int valid, int hh) {
  float lim = static_cast<float>(valid - (P4 ? 32 : 4) * hh) - 0.5f;
  // opaque to the optimizer: the bound is loop-invariant where this runs
  // once, and hoisting its 64 products would only occupy registers
  asm volatile("" : "+v"(lim));
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float key = static_cast<float>(P4 ? k_sub_row<true>(t) + r
                                              : 32 * t + 8 * (r >> 2) + (r & 3));
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

// The same tile max for the 4-bit probability tile, taken as the maxima gm
// of the lane's two MX groups (sub-tiles 2 kk and 2 kk + 1 hold group kk's
// 32 keys): the chain costs the same, and the groups' largest probabilities
// are then 2^gm, with no second pass over the 64 values.
__device__ __forceinline__ float tile_max_groups(const v16f (&s)[4], float (&gm)[2]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[2 * kk + u][r]);
    gm[kk] = mx;
  }
  return max_with_other_half(__builtin_fmaxf(gm[0], gm[1]));
}

// E4M3 probability codes of 4 elements of one lane (the dword w of sub-tile
// t of the B operand of PV): p8 = 2^x (x <= 8 up to rounding, so p8 <= 256
// needs no clamp), rounded to nearest even by the FP8 conversion; the
// float32 p8 are added to the lane's row-sum part.
__device__ __forceinline__ int p_codes4(const v16f& x, int w, float& ls) {
  const float e0 = __builtin_amdgcn_exp2f(x[4 * w + 0]);
  const float e1 = __builtin_amdgcn_exp2f(x[4 * w + 1]);
  const float e2 = __builtin_amdgcn_exp2f(x[4 * w + 2]);
  const float e3 = __builtin_amdgcn_exp2f(x[4 * w + 3]);
  ls += (e0 + e1) + (e2 + e3);
  // the high half is written next, so the low write may keep any upper
  // bits: reuse e0's register instead of a zeroed one
  uint32_t pk = cvt_pk_e4m3<false>(e0, e1, __float_as_uint(e0));
  return static_cast<int>(cvt_pk_e4m3<true>(e2, e3, pk));
}

// ExpCast codes of the same 4 elements: code = rint(8 (s - m) + K0) =
// rint(8 x + K0 - 64), one FMA each; v_cvt_pk_u8_f32 rounds half to even and
// saturates at 0 (so negative pre-codes and the -inf of masked keys give 0)
// while packing the byte; x <= 8 keeps every code <= 120, so no cap binds.
// Codes below 8 become 0: every byte is <= 120, so b + 0x78 carries into bit
// 7 exactly when b >= 8, and the mask 0x80 - 0x01 = 0x7F keeps those bytes.
// The decoded codes (hardware E4M3 -> f32, exact) are added to the lane's
// row-sum part.
__device__ __forceinline__ int expcast_codes4(const v16f& x, int w, float& ls) {
  uint32_t pk = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    pk = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(x[4 * w + e], 8.0f, kExpcastK0 - 64.0f), e,
                                        pk);
  const uint32_t m = (pk + 0x78787878u) & 0x80808080u;
  pk &= m - (m >> 7);
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(pk), false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(pk), true);
  ls += (lo[0] + lo[1]) + (hi[0] + hi[1]);
  return static_cast<int>(pk);
}

// The 4-bit probability tile of one lane: p8 = 2^x (float32, added to the
// row-sum part), then per PV k-step kk the lane's 32 keys 64 kk + 32 hh ..
// + 31 (registers r of sub-tiles 2 kk and 2 kk + 1 under the 4-bit row
// mapping) form one MX group: e = the smallest exponent >= -127 with
// max p8 <= 6 2^e -- from the float's bits: e = E - 2, plus 1 where the
// mantissa exceeds 1.5; max p8 = 2^gm[kk], gm the group's largest x from
// the tile max (2^x is monotone, so that is the largest of the p8) -- and
// the codes are E2M1(p8 2^-e), nearest with
// ties to the even code (the conversion divides by the power of two of the
// scale operand's exponent field; a zero field acts as 2^-127).  A 4-bit
// operand's lane half hh holds k positions 16 hh + (0..15) in nibbles 0-15
// and 32 + 16 hh + (0..15) in nibbles 16-31; V stores the token at
// position p with bits 4 and 5 of p swapped, so nibble n carries key
// 64 kk + 32 hh + n: register n % 16 of sub-tile 2 kk + n / 16.
template <int D, bool BF>
__device__ __forceinline__ void p_tile_mxfp4(State<D, BF>& st, float& ls, const float (&gm)[2]) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      st.s[t][r] = __builtin_amdgcn_exp2f(st.s[t][r]);
      ls += st.s[t][r];
    }
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const float mx = __builtin_amdgcn_exp2f(gm[kk]);
    const uint32_t bits = __float_as_uint(mx);
    int e = static_cast<int>(bits >> 23) - 129 + ((bits & 0x7FFFFFu) > 0x400000u ? 1 : 0);
    e = mx > 0.0f ? (e < -127 ? -127 : e) : 0;
    const float scale = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
    st.ps4[kk] = e + 127;
    // byte k holds nibbles n = 2 k, 2 k + 1: registers r, r + 1 of sub-tile
    // 2 kk + u, u = n / 16, r = n % 16 (the byte-select operand must be a
    // constant)
    auto src = [&](int k, int odd) -> float {
      const int n = 2 * k;
      return st.s[2 * kk + (n >> 4)][(n & 15) + odd];
    };
    uint32_t w[4];
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      uint32_t acc = 0u;
      acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, src(4 * dw, 0), src(4 * dw, 1), scale, 0);
      acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, src(4 * dw + 1, 0), src(4 * dw + 1, 1),
                                                     scale, 1);
      acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, src(4 * dw + 2, 0), src(4 * dw + 2, 1),
                                                     scale, 2);
      acc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, src(4 * dw + 3, 0), src(4 * dw + 3, 1),
                                                     scale, 3);
      w[dw] = acc;
    }
    st.pb[kk] = v8i{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]),
                    static_cast<int>(w[3]), 0, 0, 0, 0};
  }
}

// Matrix-core phase M(j) of one wave: S^T of key tile j (if j < nb), then
// for tile j - 1 (if j >= 1) PV and the rank-one mean restore.
//   kb: K of tile j      vb, mub: V and V mean of tile j - 1
template <int D, bool BF, int VMEAN, bool V4, int PC>
__device__ __forceinline__ void phase_mfma(const int j, const Ctx<D, BF>& c, State<D, BF>& st,
                                           const uint8_t* kb, const uint8_t* vb,
                                           const float* mub, const uint8_t* scb) {
  constexpr int DT = D / 32, NKS = Ctx<D, BF>::NKS, KRB = k_row_bytes<D, BF>();
  // the matrix-core phase issues first when both waves of the SIMD are ready
  __builtin_amdgcn_s_setprio(1);
  if (j < c.nb) {
    if constexpr (BF) {
      // k-step major: four independent accumulators in flight
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const v8bf a = as_v8bf(lds_read16(kb + t * 32 * KRB + c.k_rd[ks][0]));
          st.s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, c.qb[ks], ks == 0 ? st.bias : st.s[t],
                                                            0, 0, 0);
        }
    } else {
      const int ks_e8 = e8m0_of(st.ks);
#pragma unroll
      for (int kd = 0; kd < NKS; ++kd)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint8_t* kr = kb + k_sub_row<PC == kPcMxfp4>(t) * KRB;
          const v8i a = make_v8i(lds_read16(kr + c.k_rd[kd][0]), lds_read16(kr + c.k_rd[kd][BF ? 0 : 1]));
          st.s[t] = mfma_fp8_scaled(a, c.qa[kd], kd == 0 ? st.bias : st.s[t], ks_e8, c.q_e8);
        }
    }
  }
  if (j >= 1) {
    if constexpr (BF) {
      // O^T += V^T P^T on v_mfma_f32_32x32x16_bf16: A = 32 channels x 16
      // tokens of the bf16 V tile (its block scale folded into the values),
      // B = the 16 tokens' probabilities of the wave's 32 queries (k-step ks
      // holds sub-tile ks / 2's elements 8 (ks % 2) .. + 7 of every lane,
      // the token order the quantizer wrote V in); channel tiles innermost,
      // so DT accumulators are in flight
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const v8bf a = as_v8bf(lds_read16(vb + dt * 32 * 256 + c.v_rd[ks][0]));
          st.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, st.pbf[ks], st.acc[dt], 0, 0, 0);
        }
    } else {
    // O^T += 2^e V^T P^T: the E8M0 byte of the V block scale (a normal
    // power of two: its exponent field); P is in units of 2^8 p
    const int sv_e8 = (__float_as_int(st.vs) >> 23) & 0xFF;
    // V fragments read one product ahead (the fence keeps each read above
    // the product before it)
    auto vfrag = [&](int i) {
      const uint8_t* vr = vb + (i % DT) * 32 * kBlock;
      return make_v8i(lds_read16(vr + c.v_rd[i / DT][0]), lds_read16(vr + c.v_rd[i / DT][BF ? 0 : 1]));
    };
    if constexpr (V4) {
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
            a, st.pb[i / DT], st.acc[i % DT], 4, 0, 0, sa, 0, 127);
      }
    } else if constexpr (PC == kPcMxfp4) {
      // B = the 4-bit probability tile: lane (query, half hh) passes the 32
      // keys 64 kk + 32 hh .. + 31 as E2M1 nibbles with their E8M0 exponent
      v8i vf = vfrag(0);
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        const v8i a = vf;
        if (i + 1 < 2 * DT) vf = vfrag(i + 1);
        __builtin_amdgcn_sched_barrier(0);
        st.acc[i % DT] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a, st.pb[i / DT], st.acc[i % DT], 0, 4, 0, sv_e8, 0, st.ps4[i / DT]);
      }
    } else {
      v8i vf = vfrag(0);
#pragma unroll
      for (int i = 0; i < 2 * DT; ++i) {
        const v8i a = vf;
        if (i + 1 < 2 * DT) vf = vfrag(i + 1);
        __builtin_amdgcn_sched_barrier(0);
        st.acc[i % DT] = mfma_fp8_scaled(a, st.pb[i / DT], st.acc[i % DT], sv_e8, 127);
      }
    }
    }
    if (VMEAN == VS_VMEAN_BLOCK) {
      // + mu (x) l_tile, one outer product per pair of channel tiles: lanes
      // 0-31 carry mu of tile 2pr, lanes 32-63 of tile 2pr + 1, and every
      // lane the row sum of its own query
#pragma unroll
      for (int pr = 0; pr < DT / 2; ++pr) {
        const float mu = mub[64 * pr + c.lane];
        v32f c2;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          c2[r] = st.acc[2 * pr][r];
          c2[16 + r] = st.acc[2 * pr + 1][r];
        }
        c2 = __builtin_amdgcn_mfma_f32_32x32x1f32(mu, st.ell, c2, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          st.acc[2 * pr][r] = c2[r];
          st.acc[2 * pr + 1][r] = c2[16 + r];
        }
      }
    }
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
// the running max's update where it grew, E4M3 (or ExpCast) probabilities of
// key tile j, the tile row sum and l.  With dbg, the lane's codes are
// written to its row of the diagnostic code buffer.
template <int D, bool BF, int PC>
__device__ __forceinline__ void phase_valu(const int j, const Ctx<D, BF>& c, State<D, BF>& st,
                                           uint8_t* dbg) {
  constexpr bool EXPCAST = PC == kPcExpcast;
  constexpr int DT = D / 32;
  if (j == c.nb - 1 && (c.S & (kBlock - 1)))
    mask_tile<PC == kPcMxfp4>(st.s, c.S - j * kBlock, c.hh);
  float gm[2];                      // 4-bit tile: the lane's MX group maxima of x
  const float xm = PC == kPcMxfp4 ? tile_max_groups(st.s, gm)
                                  : tile_max(st.s);   // max of s - m + 8 over the row's 128 keys
  // Tile 0 sets the reference (the bias was 0, so x = s); later tiles move
  // it where the row max grew.  tau = b - b' is the shift actually applied,
  // so x, O^T and l stay consistent with the new bias b'.
  const bool first = j == 0;
  if (first || __ballot(xm > 8.0f)) {
    const float d = (first || xm > 8.0f) ? xm - 8.0f : 0.0f;
    const float b_new = st.b - d;
    const float tau = st.b - b_new;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.s[t][r] -= tau;
    if constexpr (PC == kPcMxfp4) {
      // the same rounded subtraction of each group's largest x: still its max
      gm[0] -= tau;
      gm[1] -= tau;
    }
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(-tau);
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.acc[t][r] *= alpha;
      st.l *= alpha;
    }
    st.b = b_new;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.bias[r] = b_new;
  }
  float ls = 0.0f;
  int pk[16];
  if constexpr (PC == kPcMxfp4) {
    p_tile_mxfp4(st, ls, gm);
  } else {
#pragma unroll
  for (int q = 0; q < 16; ++q)
    pk[q] = EXPCAST ? expcast_codes4(st.s[q >> 2], q & 3, ls) : p_codes4(st.s[q >> 2], q & 3, ls);
  }
  if constexpr (PC == kPcMxfp4) {
  } else if constexpr (BF) {
    // the codes' values as bf16 (exact), B operand of the bf16 PV: k-step
    // ks takes dwords 2 ks and 2 ks + 1
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pk[2 * ks], 1.0f, false);
      const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pk[2 * ks], 1.0f, true);
      const v2bf c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pk[2 * ks + 1], 1.0f, false);
      const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pk[2 * ks + 1], 1.0f, true);
      st.pbf[ks] = v8bf{a[0], a[1], b[0], b[1], c2[0], c2[1], d[0], d[1]};
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) st.pb[q >> 3][q & 7] = pk[q];
  }
  // the other 64 keys of the row are in lane ^ 32
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ls), __float_as_uint(ls),
                                                    false, false);
    ls = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  st.ell = ls;
  st.l += ls;
  if (PC != kPcMxfp4 && dbg) {
    // dword q holds keys 32 (q / 4) + 8 (q % 4) + 4 hh .. + 3 of the tile
#pragma unroll
    for (int q = 0; q < 16; ++q)
      *reinterpret_cast<int*>(dbg + j * kBlock + 32 * (q >> 2) + 8 * (q & 3) + 4 * c.hh) = pk[q];
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
template <int D, bool BF, int PC, int VMEAN, bool V4, bool DBG>
__device__ __forceinline__ void pingpong_trip(const int j, const Ctx<D, BF>& c, State<D, BF>& st,
                                              const uint8_t* kb, uint8_t* kw,
                                              const uint8_t* vb, uint8_t* vw,
                                              const float* mub, float* muw,
                                              const uint8_t* scb, uint8_t* scw, uint8_t* dbg) {
  if (c.dma_wave >= 0 && j < c.nb) {
    if (j + 1 < c.nb) issue_k<D, BF>(c, j + 1, kw);
    issue_v<D, BF, VMEAN, V4>(c, j, vw, muw, scw);
  }
  phase_mfma<D, BF, VMEAN, V4, PC>(j, c, st, kb, vb, mub, scb);
  __syncthreads();
  if (j < c.nb) phase_valu<D, BF, PC>(j, c, st, DBG ? dbg : nullptr);
  if (c.dma_wave >= 0) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

template <int D, bool BF, int PC, int VMEAN, bool V4, bool DBG>
__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ v8, const float* __restrict__ v_scale,
    const float* __restrict__ v_mean, const float* __restrict__ q_mu, int S, int H,
    int nb, int npairs, int total, void* __restrict__ out, int out_bf16,
    float* __restrict__ lse2, uint8_t* __restrict__ dbg_codes, int dbg_stride) {
  constexpr int DT = D / 32;                 // 32-channel tiles of O^T
  constexpr int KRB = k_row_bytes<D, BF>();
  constexpr int KTB = kBlock * KRB;          // bytes of one K tile
  constexpr int VTB = v_tile_bytes<D, BF, V4>();   // bytes of one V tile
  constexpr int KRC = KRB / 16;              // 16-byte chunks per K row
  constexpr int NKS = Ctx<D, BF>::NKS;
  // separate variables per buffer: the compiler then knows a DMA into one
  // buffer does not alias reads of the other and does not wait for it
  __shared__ __attribute__((aligned(1024))) uint8_t sk0[KTB];
  __shared__ __attribute__((aligned(1024))) uint8_t sk1[KTB];
  __shared__ __attribute__((aligned(1024))) uint8_t sv0[BF ? VTB : kBlock * D];
  __shared__ __attribute__((aligned(1024))) uint8_t sv1[BF ? VTB : kBlock * D];
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

  Ctx<D, BF> c;
  c.dma_wave = group == 0 ? wave : -1;
  c.lane = lane;
  c.hh = hh;
  c.nb = nb;
  c.S = S;
  const int qrow = qb * kBlock + (wave & 3) * 32 + l32;
  if constexpr (BF) {
    // bf16 Q: k-step ks holds channels 16 ks + 8 hh .. + 7
    const uint16_t* qptr = reinterpret_cast<const uint16_t*>(q8) + (bh * S_pad + qrow) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      c.qb[ks] = as_v8bf(*reinterpret_cast<const uint4*>(qptr + 16 * ks));
  } else {
    const uint8_t* qptr = q8 + (bh * S_pad + qrow) * D + 32 * hh;
#pragma unroll
    for (int kd = 0; kd < NKS; ++kd)
      c.qa[kd] = make_v8i(*reinterpret_cast<const uint4*>(qptr + 64 * kd),
                          *reinterpret_cast<const uint4*>(qptr + 64 * kd + 16));
    c.q_e8 = e8m0_of(q_scale[bh * nb + qb]);
  }
  c.krs = make_rsrc(k8 + bh * S_pad * KRB, S_pad * KRB);
  c.vrs = make_rsrc(v8 + bh * nb * VTB, static_cast<size_t>(nb) * VTB);
  c.scrs = make_rsrc(V4 ? reinterpret_cast<const uint8_t*>(v_scale) + bh * nb * D * 4
                        : reinterpret_cast<const uint8_t*>(v_scale),
                     V4 ? nb * D * 4 : 0);
  c.murs = make_rsrc(VMEAN == VS_VMEAN_BLOCK ? v_mean + bh * nb * D : v_mean,
                     VMEAN == VS_VMEAN_BLOCK ? nb * D * sizeof(float) : 0);
  c.ksc = k_scale + bh * nb;
  c.vsc = v_scale + bh * nb;
#pragma unroll
  for (int i = 0; i < (KRC == 16 ? 4 : 2); ++i) c.k_src[i] = dma_src_chunk<KRC>(lane, i) * 16;
  if constexpr (PC == kPcMxfp4 && KRC == 8) {
    // bit 5 of a row is bit 2 of its 1 KB block, i.e. the DMA wave's bit 0
    // (four blocks per wave): that wave's sources flip chunk bit 2
    if (c.dma_wave >= 0 && (c.dma_wave & 1)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) c.k_src[i] ^= 64;
    }
  }
#pragma unroll
  for (int i = 0; i < (BF ? 4 : 2); ++i)
    c.v_src[i] = dma_src_chunk<BF ? 16 : V4 ? 4 : 8>(lane, i) * 16;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
    c.v4_rd[kk] = l32 * 64 + (((2 * kk + hh) ^ row_swz<4>(l32)) << 4);
  if constexpr (BF) {
    // A operand of k-step ks: key l32, channels 16 ks + 8 hh .. + 7 (chunk 2 ks + hh)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      c.k_rd[ks][0] = l32 * KRB + (((2 * ks + hh) ^ row_swz<KRC>(l32)) << 4);
  } else {
    // A-row l32 of a sub-tile: key row l32, or krow4(l32) with the 4-bit tile
    const int krow = PC == kPcMxfp4 ? krow4(l32) : l32;
    const int ksw = PC == kPcMxfp4 && KRC == 8 ? row_swz8_p4(krow) : row_swz<KRC>(krow);
#pragma unroll
    for (int kd = 0; kd < NKS; ++kd)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        c.k_rd[kd][BF ? 0 : e] = krow * KRB + (((4 * kd + 2 * hh + e) ^ ksw) << 4);
  }
  if constexpr (BF) {
    // bf16 V rows of 256 bytes: k-step ks of lane half hh is chunk 2 ks + hh
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      c.v_rd[ks][0] = l32 * 256 + (((2 * ks + hh) ^ row_swz<16>(l32)) << 4);
  } else {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        c.v_rd[kk][BF ? 0 : e] = l32 * kBlock + (((4 * kk + 2 * hh + e) ^ row_swz<8>(l32)) << 4);
  }

  // diagnostic codes of this lane's row (every dbg_stride-th valid row)
  uint8_t* dbg = nullptr;
  if (DBG && qb_raw < nb && qrow < S && qrow % dbg_stride == 0)
    dbg = dbg_codes + (bh * ((S + dbg_stride - 1) / dbg_stride) + qrow / dbg_stride) * S_pad;

  State<D, BF> st;
  st.ks = c.ksc[0];
  st.vs = V4 ? 1.0f : c.vsc[0];
  st.b = 0.0f;
  st.l = 0.0f;
  st.ell = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) st.bias[r] = 0.0f;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.acc[t][r] = 0.0f;

  // ---- prologue: K of tile 0; group 1 runs one phase behind group 0 ----
  if (c.dma_wave >= 0) {
    issue_k<D, BF>(c, 0, sk0);
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  if (group == 1) __syncthreads();

  // ---- nb + 1 trips, two per loop iteration (static buffer roles) ----
  for (int j = 0; j <= nb; j += 2) {
    pingpong_trip<D, BF, PC, VMEAN, V4, DBG>(j, c, st, sk0, sk1, sv1, sv0, smu1, smu0,
                                                    ssc1, ssc0, dbg);
    if (j + 1 <= nb)
      pingpong_trip<D, BF, PC, VMEAN, V4, DBG>(j + 1, c, st, sk1, sk0, sv0, sv1, smu0,
                                                      smu1, ssc0, ssc1, dbg);
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
    // m = 8 - b and l in units of 2^8 p: lse2 = m + log2(l) - 8 + q_mu
    if (hh == 0)
      lse2[bh * S + qrow] = __builtin_amdgcn_logf(st.l) - st.b + (q_mu ? q_mu[bh * S + qrow] : 0.0f);
  }
}

struct Launch {
  int total, S, H, nb, npairs, out_bf16, dbg_stride;
  hipStream_t st;
  const uint8_t *q8, *k8, *v8;
  const float *qs, *ks, *vs, *vm, *qmu;
  void* out;
  float* lse2;
  uint8_t* dbg;
};

template <int D, bool BF, int PC, bool V4, bool DBG>
void launch_vm(int vmean_mode, const Launch& a) {
  const dim3 grid(a.total), block(512);
#define VS_LAUNCH(VM)                                                                             \
  hipLaunchKernelGGL((attn_fwd_kernel<D, BF, PC, VM, V4, DBG>), grid, block, 0, a.st,          \
                     a.q8, a.qs, a.k8, a.ks, a.v8, a.vs, a.vm, a.qmu, a.S, a.H, a.nb, a.npairs,    \
                     a.total, a.out, a.out_bf16, a.lse2, a.dbg, a.dbg_stride)
  if (vmean_mode == VS_VMEAN_BLOCK) VS_LAUNCH(VS_VMEAN_BLOCK);
  else if (vmean_mode == VS_VMEAN_SEQ) VS_LAUNCH(VS_VMEAN_SEQ);
  else VS_LAUNCH(VS_VMEAN_NONE);
#undef VS_LAUNCH
}

int attn_fwd(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
             const uint8_t* v8, const float* v_scale, const float* v_mean, int vmean_mode,
             const float* q_mu, int B, int S, int H, int D, unsigned flags, void* out,
             float* lse2, uint8_t* dbg, int dbg_stride, void* stream) {
  if (B < 0 || S < 0 || H < 0) return VS_ERR_INVALID_ARG;
  if (vmean_mode != VS_VMEAN_NONE && vmean_mode != VS_VMEAN_BLOCK && vmean_mode != VS_VMEAN_SEQ)
    return VS_ERR_INVALID_ARG;
  if (flags & ~(VS_EXPCAST | VS_V_MXFP4 | VS_OUT_BF16 | VS_BF16_MMA | VS_P_MXFP4))
    return VS_ERR_INVALID_ARG;
  if (dbg && dbg_stride < 1) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (dbg && (flags & VS_V_MXFP4)) return VS_ERR_UNSUPPORTED;
  // the bf16 products take V as bf16 values, whatever format quantized it
  if ((flags & VS_BF16_MMA) && (flags & VS_V_MXFP4)) return VS_ERR_INVALID_ARG;
  // the 4-bit probability tile is its own cast, on the FP8 matrix core, with
  // E4M3 V in token order
  if ((flags & VS_P_MXFP4) && (flags & (VS_EXPCAST | VS_V_MXFP4 | VS_BF16_MMA)))
    return VS_ERR_INVALID_ARG;
  if (dbg && (flags & VS_P_MXFP4)) return VS_ERR_UNSUPPORTED;
  if (B == 0 || S == 0 || H == 0) return VS_OK;
  if ((vmean_mode == VS_VMEAN_NONE) != (v_mean == nullptr)) return VS_ERR_INVALID_ARG;
  const bool qk16 = (flags & VS_BF16_MMA) != 0;
  if (!q8 || (!qk16 && !q_scale) || !k8 || (!qk16 && !k_scale) || !v8 || !v_scale || !out || !lse2)
    return VS_ERR_INVALID_ARG;
  const void* ptrs[] = {q8, q_scale, k8, k_scale, v8, v_scale, v_mean, q_mu, out, lse2, dbg};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VS_ERR_UNSUPPORTED;
  const int nb = n_blocks(S);
  // one workgroup per (batch, head, pair of 128-query blocks)
  const int npairs = (nb + 1) / 2;
  const long long total = static_cast<long long>(B) * H * npairs;
  if (total > 0x7FFFFFFFLL) return VS_ERR_UNSUPPORTED;
  // one head's K and V (codes or bf16) are addressed through 32-bit buffer ranges
  if (static_cast<long long>(nb) * kBlock * D * (qk16 ? 2 : 1) > 0x7FFFFFFFLL)
    return VS_ERR_UNSUPPORTED;

  Launch a;
  a.total = static_cast<int>(total);
  a.S = S; a.H = H; a.nb = nb; a.npairs = npairs;
  a.out_bf16 = (flags & VS_OUT_BF16) != 0;
  a.dbg_stride = dbg ? dbg_stride : 1;
  a.st = as_stream(stream);
  a.q8 = q8; a.k8 = k8; a.v8 = v8;
  // the bf16 form carries the Q and K scales in its values; the kernel
  // never reads them then (the block scale loads are kept in range)
  a.qs = q_scale ? q_scale : v_scale;
  a.ks = k_scale ? k_scale : v_scale;
  a.vs = v_scale; a.vm = v_mean; a.qmu = q_mu;
  a.out = out; a.lse2 = lse2; a.dbg = dbg;
  const bool ec = (flags & VS_EXPCAST) != 0, v4 = (flags & VS_V_MXFP4) != 0;
  const bool p4 = (flags & VS_P_MXFP4) != 0;
  if (p4) {
    if (D == 128) launch_vm<128, false, kPcMxfp4, false, false>(vmean_mode, a);
    else launch_vm<64, false, kPcMxfp4, false, false>(vmean_mode, a);
    return launch_status();
  }
  constexpr int E = kPcE4m3, X = kPcExpcast;
  const int sel = (D == 128 ? 8 : 0) | (qk16 ? 4 : 0) | (ec ? 2 : 0) | (v4 ? 1 : 0);
  if (dbg) {
    switch (sel) {
      case 0: launch_vm<64, false, E, false, true>(vmean_mode, a); break;
      case 2: launch_vm<64, false, X, false, true>(vmean_mode, a); break;
      case 4: launch_vm<64, true, E, false, true>(vmean_mode, a); break;
      case 6: launch_vm<64, true, X, false, true>(vmean_mode, a); break;
      case 8: launch_vm<128, false, E, false, true>(vmean_mode, a); break;
      case 10: launch_vm<128, false, X, false, true>(vmean_mode, a); break;
      case 12: launch_vm<128, true, E, false, true>(vmean_mode, a); break;
      default: launch_vm<128, true, X, false, true>(vmean_mode, a); break;
    }
    return launch_status();
  }
  switch (sel) {
#define VS_A(n, d, q, e, v) case n: launch_vm<d, q, e, v, false>(vmean_mode, a); break;
    VS_A(0, 64, false, E, false) VS_A(1, 64, false, E, true)
    VS_A(2, 64, false, X, false) VS_A(3, 64, false, X, true)
    VS_A(4, 64, true, E, false) VS_A(6, 64, true, X, false)
    VS_A(8, 128, false, E, false) VS_A(9, 128, false, E, true)
    VS_A(10, 128, false, X, false) VS_A(11, 128, false, X, true)
    VS_A(12, 128, true, E, false)
    default: launch_vm<128, true, X, false, false>(vmean_mode, a); break;
#undef VS_A
  }
  return launch_status();
}

}  // namespace
}  // namespace vs

extern "C" int vs_fp8_attn_fwd(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                               const float* k_scale, const uint8_t* v8, const float* v_scale,
                               const float* v_mean, int vmean_mode, const float* q_mu, int B,
                               int S, int H, int D, unsigned flags, void* out, float* lse2,
                               void* stream) {
  return vs::attn_fwd(q8, q_scale, k8, k_scale, v8, v_scale, v_mean, vmean_mode, q_mu, B, S, H, D,
                      flags, out, lse2, nullptr, 0, stream);
}

extern "C" int vs_fp8_attn_fwd_pcodes(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                                      const float* k_scale, const uint8_t* v8,
                                      const float* v_scale, const float* v_mean, int vmean_mode,
                                      const float* q_mu, int B, int S, int H, int D,
                                      unsigned flags, void* out, float* lse2, uint8_t* p_codes,
                                      int row_stride, void* stream) {
  if (!p_codes && B > 0 && S > 0 && H > 0) return VS_ERR_INVALID_ARG;
  if (row_stride < 1) return VS_ERR_INVALID_ARG;
  return vs::attn_fwd(q8, q_scale, k8, k_scale, v8, v_scale, v_mean, vmean_mode, q_mu, B, S, H, D,
                      flags, out, lse2, p_codes, row_stride, stream);
}

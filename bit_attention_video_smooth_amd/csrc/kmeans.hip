// vs_kmeans_permute: V-Smooth grouping on gfx950.
//
// VC-Attention summary (Key Contribution 1, "Methodology in Plain English"):
// tokens are grouped by a lightweight online k-means over the value tokens,
// the labels are sorted into a permutation and K and V are permuted together
// by it; attention is unchanged since the one reordering moves the columns
// of the probability matrix and the rows of V alike.
//
// The grouping is an integer computation (see vsmooth.h), so labels and the
// permutation are the same on every run and every implementation:
//   amax    grid (nb,H,B): per-head max |V| (bf16 magnitude bits, an integer
//           max, combined with an integer atomic max)
//   codes   grid (nb,H,B): codes = rint(V * 2^-e) as int8 in two layouts of
//           32-token blocks (S32 = S rounded up to 32, zero padded): token
//           rows [B,H,S32/32,D/32,32,32] for the distance products and
//           channel rows [B,H,S32/32,D,32] (an LDS transpose) for the
//           member-sum products -- each 32 x 32-byte operand tile of a wave
//           is then one contiguous 1 KB read
//   init    grid (H,B): centroid j = codes of token floor(j*S/k)
//   T x { assign grid (ceil(S/2048),H,B): distances |c|^2 - 2 v.c as int8
//           matrix-core products (centroid tile x 32 tokens, exact int32),
//           first minimum wins; member sums as a second int8 product,
//           one-hot(labels) x channel-major codes, reduced over the
//           workgroup's 2048 tokens and written as one partial per chunk;
//         update grid (H,B): partials summed in chunk order (deterministic),
//           c = round-half-away(sum/count), empty clusters keep theirs }
//   hist    grid (ceil(S/256),H,B): label histogram per 256-token chunk
//   scan    grid (H,B): per (chunk, label) start offsets of a stable sort
//   scatter grid (ceil(S/256),H,B): rank among equal labels inside a wave
//           from ballots, wave counts through LDS -> perm
//   gather  grid (ceil(S/rows),H,B): K'[i] = K[perm[i]], V'[i] = V[perm[i]]
// All but the assign pass are HBM-bound copies/reductions; the assign pass is
// 2*S*k*D int8 MACs per head on v_mfma_i32_32x32x32_i8.
#include <algorithm>

#include "common.h"

namespace vs {
namespace {

constexpr int kChunk = 256;                 // tokens per sort workgroup
constexpr int kAsg = 2048;                  // tokens per assign workgroup (4 waves x 16 x 32)

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct KmWs {
  uint32_t* amax;     // [B,H]
  int8_t* codes;      // [B,H,S32/32,D/32,32 tokens,32 channels]
  int8_t* codes_t;    // [B,H,S32/32,D,32 tokens]
  int8_t* cent;       // [B,H,k,D]
  int32_t* psum;      // [B,H,nasg,k,D] partial member sums per assign chunk
  int32_t* pcnt;      // [B,H,nasg,k] partial member counts per assign chunk
  int32_t* chunk;     // [B,H,nchunk,k]
};

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
__host__ __device__ inline int round32(int S) { return (S + 31) & ~31; }

size_t km_layout(int B, int S, int H, int D, int k, char* base, KmWs* ws) {
  const size_t bh = static_cast<size_t>(B) * H;
  const size_t nchunk = (static_cast<size_t>(S) + kChunk - 1) / kChunk;
  const size_t nasg = (static_cast<size_t>(S) + kAsg - 1) / kAsg;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  char* a = take(bh * sizeof(uint32_t));
  char* c = take(bh * D * static_cast<size_t>(round32(S)));
  char* ct = take(bh * D * static_cast<size_t>(round32(S)));
  char* ce = take(bh * k * D);
  char* ps = take(bh * nasg * k * D * sizeof(int32_t));
  char* pc = take(bh * nasg * k * sizeof(int32_t));
  char* ch = take(bh * nchunk * k * sizeof(int32_t));
  if (ws) {
    ws->amax = reinterpret_cast<uint32_t*>(a);
    ws->codes = reinterpret_cast<int8_t*>(c);
    ws->codes_t = reinterpret_cast<int8_t*>(ct);
    ws->cent = reinterpret_cast<int8_t*>(ce);
    ws->psum = reinterpret_cast<int32_t*>(ps);
    ws->pcnt = reinterpret_cast<int32_t*>(pc);
    ws->chunk = reinterpret_cast<int32_t*>(ch);
  }
  return off;
}

// Byte offsets inside one head's codes (token rows) and channel-row copy.
template <int D>
__device__ __forceinline__ size_t xrow_off(int t, int d) {
  return ((static_cast<size_t>(t >> 5) * (D / 32) + (d >> 5)) << 10) + ((t & 31) << 5) + (d & 31);
}
template <int D>
__device__ __forceinline__ size_t xcol_off(int t, int d) {
  return (static_cast<size_t>(t >> 5) * D + d) * 32 + (t & 31);
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t val) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = val;
}

template <int D>
__global__ __launch_bounds__(256) void km_amax_kernel(const uint16_t* __restrict__ v, int S,
                                                      int H, uint32_t* __restrict__ amax,
                                                      int hfast) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  __shared__ uint32_t red[4];
  // the head is the fastest grid index (V is token-major): workgroups that
  // run together read neighbouring pieces of the same token rows
  const int j = hfast ? blockIdx.y : blockIdx.x, h = hfast ? blockIdx.x : blockIdx.y,
            b = blockIdx.z;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    if (tok < S) {
      const uint4 w = *reinterpret_cast<const uint4*>(v + token_offset(VS_LAYOUT_BSHD, b, tok, h, S, H, D) + 8 * c);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mx = max(mx, ww[e] & 0x7FFFu);
        mx = max(mx, (ww[e] >> 16) & 0x7FFFu);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), o, 64)));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    mx = max(max(red[0], red[1]), max(red[2], red[3]));
    atomicMax(&amax[static_cast<size_t>(b) * H + h], mx);
  }
}

// smallest e with amax <= 127 * 2^e (0 for amax == 0)
__device__ __forceinline__ int code_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  const double a = static_cast<double>(bf16_to_f32(amax_bits));
  int E;
  (void)frexp(a / 127.0, &E);
  int e = E;
  while (a > ldexp(127.0, e)) ++e;
  while (a <= ldexp(127.0, e - 1)) --e;
  return e;
}

template <int D>
__global__ __launch_bounds__(256) void km_codes_kernel(const uint16_t* __restrict__ v, int S,
                                                       int H, const uint32_t* __restrict__ amax,
                                                       int8_t* __restrict__ codes,
                                                       int8_t* __restrict__ codes_t,
                                                       int hfast) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  constexpr int TS = D + 4;                 // LDS row stride (bytes): fewer bank conflicts
  __shared__ __attribute__((aligned(16))) uint8_t tile[kBlock * TS];
  // the head is the fastest grid index (V is token-major): workgroups that
  // run together read neighbouring pieces of the same token rows
  const int j = hfast ? blockIdx.y : blockIdx.x, h = hfast ? blockIdx.x : blockIdx.y,
            b = blockIdx.z;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int S32 = round32(S);
  const double sc = ldexp(1.0, -code_exponent(amax[bh]));
  int8_t* const xr = codes + bh * S32 * D;
  int8_t* const xc = codes_t ? codes_t + bh * S32 * D : nullptr;
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int row = r + ROWS * i, tok = j * kBlock + row;
    uint32_t out[2] = {0u, 0u};
    if (tok < S) {
      const uint4 w = *reinterpret_cast<const uint4*>(v + token_offset(VS_LAYOUT_BSHD, b, tok, h, S, H, D) + 8 * c);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int lo = static_cast<int>(rint(static_cast<double>(bf16_to_f32(ww[e] & 0xFFFFu)) * sc));
        const int hi = static_cast<int>(rint(static_cast<double>(bf16_to_f32(ww[e] >> 16)) * sc));
        out[e >> 1] |= ((static_cast<uint32_t>(lo) & 0xFFu) | ((static_cast<uint32_t>(hi) & 0xFFu) << 8))
                       << (16 * (e & 1));
      }
    }
    // tokens past S (up to S32) get zero codes in both layouts
    if (tok < S32) *reinterpret_cast<uint2*>(xr + xrow_off<D>(tok, 8 * c)) = make_uint2(out[0], out[1]);
    *reinterpret_cast<uint32_t*>(tile + row * TS + 8 * c) = out[0];
    *reinterpret_cast<uint32_t*>(tile + row * TS + 8 * c + 4) = out[1];
  }
  // the channel-major copy is only written for the multi-tile assign pass
  if (codes_t == nullptr) return;
  __syncthreads();
  // channel rows: per 32-token sub-block, D rows of 32 bytes; thread q
  // writes 16 bytes, consecutive q consecutive in memory
  for (int q = threadIdx.x; q < D * (kBlock / 16); q += 256) {
    const int sub = q / (2 * D), d = (q >> 1) % D, t0 = 32 * sub + 16 * (q & 1);
    const int tok0 = j * kBlock + t0;
    if (tok0 >= S32) continue;
    uint32_t wv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t x = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) x |= static_cast<uint32_t>(tile[(t0 + 4 * e + u) * TS + d]) << (8 * u);
      wv[e] = x;
    }
    *reinterpret_cast<uint4*>(xc + xcol_off<D>(tok0, d)) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void km_init_kernel(const int8_t* __restrict__ codes, int S,
                                                      int H, int k, int8_t* __restrict__ cent) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = static_cast<size_t>(b) * H + h;
  for (int idx = threadIdx.x; idx < k * D; idx += blockDim.x) {
    const int jj = idx / D, d = idx % D;
    const long long src = (static_cast<long long>(jj) * S) / k;
    cent[bh * k * D + idx] = codes[bh * round32(S) * D + xrow_off<D>(static_cast<int>(src), d)];
  }
}

// Per byte of x: 1 where the byte is zero, else 0 (no carries between
// bytes: the low seven bits are added separately from the top bit).
__device__ __forceinline__ uint32_t zero_bytes_to_ones(uint32_t x) {
  const uint32_t t = (x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
  return (~(t | x | 0x7F7F7F7Fu)) >> 7;
}

// Assign pass over a chunk of 2048 tokens: 4 waves x 16 blocks of 32 tokens.
//   labels: dist^T (centroids x tokens) = C X^T on v_mfma_i32_32x32x32_i8, per
//     32-centroid tile and 32-channel k-step (A = centroid rows from LDS, B =
//     the block's token codes); a lane holds 16 centroids of one token, the
//     other 16 in lane ^ 32, so the argmin is a register scan plus one
//     v_permlane32_swap (ties: lowest index).
//   sums: S (centroid tile x channels) += onehot(labels) (tile x tokens) *
//     X (tokens x channels), B = 16 tokens of one channel from the
//     channel-major codes; the four waves' tiles meet in LDS and one partial
//     per (chunk, tile) goes to global memory.  Tokens past S have zero codes
//     there, so their one-hot bytes need no mask.
//   ONE (k <= 32, a single centroid tile): the sums are taken block by block
//     right after the labels, from the block's token codes already in
//     registers, turned into channel rows through a 32 x D byte tile per
//     wave in LDS; the channel-major copy is then neither written nor read.
template <int D, bool ONE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(ONE ? 3 : 1))) void km_assign_kernel(const int8_t* __restrict__ codes,
                                                        const int8_t* __restrict__ codes_t,
                                                        int S, int H, int k,
                                                        const int8_t* __restrict__ cent,
                                                        int32_t* __restrict__ labels,
                                                        int32_t* __restrict__ psum,
                                                        int32_t* __restrict__ pcnt) {
  constexpr int KS = D / 32;                // 32-channel k-steps
  constexpr int BPW = kAsg / 32 / 4;        // 32-token blocks per wave
  // centroids: ceil(k / 32) * 32 rows of D codes, sized at launch
  extern __shared__ __attribute__((aligned(16))) int8_t scent[];
  __shared__ int32_t snorm[256];
  __shared__ int32_t scnt[256];
  __shared__ __attribute__((aligned(16))) uint8_t slab[kAsg];
  __shared__ int32_t sred[32 * D];
  // ONE: per wave, D channel rows of the block's 32 token bytes
  __shared__ __attribute__((aligned(16))) int8_t stt[ONE ? 4 * D * 32 : 16];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int nasg = gridDim.x;
  const int S32 = round32(S);
  const int lane = threadIdx.x & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntile = ONE ? 1 : (k + 31) / 32;

  const int4* gc = reinterpret_cast<const int4*>(cent + bh * k * D);
  for (int i = threadIdx.x; i < k * D / 16; i += 256) reinterpret_cast<int4*>(scent)[i] = gc[i];
  for (int i = k * D / 16 + threadIdx.x; i < ntile * 32 * D / 16; i += 256)
    reinterpret_cast<int4*>(scent)[i] = int4{0, 0, 0, 0};
  for (int i = threadIdx.x; i < 256; i += 256) scnt[i] = 0;
  for (int i = threadIdx.x; i < 32 * D; i += 256) sred[i] = 0;
  __syncthreads();
  for (int jj = threadIdx.x; jj < k; jj += 256) {
    int n2 = 0;
    const int32_t* row = reinterpret_cast<const int32_t*>(scent + jj * D);
#pragma unroll 8
    for (int i = 0; i < D / 4; ++i) n2 = __builtin_amdgcn_sdot4(row[i], row[i], n2, false);
    snorm[jj] = n2;
  }
  __syncthreads();

  // 32-token blocks of this wave that hold tokens (the rest of the chunk is
  // past S); tokens past S inside a block have zero codes
  const int tb0 = chunk * kAsg + wave * BPW * 32;
  const int nblk = max(0, min(BPW, (S - tb0 + 31) / 32));
  const int8_t* const xr = codes + bh * S32 * D;
  const int8_t* const xc = ONE ? nullptr : codes_t + bh * S32 * D;
  int8_t* const tw = stt + (ONE ? wave * D * 32 : 0);
  // channel row c sits at row c ^ ((c >> 2) & 4): rows 16 apart (the two
  // lane halves' byte stores) then fall on different banks
  auto trow = [](int c) { return c ^ ((c >> 2) & 4); };
  v16i sacc[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) sacc[s] = v16i{};

  // ---- labels ----
  // operands of the next block are loaded while this one is processed
  auto load_x = [&](int i, v4i (&x)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      x[s] = *reinterpret_cast<const v4i*>(xr + xrow_off<D>(tb0 + 32 * i + l32, 32 * s + 16 * hh));
  };
  v4i x[KS];
  if (nblk > 0) load_x(0, x);
  for (int i = 0; i < nblk; ++i) {
    const int blk = wave * BPW + i;
    const int tok = tb0 + 32 * i + l32;
    const bool valid = tok < S;
    v4i xn[KS];
    if (i + 1 < nblk) load_x(i + 1, xn);
    int best = 0x7FFFFFFF, bidx = 0;
    for (int ct = 0; ct < ntile; ++ct) {
      v16i dot = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const v4i a = *reinterpret_cast<const v4i*>(scent + (ct * 32 + l32) * D + 32 * s + 16 * hh);
        dot = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, x[s], dot, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = ct * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < k) {
          const int dist = snorm[row] - 2 * dot[r];
          if (dist < best) { best = dist; bidx = row; }
        }
      }
    }
    // the other 16 centroids of each token sit in lane ^ 32
    const auto pd = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(best),
                                                     static_cast<unsigned>(best), false, false);
    const auto pi = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(bidx),
                                                     static_cast<unsigned>(bidx), false, false);
    const int obest = static_cast<int>(hh ? pd[0] : pd[1]);
    const int oidx = static_cast<int>(hh ? pi[0] : pi[1]);
    if (obest < best || (obest == best && oidx < bidx)) { best = obest; bidx = oidx; }
    if (hh == 0) {
      slab[blk * 32 + l32] = valid ? static_cast<uint8_t>(bidx) : 0;
      if (valid) {
        labels[bh * S + tok] = bidx;
        atomicAdd(&scnt[bidx], 1);
      }
    }
    if constexpr (ONE) {
      // lane (l32, hh) holds token l32, channels 32 s + 16 hh + e: store them
      // as channel rows, read back 16 tokens of channel 32 s + l32
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          tw[trow(32 * s + 16 * hh + e) * 32 + l32] =
              static_cast<int8_t>(static_cast<uint32_t>(x[s][e >> 2]) >> (8 * (e & 3)));
      // the stores above (and the labels in slab) come from other lanes of
      // this wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint4 lb = *reinterpret_cast<const uint4*>(slab + blk * 32 + 16 * hh);
      const uint32_t cid = static_cast<uint32_t>(l32) * 0x01010101u;
      const v4i oh = {static_cast<int>(zero_bytes_to_ones(lb.x ^ cid)),
                      static_cast<int>(zero_bytes_to_ones(lb.y ^ cid)),
                      static_cast<int>(zero_bytes_to_ones(lb.z ^ cid)),
                      static_cast<int>(zero_bytes_to_ones(lb.w ^ cid))};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const v4i xt = *reinterpret_cast<const v4i*>(tw + trow(32 * s + l32) * 32 + 16 * hh);
        sacc[s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(oh, xt, sacc[s], 0, 0, 0);
      }
      // the next block's stores must not overtake these reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (i + 1 < nblk) {
#pragma unroll
      for (int s = 0; s < KS; ++s) x[s] = xn[s];
    }
  }
  __syncthreads();
  for (int jj = threadIdx.x; jj < k; jj += 256)
    pcnt[(bh * nasg + chunk) * k + jj] = scnt[jj];

  // ---- member sums, one 32-centroid tile at a time ----
  auto load_xt = [&](int i, v4i (&xt)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      xt[s] = *reinterpret_cast<const v4i*>(xc + xcol_off<D>(tb0 + 32 * i + 16 * hh, 32 * s + l32));
  };
  for (int ct = 0; ct < ntile; ++ct) {
    v16i acc[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) acc[s] = ONE ? sacc[s] : v16i{};
    const uint32_t cid = static_cast<uint32_t>(ct * 32 + l32) * 0x01010101u;
    v4i xt[KS];
    if (!ONE && nblk > 0) load_xt(0, xt);
    for (int i = 0; i < (ONE ? 0 : nblk); ++i) {
      const int blk = wave * BPW + i;
      v4i xtn[KS];
      if (i + 1 < nblk) load_xt(i + 1, xtn);
      const uint4 lb = *reinterpret_cast<const uint4*>(slab + blk * 32 + 16 * hh);
      const v4i oh = {static_cast<int>(zero_bytes_to_ones(lb.x ^ cid)),
                      static_cast<int>(zero_bytes_to_ones(lb.y ^ cid)),
                      static_cast<int>(zero_bytes_to_ones(lb.z ^ cid)),
                      static_cast<int>(zero_bytes_to_ones(lb.w ^ cid))};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc[s] = __builtin_amdgcn_mfma_i32_32x32x32_i8(oh, xt[s], acc[s], 0, 0, 0);
      if (i + 1 < nblk) {
#pragma unroll
        for (int s = 0; s < KS; ++s) xt[s] = xtn[s];
      }
    }
    // lane holds channel 32 s + l32 of centroids 8 (r / 4) + 4 hh + r % 4
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        atomicAdd(&sred[(8 * (r >> 2) + 4 * hh + (r & 3)) * D + 32 * s + l32], acc[s][r]);
    __syncthreads();
    const int rows = min(32, k - ct * 32);
    int32_t* dst = psum + ((bh * nasg + chunk) * k + ct * 32) * D;
    for (int i = threadIdx.x; i < rows * D; i += 256) {
      dst[i] = sred[i];
      sred[i] = 0;
    }
    for (int i = rows * D + threadIdx.x; i < 32 * D; i += 256) sred[i] = 0;
    __syncthreads();
  }
}

// One thread per (centroid, channel): partials summed in chunk order.
template <int D>
__global__ __launch_bounds__(256) void km_update_kernel(int H, int k, int nasg,
                                                        int8_t* __restrict__ cent,
                                                        const int32_t* __restrict__ psum,
                                                        const int32_t* __restrict__ pcnt) {
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= k * D) return;
  const int jj = idx / D;
  int n = 0;
  long long sum = 0;
  for (int c = 0; c < nasg; ++c) {
    n += pcnt[(bh * nasg + c) * k + jj];
    sum += psum[(bh * nasg + c) * k * D + idx];
  }
  if (n > 0) {
    const long long mag = (2LL * (sum < 0 ? -sum : sum) + n) / (2LL * n);
    cent[bh * k * D + idx] = static_cast<int8_t>(sum < 0 ? -mag : mag);
  }
}

__global__ __launch_bounds__(256) void km_hist_kernel(const int32_t* __restrict__ labels, int S,
                                                      int H, int k, int nchunk,
                                                      int32_t* __restrict__ chunk) {
  __shared__ int32_t hist[256];
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = static_cast<size_t>(b) * H + h;
  hist[threadIdx.x] = 0;
  __syncthreads();
  const int tok = blockIdx.x * kChunk + threadIdx.x;
  if (tok < S) atomicAdd(&hist[labels[bh * S + tok]], 1);
  __syncthreads();
  if (threadIdx.x < k) chunk[(bh * nchunk + blockIdx.x) * k + threadIdx.x] = hist[threadIdx.x];
}

// counts -> start offsets, in place: offset(c, j) = sum_{j' < j} total(j') +
// sum_{c' < c} count(c', j).
// Exclusive offsets of the counting sort: chunk[c][j] becomes the number of
// tokens with a smaller label, plus those with label j in chunks before c
// (integer, so any summation order gives the same result).  The 256 threads
// split into P = 256 / k parts per label, each over a contiguous range of
// chunks: range sums, then per label a scan over the parts and the
// labels before it, then each range written out.
__global__ __launch_bounds__(256) void km_scan_kernel(int H, int k, int nchunk,
                                                      int32_t* __restrict__ chunk) {
  __shared__ int32_t part[256];
  __shared__ int32_t tot[256];
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = static_cast<size_t>(b) * H + h;
  int32_t* ch = chunk + bh * nchunk * k;
  const int P = 256 / k;                     // parts per label (k <= 256)
  const int jj = threadIdx.x % k, p = threadIdx.x / k;
  const bool active = p < P;
  const int c0 = active ? static_cast<int>(static_cast<long long>(p) * nchunk / P) : 0;
  const int c1 = active ? static_cast<int>(static_cast<long long>(p + 1) * nchunk / P) : 0;
  int t = 0;
  for (int c = c0; c < c1; ++c) t += ch[static_cast<size_t>(c) * k + jj];
  if (active) part[p * k + jj] = t;
  __syncthreads();
  if (threadIdx.x < k) {
    int s = 0;
    for (int q = 0; q < P; ++q) s += part[q * k + threadIdx.x];
    tot[threadIdx.x] = s;
  }
  __syncthreads();
  if (active) {
    int base = 0;
    for (int i = 0; i < jj; ++i) base += tot[i];
    for (int q = 0; q < p; ++q) base += part[q * k + jj];
    for (int c = c0; c < c1; ++c) {
      const int n = ch[static_cast<size_t>(c) * k + jj];
      ch[static_cast<size_t>(c) * k + jj] = base;
      base += n;
    }
  }
}

__global__ __launch_bounds__(256) void km_scatter_kernel(const int32_t* __restrict__ labels, int S,
                                                         int H, int k, int nchunk,
                                                         const int32_t* __restrict__ chunk,
                                                         int32_t* __restrict__ perm) {
  __shared__ int32_t wcnt[4][256];
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 4 * 256; i += 256) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const int tok = blockIdx.x * kChunk + threadIdx.x;
  const bool valid = tok < S;
  const int lab = valid ? labels[bh * S + tok] : 0;
  // lanes of this wave holding the same label
  unsigned long long same = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const unsigned long long bal = __ballot((lab >> bit) & 1);
    same &= ((lab >> bit) & 1) ? bal : ~bal;
  }
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(same & below);
  if (valid && rank == 0) wcnt[w][lab] = __popcll(same);
  __syncthreads();
  if (valid) {
    int pos = chunk[(bh * nchunk + blockIdx.x) * k + lab] + rank;
    for (int ww = 0; ww < w; ++ww) pos += wcnt[ww][lab];
    perm[bh * S + pos] = tok;
  }
}

template <int D>
__global__ __launch_bounds__(256) void km_gather_kernel(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, int S,
                                                        int H, const int32_t* __restrict__ perm,
                                                        uint16_t* __restrict__ kp,
                                                        uint16_t* __restrict__ vp) {
  constexpr int TPR = D / 8, RPW = 256 / TPR;
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int i = blockIdx.x * RPW + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (i >= S) return;
  const int src = perm[bh * S + i];
  const size_t so = token_offset(VS_LAYOUT_BSHD, b, src, h, S, H, D) + 8 * c;
  const size_t d0 = (bh * S + i) * D + 8 * c;
  *reinterpret_cast<uint4*>(kp + d0) = *reinterpret_cast<const uint4*>(k + so);
  *reinterpret_cast<uint4*>(vp + d0) = *reinterpret_cast<const uint4*>(v + so);
}

template <int D>
void run_kmeans(const uint16_t* k, const uint16_t* v, int B, int S, int H, int kc, int iters,
                int32_t* labels, int32_t* perm, uint16_t* kp, uint16_t* vp, const KmWs& ws,
                hipStream_t st) {
  const int nb = n_blocks(S);
  const int nchunk = (S + kChunk - 1) / kChunk;
  const size_t bh = static_cast<size_t>(B) * H;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(static_cast<unsigned>(std::min<size_t>((bh + 255) / 256, 1024))),
                     dim3(256), 0, st, ws.amax, bh, 0u);
  // the amax pass only reads V: head-fastest order (neighbouring pieces of
  // the same token rows) measured 28-34% faster; the codes pass, whose
  // writes go to head-major layouts, runs block-fastest (5% faster so)
  const int hfast = nb <= 65535;
  hipLaunchKernelGGL(km_amax_kernel<D>, hfast ? dim3(H, nb, B) : dim3(nb, H, B), dim3(256), 0, st,
                     v, S, H, ws.amax, hfast);
  // up to 32 clusters the assign pass builds the channel rows itself
  const bool one = kc <= 32;
  hipLaunchKernelGGL(km_codes_kernel<D>, dim3(nb, H, B), dim3(256), 0, st, v, S, H, ws.amax,
                     ws.codes, one ? nullptr : ws.codes_t, 0);
  hipLaunchKernelGGL(km_init_kernel<D>, dim3(H, B), dim3(256), 0, st, ws.codes, S, H, kc, ws.cent);
  const int nasg = (S + kAsg - 1) / kAsg;
  for (int it = 0; it < iters; ++it) {
    if (one)
      hipLaunchKernelGGL((km_assign_kernel<D, true>), dim3(nasg, H, B), dim3(256),
                         static_cast<unsigned>(32 * D), st, ws.codes, nullptr, S, H, kc, ws.cent,
                         labels, ws.psum, ws.pcnt);
    else
      hipLaunchKernelGGL((km_assign_kernel<D, false>), dim3(nasg, H, B), dim3(256),
                         static_cast<unsigned>((kc + 31) / 32 * 32 * D), st, ws.codes,
                         ws.codes_t, S, H, kc, ws.cent, labels, ws.psum, ws.pcnt);
    hipLaunchKernelGGL(km_update_kernel<D>, dim3((kc * D + 255) / 256, H, B), dim3(256), 0, st, H,
                       kc, nasg, ws.cent, ws.psum, ws.pcnt);
  }
  hipLaunchKernelGGL(km_hist_kernel, dim3(nchunk, H, B), dim3(256), 0, st, labels, S, H, kc, nchunk,
                     ws.chunk);
  hipLaunchKernelGGL(km_scan_kernel, dim3(H, B), dim3(256), 0, st, H, kc, nchunk, ws.chunk);
  hipLaunchKernelGGL(km_scatter_kernel, dim3(nchunk, H, B), dim3(256), 0, st, labels, S, H, kc,
                     nchunk, ws.chunk, perm);
  if (!kp) return;
  constexpr int RPW = 256 / (D / 8);
  hipLaunchKernelGGL(km_gather_kernel<D>, dim3((S + RPW - 1) / RPW, H, B), dim3(256), 0, st, k, v, S,
                     H, perm, kp, vp);
}

}  // namespace
}  // namespace vs

extern "C" int vs_kmeans_workspace_bytes(int B, int S, int H, int D, int k_clusters,
                                         size_t* bytes) {
  if (!bytes || B < 0 || S < 0 || H < 0) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (k_clusters < 1) return VS_ERR_INVALID_ARG;
  if (k_clusters > 256) return VS_ERR_UNSUPPORTED;
  *bytes = vs::km_layout(B, S, H, D, k_clusters, nullptr, nullptr);
  return VS_OK;
}

extern "C" int vs_kmeans_permute(const uint16_t* k, const uint16_t* v, int B, int S, int H, int D,
                                 int k_clusters, int iters, int32_t* labels, int32_t* perm,
                                 uint16_t* k_perm, uint16_t* v_perm, void* ws, size_t ws_bytes,
                                 void* stream) {
  using namespace vs;
  if (B < 0 || S < 0 || H < 0 || iters < 1 || k_clusters < 1) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (k_clusters > 256) return VS_ERR_UNSUPPORTED;
  if (B == 0 || S == 0 || H == 0) return VS_OK;
  if (!k || !v || !labels || !perm) return VS_ERR_INVALID_ARG;
  // both gather outputs or neither (then labels and perm only)
  if ((k_perm == nullptr) != (v_perm == nullptr)) return VS_ERR_INVALID_ARG;
  const void* ptrs[] = {k, v, labels, perm, k_perm, v_perm};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VS_ERR_UNSUPPORTED;
  const size_t need = km_layout(B, S, H, D, k_clusters, nullptr, nullptr);
  if (!ws || ws_bytes < need) return VS_ERR_WORKSPACE;
  if (!aligned16(ws)) return VS_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535) return VS_ERR_UNSUPPORTED;
  KmWs w;
  km_layout(B, S, H, D, k_clusters, static_cast<char*>(ws), &w);
  hipStream_t st = as_stream(stream);
  if (D == 128) run_kmeans<128>(k, v, B, S, H, k_clusters, iters, labels, perm, k_perm, v_perm, w, st);
  else run_kmeans<64>(k, v, B, S, H, k_clusters, iters, labels, perm, k_perm, v_perm, w, st);
  return launch_status();
}

// vs_kmeans_permute: V-Smooth grouping on gfx950.
//
// VC-Attention summary (Key Contribution 1, "Methodology in Plain English"):
// tokens are grouped by a lightweight online k-means over the value tokens,
// the labels are sorted into a permutation and K and V are permuted together
// by it; attention is unchanged because permuting keys permutes the columns
// of the probability matrix exactly as the rows of V.
//
// The grouping is an integer computation (see vsmooth.h), so labels and the
// permutation are the same on every run and every implementation:
//   amax    grid (nb,H,B): per-head max |V| (bf16 magnitude bits, an integer
//           max, combined with an integer atomic max)
//   codes   grid (nb,H,B): codes = rint(V * 2^-e) as int8 [B,H,S,D]
//   init    grid (H,B): centroid j = codes of token floor(j*S/k)
//   T x { assign grid (ceil(S/256),H,B): one token per thread, distances
//           |c|^2 - 2 v.c with v_dot4_i32_i8 against centroids broadcast from
//           LDS, first minimum wins; member sums and counts accumulated in
//           LDS with integer atomics (order-independent), then added to the
//           global sums with integer atomics;
//         update grid (H,B): c = round-half-away(sum/count), empty keeps }
//   hist    grid (ceil(S/256),H,B): label histogram per 256-token chunk
//   scan    grid (H,B): per (chunk, label) start offsets of a stable sort
//   scatter grid (ceil(S/256),H,B): rank among equal labels inside a wave
//           from ballots, wave counts through LDS -> perm
//   gather  grid (ceil(S/rows),H,B): K'[i] = K[perm[i]], V'[i] = V[perm[i]]
// All but the assign pass are HBM-bound copies/reductions; the assign pass is
// S*k*D int8 MACs per head at 4 MACs per lane-op.
#include <algorithm>

#include "common.h"

namespace vs {
namespace {

constexpr int kChunk = 256;                 // tokens per assign / sort workgroup

struct KmWs {
  uint32_t* amax;     // [B,H]
  int8_t* codes;      // [B,H,S,D]
  int8_t* cent;       // [B,H,k,D]
  int32_t* sums;      // [B,H,k,D]
  int32_t* cnt;       // [B,H,k]
  int32_t* chunk;     // [B,H,nchunk,k]
};

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t km_layout(int B, int S, int H, int D, int k, char* base, KmWs* ws) {
  const size_t bh = static_cast<size_t>(B) * H;
  const size_t nchunk = (static_cast<size_t>(S) + kChunk - 1) / kChunk;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  char* a = take(bh * sizeof(uint32_t));
  char* c = take(bh * S * D);
  char* ce = take(bh * k * D);
  char* su = take(bh * k * D * sizeof(int32_t));
  char* cn = take(bh * k * sizeof(int32_t));
  char* ch = take(bh * nchunk * k * sizeof(int32_t));
  if (ws) {
    ws->amax = reinterpret_cast<uint32_t*>(a);
    ws->codes = reinterpret_cast<int8_t*>(c);
    ws->cent = reinterpret_cast<int8_t*>(ce);
    ws->sums = reinterpret_cast<int32_t*>(su);
    ws->cnt = reinterpret_cast<int32_t*>(cn);
    ws->chunk = reinterpret_cast<int32_t*>(ch);
  }
  return off;
}

__global__ void fill_u32_kernel(uint32_t* p, size_t n, uint32_t val) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = val;
}

template <int D>
__global__ __launch_bounds__(256) void km_amax_kernel(const uint16_t* __restrict__ v, int S,
                                                      int H, uint32_t* __restrict__ amax) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  __shared__ uint32_t red[4];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
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
                                                       int8_t* __restrict__ codes) {
  constexpr int CH = D / 8, ROWS = 256 / CH, TPT = kBlock / ROWS;
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const double sc = ldexp(1.0, -code_exponent(amax[bh]));
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    if (tok < S) {
      const uint4 w = *reinterpret_cast<const uint4*>(v + token_offset(VS_LAYOUT_BSHD, b, tok, h, S, H, D) + 8 * c);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
      uint32_t out[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int lo = static_cast<int>(rint(static_cast<double>(bf16_to_f32(ww[e] & 0xFFFFu)) * sc));
        const int hi = static_cast<int>(rint(static_cast<double>(bf16_to_f32(ww[e] >> 16)) * sc));
        out[e >> 1] |= ((static_cast<uint32_t>(lo) & 0xFFu) | ((static_cast<uint32_t>(hi) & 0xFFu) << 8))
                       << (16 * (e & 1));
      }
      *reinterpret_cast<uint2*>(codes + (bh * S + tok) * D + 8 * c) = make_uint2(out[0], out[1]);
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void km_init_kernel(const int8_t* __restrict__ codes, int S,
                                                      int H, int k, int8_t* __restrict__ cent,
                                                      int32_t* __restrict__ sums,
                                                      int32_t* __restrict__ cnt) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = static_cast<size_t>(b) * H + h;
  for (int idx = threadIdx.x; idx < k * D; idx += blockDim.x) {
    const int jj = idx / D, d = idx % D;
    const long long src = (static_cast<long long>(jj) * S) / k;
    cent[bh * k * D + idx] = codes[(bh * S + src) * D + d];
    sums[bh * k * D + idx] = 0;
  }
  for (int jj = threadIdx.x; jj < k; jj += blockDim.x) cnt[bh * k + jj] = 0;
}

// One token per thread.  LDS: centroids (int8, k x D), their squared norms,
// and a slice of member sums (int32) of 4096 entries (16 KB); k above the
// slice size takes several passes over the slices.
template <int D>
__global__ __launch_bounds__(256) void km_assign_kernel(const int8_t* __restrict__ codes, int S,
                                                        int H, int k,
                                                        const int8_t* __restrict__ cent,
                                                        int32_t* __restrict__ labels,
                                                        int32_t* __restrict__ sums,
                                                        int32_t* __restrict__ cnt) {
  constexpr int DW = D / 4;                         // int8x4 words per token
  constexpr int SLICE = 4096 / D;                   // clusters per LDS sum slice
  __shared__ __attribute__((aligned(16))) int32_t scent[256 * DW];
  __shared__ int32_t snorm[256];
  __shared__ int32_t scnt[256];
  __shared__ int32_t ssum[SLICE * D];
  const int h = blockIdx.y, b = blockIdx.z;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int tok = blockIdx.x * kChunk + threadIdx.x;
  const bool valid = tok < S;

  const int32_t* gc = reinterpret_cast<const int32_t*>(cent + bh * k * D);
  for (int i = threadIdx.x; i < k * DW; i += 256) scent[i] = gc[i];
  for (int i = threadIdx.x; i < k; i += 256) scnt[i] = 0;
  __syncthreads();
  for (int jj = threadIdx.x; jj < k; jj += 256) {
    int n2 = 0;
#pragma unroll 8
    for (int i = 0; i < DW; ++i) n2 = __builtin_amdgcn_sdot4(scent[jj * DW + i], scent[jj * DW + i], n2, false);
    snorm[jj] = n2;
  }

  int32_t x[DW];
  if (valid) {
    const int4* src = reinterpret_cast<const int4*>(codes + (bh * S + tok) * D);
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
      const int4 w = src[i];
      x[4 * i] = w.x; x[4 * i + 1] = w.y; x[4 * i + 2] = w.z; x[4 * i + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < DW; ++i) x[i] = 0;
  }
  __syncthreads();

  int best = 0x7FFFFFFF, lab = 0;
  for (int jj = 0; jj < k; ++jj) {
    int dot = 0;
#pragma unroll
    for (int i = 0; i < DW; ++i) dot = __builtin_amdgcn_sdot4(x[i], scent[jj * DW + i], dot, false);
    const int dist = snorm[jj] - 2 * dot;
    if (dist < best) { best = dist; lab = jj; }
  }
  if (valid) {
    labels[bh * S + tok] = lab;
    atomicAdd(&scnt[lab], 1);
  }

  for (int s0 = 0; s0 < k; s0 += SLICE) {
    const int ns = min(SLICE, k - s0);
    __syncthreads();
    for (int i = threadIdx.x; i < ns * D; i += 256) ssum[i] = 0;
    __syncthreads();
    if (valid && lab >= s0 && lab < s0 + ns) {
      int32_t* row = ssum + (lab - s0) * D;
#pragma unroll
      for (int i = 0; i < DW; ++i) {
        atomicAdd(&row[4 * i + 0], static_cast<int32_t>(static_cast<int8_t>(x[i] & 0xFF)));
        atomicAdd(&row[4 * i + 1], static_cast<int32_t>(static_cast<int8_t>((x[i] >> 8) & 0xFF)));
        atomicAdd(&row[4 * i + 2], static_cast<int32_t>(static_cast<int8_t>((x[i] >> 16) & 0xFF)));
        atomicAdd(&row[4 * i + 3], static_cast<int32_t>(static_cast<int8_t>((x[i] >> 24) & 0xFF)));
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < ns * D; i += 256)
      if (ssum[i] != 0) atomicAdd(&sums[bh * k * D + static_cast<size_t>(s0) * D + i], ssum[i]);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += 256)
    if (scnt[i] != 0) atomicAdd(&cnt[bh * k + i], scnt[i]);
}

template <int D>
__global__ __launch_bounds__(256) void km_update_kernel(int H, int k, int8_t* __restrict__ cent,
                                                        int32_t* __restrict__ sums,
                                                        int32_t* __restrict__ cnt) {
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = static_cast<size_t>(b) * H + h;
  for (int idx = threadIdx.x; idx < k * D; idx += blockDim.x) {
    const int n = cnt[bh * k + idx / D];
    const int s = sums[bh * k * D + idx];
    if (n > 0) {
      const long long mag = (2LL * (s < 0 ? -static_cast<long long>(s) : s) + n) / (2LL * n);
      cent[bh * k * D + idx] = static_cast<int8_t>(s < 0 ? -mag : mag);
    }
    sums[bh * k * D + idx] = 0;
  }
  __syncthreads();
  for (int jj = threadIdx.x; jj < k; jj += blockDim.x) cnt[bh * k + jj] = 0;
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
__global__ __launch_bounds__(256) void km_scan_kernel(int H, int k, int nchunk,
                                                      int32_t* __restrict__ chunk) {
  __shared__ int32_t tot[256];
  const int h = blockIdx.x, b = blockIdx.y;
  const size_t bh = static_cast<size_t>(b) * H + h;
  int32_t* ch = chunk + bh * nchunk * k;
  const int jj = threadIdx.x;
  int t = 0;
  if (jj < k)
    for (int c = 0; c < nchunk; ++c) t += ch[static_cast<size_t>(c) * k + jj];
  tot[jj] = (jj < k) ? t : 0;
  __syncthreads();
  if (jj < k) {
    int base = 0;
    for (int i = 0; i < jj; ++i) base += tot[i];
    for (int c = 0; c < nchunk; ++c) {
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
  hipLaunchKernelGGL(km_amax_kernel<D>, dim3(nb, H, B), dim3(256), 0, st, v, S, H, ws.amax);
  hipLaunchKernelGGL(km_codes_kernel<D>, dim3(nb, H, B), dim3(256), 0, st, v, S, H, ws.amax, ws.codes);
  hipLaunchKernelGGL(km_init_kernel<D>, dim3(H, B), dim3(256), 0, st, ws.codes, S, H, kc, ws.cent,
                     ws.sums, ws.cnt);
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL(km_assign_kernel<D>, dim3(nchunk, H, B), dim3(256), 0, st, ws.codes, S, H, kc,
                       ws.cent, labels, ws.sums, ws.cnt);
    hipLaunchKernelGGL(km_update_kernel<D>, dim3(H, B), dim3(256), 0, st, H, kc, ws.cent, ws.sums,
                       ws.cnt);
  }
  hipLaunchKernelGGL(km_hist_kernel, dim3(nchunk, H, B), dim3(256), 0, st, labels, S, H, kc, nchunk,
                     ws.chunk);
  hipLaunchKernelGGL(km_scan_kernel, dim3(H, B), dim3(256), 0, st, H, kc, nchunk, ws.chunk);
  hipLaunchKernelGGL(km_scatter_kernel, dim3(nchunk, H, B), dim3(256), 0, st, labels, S, H, kc,
                     nchunk, ws.chunk, perm);
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
  if (!k || !v || !labels || !perm || !k_perm || !v_perm) return VS_ERR_INVALID_ARG;
  const void* ptrs[] = {k, v, labels, perm, k_perm, v_perm};
  for (const void* p : ptrs)
    if (!aligned16(p)) return VS_ERR_UNSUPPORTED;
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

// vs_smooth_stats: exact K/V statistics in one pass over K and V.
//
// TeleFuser PR #40 ("Changes") fuses exact K/V statistics into a single
// reduction, centres K by its sequence mean in FP32 and centres V; the
// VC-Attention summary (Key Contribution 1) subtracts each hardware block's
// V mean.  Both means come out of the same pass here:
//
//   stage 1, grid (nb, H, B): one workgroup per 128-token block sums K and V
//     over its valid tokens in float64 (a bf16 value has 8 significant bits,
//     so these sums are exact), writes the block mean of V and keeps the two
//     block sums in the workspace.  With no V output requested V is not
//     read (v == nullptr).
//   stage 2, grid (H, B): sums the nb block sums in a fixed order and writes
//     the sequence means.  Fixed orders make the result deterministic.
//
// With rotary tables (cos / sin, [S, D/2] float32, row = token) K is
// rotated first, in the order and precision the Q/K quantizers use, so the
// mean is that of the rotated keys the attention sees.
//
// HBM-bound: K and V are read once (4 bytes per element pair); the float64
// adds are far below the FP64 vector rate.
#include <mutex>

#include "common.h"

namespace vs {
namespace {

template <int D, bool ROPE>
__global__ __launch_bounds__(256) void stats_block_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int layout,
    int S, int H, int nb, float* __restrict__ v_block_mean,
    double* __restrict__ ws_k, double* __restrict__ ws_v, int hfast,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin) {
  constexpr int CH = D / 8;           // 16-byte chunks per token row
  constexpr int ROWS = 256 / CH;      // token lanes per workgroup
  constexpr int TPT = kBlock / ROWS;  // tokens per thread
  __shared__ double red[ROWS][D];

  // token-major input: the head is the fastest grid index, so workgroups
  // that run together read neighbouring pieces of the same token rows
  const int j = hfast ? blockIdx.y : blockIdx.x, h = hfast ? blockIdx.x : blockIdx.y,
            b = blockIdx.z;
  const int c = threadIdx.x % CH, r = threadIdx.x / CH;
  double sk[8], sv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sk[e] = sv[e] = 0.0;

#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int tok = j * kBlock + r + ROWS * i;
    if (tok < S) {
      const size_t off = token_offset(layout, b, tok, h, S, H, D) + 8 * c;
      const uint4 kk = *reinterpret_cast<const uint4*>(k + off);
      const uint4 vv = v ? *reinterpret_cast<const uint4*>(v + off) : uint4{0u, 0u, 0u, 0u};
      const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = bf16_to_f32(kw[e] & 0xFFFFu);
        kf[2 * e + 1] = bf16_to_f32(kw[e] >> 16);
      }
      if (ROPE) {
        const size_t t = static_cast<size_t>(tok) * (D / 2) + 4 * c;
        rope8(kf, *reinterpret_cast<const float4*>(rope_cos + t),
              *reinterpret_cast<const float4*>(rope_sin + t));
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sk[2 * e] += static_cast<double>(kf[2 * e]);
        sk[2 * e + 1] += static_cast<double>(kf[2 * e + 1]);
        sv[2 * e] += static_cast<double>(bf16_to_f32(vw[e] & 0xFFFFu));
        sv[2 * e + 1] += static_cast<double>(bf16_to_f32(vw[e] >> 16));
      }
    }
  }

  const int n = min(kBlock, S - j * kBlock);
  const size_t out = ((static_cast<size_t>(b) * H + h) * nb + j) * D;
  // K block sums
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r][8 * c + e] = sk[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
    for (int rr = 0; rr < ROWS; ++rr) s += red[rr][threadIdx.x];
    ws_k[out + threadIdx.x] = s;
  }
  if (!v) return;
  __syncthreads();
  // V block sums and block means
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r][8 * c + e] = sv[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
    for (int rr = 0; rr < ROWS; ++rr) s += red[rr][threadIdx.x];
    ws_v[out + threadIdx.x] = s;
    if (v_block_mean) v_block_mean[out + threadIdx.x] = static_cast<float>(s / static_cast<double>(n));
  }
}

// One workgroup per (b, h, 32-channel slice): G = 32 groups of 32 threads
// each sum a strided subset of the block sums of the slice's channels, then
// group 0 adds the G partials in order.  The float64 sums of bf16 values
// are exact, so the result does not depend on the split.
template <int D>
__global__ __launch_bounds__(1024) void stats_seq_kernel(
    const double* __restrict__ ws_k, const double* __restrict__ ws_v, int S,
    int H, int nb, float* __restrict__ k_mean, float* __restrict__ v_seq_mean) {
  constexpr int C = 32, G = 1024 / C;
  __shared__ double part[2][G][C];
  const int h = blockIdx.x, b = blockIdx.y;
  const int c = threadIdx.x % C, g = threadIdx.x / C;
  const int d = blockIdx.z * C + c;
  const size_t base = (static_cast<size_t>(b) * H + h) * nb * D;
  double sk = 0.0, sv = 0.0;
  for (int j = g; j < nb; j += G) {
    sk += ws_k[base + static_cast<size_t>(j) * D + d];
    if (v_seq_mean) sv += ws_v[base + static_cast<size_t>(j) * D + d];
  }
  part[0][g][c] = sk;
  part[1][g][c] = sv;
  __syncthreads();
  if (g == 0) {
    double tk = 0.0, tv = 0.0;
    for (int gg = 0; gg < G; ++gg) {
      tk += part[0][gg][c];
      tv += part[1][gg][c];
    }
    const size_t o = (static_cast<size_t>(b) * H + h) * D + d;
    if (k_mean) k_mean[o] = static_cast<float>(tk / static_cast<double>(S));
    if (v_seq_mean) v_seq_mean[o] = static_cast<float>(tv / static_cast<double>(S));
  }
}

size_t ws_bytes_needed(int B, int S, int H, int D) {
  return 2 * static_cast<size_t>(B) * H * n_blocks(S) * D * sizeof(double);
}

}  // namespace
}  // namespace vs

extern "C" int vs_smooth_stats_workspace_bytes(int B, int S, int H, int D, size_t* bytes) {
  if (!bytes || B < 0 || S < 0 || H < 0) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  *bytes = vs::ws_bytes_needed(B, S, H, D);
  return VS_OK;
}

namespace vs {
namespace {

// Argument checks shared by both entry points (workspace excepted).
int check_args(const uint16_t* k, const uint16_t* v, int B, int S, int H, int D, int layout,
               const float* k_mean, const float* v_block_mean, const float* v_seq_mean,
               const float* rope_cos = nullptr, const float* rope_sin = nullptr) {
  if (B < 0 || S < 0 || H < 0) return VS_ERR_INVALID_ARG;
  if (!rope_cos != !rope_sin) return VS_ERR_INVALID_ARG;
  if (layout != VS_LAYOUT_BSHD && layout != VS_LAYOUT_BHSD) return VS_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return VS_ERR_UNSUPPORTED;
  if (B == 0 || S == 0 || H == 0) return VS_OK;
  if (!k_mean && !v_block_mean && !v_seq_mean) return VS_ERR_INVALID_ARG;
  if (!k || (!v && (v_block_mean || v_seq_mean))) return VS_ERR_INVALID_ARG;
  if (!aligned16(k) || (v && !aligned16(v)) || (k_mean && !aligned16(k_mean)) ||
      (v_block_mean && !aligned16(v_block_mean)) || (v_seq_mean && !aligned16(v_seq_mean)) ||
      (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))))
    return VS_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535) return VS_ERR_UNSUPPORTED;
  return VS_OK;
}

// Both stages on a workspace of at least ws_bytes_needed() bytes.  Stage 1
// writes every block sum it covers before stage 2 reads it, so the
// workspace needs no clearing.
template <int D, bool ROPE>
void launch_stats_d(const uint16_t* k, const uint16_t* v, int S, int H, int nb, int layout,
                    float* k_mean, float* v_block_mean, float* v_seq_mean, double* ws_k,
                    double* ws_v, int hfast, const dim3& g1, const dim3& g2,
                    const float* rope_cos, const float* rope_sin, hipStream_t st) {
  hipLaunchKernelGGL((stats_block_kernel<D, ROPE>), g1, dim3(256), 0, st, k, v, layout, S, H, nb,
                     v_block_mean, ws_k, ws_v, hfast, rope_cos, rope_sin);
  hipLaunchKernelGGL(stats_seq_kernel<D>, g2, dim3(1024), 0, st, ws_k, ws_v, S, H, nb, k_mean,
                     v_seq_mean);
}

int launch_stats(const uint16_t* k, const uint16_t* v, int B, int S, int H, int D, int layout,
                 float* k_mean, float* v_block_mean, float* v_seq_mean, double* ws,
                 const float* rope_cos, const float* rope_sin, hipStream_t st) {
  const int nb = n_blocks(S);
  double* ws_k = ws;
  double* ws_v = ws_k + static_cast<size_t>(B) * H * nb * D;
  const int hfast = layout == VS_LAYOUT_BSHD && nb <= 65535;
  const dim3 g1 = hfast ? dim3(H, nb, B) : dim3(nb, H, B), g2(H, B, D / 32);
#define VS_STATS(DD, R)                                                                      \
  launch_stats_d<DD, R>(k, v, S, H, nb, layout, k_mean, v_block_mean, v_seq_mean, ws_k, ws_v, \
                        hfast, g1, g2, rope_cos, rope_sin, st)
  if (D == 128) {
    if (rope_cos) VS_STATS(128, true); else VS_STATS(128, false);
  } else {
    if (rope_cos) VS_STATS(64, true); else VS_STATS(64, false);
  }
#undef VS_STATS
  return launch_status();
}

// The statistics workspace of vs_smooth_stats_noalloc: one array per GPU,
// held by the loaded library for the life of the process.  In host code the
// name is only a stand-in for the device symbol; its device address, which
// differs per GPU, comes from hipGetSymbolAddress once per device.
constexpr size_t kScratchBytes = static_cast<size_t>(VS_NOALLOC_STATS_SCRATCH_BYTES);
__device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
double* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (the current device), looked up
// on the first call on that device; nullptr if HIP reports an error.
double* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = static_cast<double*>(ptr);
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace vs

extern "C" int vs_smooth_stats_ex(const uint16_t* k, const uint16_t* v, int B, int S, int H,
                                  int D, int layout, const float* rope_cos,
                                  const float* rope_sin, float* k_mean, float* v_block_mean,
                                  float* v_seq_mean, void* ws, size_t ws_bytes, void* stream) {
  using namespace vs;
  const int rc =
      check_args(k, v, B, S, H, D, layout, k_mean, v_block_mean, v_seq_mean, rope_cos, rope_sin);
  if (rc != VS_OK || B == 0 || S == 0 || H == 0) return rc;
  const size_t need = ws_bytes_needed(B, S, H, D);
  if (!ws || ws_bytes < need) return VS_ERR_WORKSPACE;
  if (!aligned16(ws)) return VS_ERR_UNSUPPORTED;
  return launch_stats(k, v, B, S, H, D, layout, k_mean, v_block_mean, v_seq_mean,
                      static_cast<double*>(ws), rope_cos, rope_sin, as_stream(stream));
}

extern "C" int vs_smooth_stats(const uint16_t* k, const uint16_t* v, int B, int S, int H,
                               int D, int layout, float* k_mean, float* v_block_mean,
                               float* v_seq_mean, void* ws, size_t ws_bytes, void* stream) {
  return vs_smooth_stats_ex(k, v, B, S, H, D, layout, nullptr, nullptr, k_mean, v_block_mean,
                            v_seq_mean, ws, ws_bytes, stream);
}

extern "C" int vs_smooth_stats_noalloc(const uint16_t* k, const uint16_t* v, int B, int S,
                                       int H, int D, int layout, float* k_mean,
                                       float* v_block_mean, float* v_seq_mean, void* stream) {
  using namespace vs;
  const int rc = check_args(k, v, B, S, H, D, layout, k_mean, v_block_mean, v_seq_mean);
  if (rc != VS_OK || B == 0 || S == 0 || H == 0) return rc;
  if (ws_bytes_needed(B, S, H, D) > kScratchBytes) return VS_ERR_WORKSPACE;
  double* ws = scratch_for_current_device();
  if (!ws) return VS_ERR_HIP;
  return launch_stats(k, v, B, S, H, D, layout, k_mean, v_block_mean, v_seq_mean, ws, nullptr,
                      nullptr, as_stream(stream));
}

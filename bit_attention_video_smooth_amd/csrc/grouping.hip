// vs_cube_permutation: the static spatiotemporal-cube grouping of a video
// token grid (VC-Attention summary, Main Findings: block demeaning under a
// static space-time cube ordering; Key Contribution 3: permutations reused
// across calls).  Host code: the permutation depends on the grid alone, so a
// caller forms it once and hands it to vs_quantize_residual_perm on every
// call, like a k-means permutation it keeps.
//
// Token s sits at grid position (t, y, x), s = (t * Hg + y) * W + x; cubes of
// ct x ch x cw positions tile the grid from the origin (shorter at the far
// edges) and are visited in raster order of the cube grid, the tokens of a
// cube in raster order; positions s >= S (a grid larger than the sequence)
// hold no token and are skipped.
#include "common.h"

extern "C" int vs_cube_permutation(int S, int T, int Hg, int W, int ct, int ch, int cw,
                                   int32_t* perm) {
  if (S < 0 || T < 1 || Hg < 1 || W < 1 || ct < 1 || ch < 1 || cw < 1) return VS_ERR_INVALID_ARG;
  if (static_cast<long long>(T) * Hg * W < S) return VS_ERR_INVALID_ARG;
  if (S == 0) return VS_OK;
  if (!perm) return VS_ERR_INVALID_ARG;
  long long i = 0;
  for (int t0 = 0; t0 < T; t0 += ct)
    for (int y0 = 0; y0 < Hg; y0 += ch)
      for (int x0 = 0; x0 < W; x0 += cw) {
        const int t1 = t0 + ct < T ? t0 + ct : T;
        const int y1 = y0 + ch < Hg ? y0 + ch : Hg;
        const int x1 = x0 + cw < W ? x0 + cw : W;
        for (int t = t0; t < t1; ++t)
          for (int y = y0; y < y1; ++y) {
            const long long row = (static_cast<long long>(t) * Hg + y) * W;
            if (row >= S) continue;
            for (int x = x0; x < x1; ++x)
              if (row + x < S) perm[i++] = static_cast<int32_t>(row + x);
          }
      }
  return i == S ? VS_OK : VS_ERR_INVALID_ARG;
}

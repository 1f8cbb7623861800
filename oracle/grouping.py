"""Static spatiotemporal-cube grouping of video tokens.

Test infrastructure (see ``oracle/__init__``).

VC-Attention summary ("Main Findings"): block demeaning pays only when the
tokens of a block are alike; besides sequence order and k-means grouping the
page measures a *static spatiotemporal cube* ordering, in which the tokens of
a video latent's T x H x W grid are regrouped so that each hardware block
holds one small space-time cube (it removes more block energy than sequence
order, far less than k-means).  Being fixed by the grid, it costs nothing per
call and can be reused across calls, as can any permutation (the page's
grouping schedule reuses k-means permutations across adjacent denoising
steps, Key Contribution 3).

The page fixes neither the cube's extent nor the order of cubes.  Reading:

* token s of the sequence sits at grid position (t, y, x) in raster order,
  s = (t * H + y) * W + x; a grid larger than the sequence (T H W >= S) is
  truncated, i.e. positions s >= S hold no token;
* cubes of ct x ch x cw positions tile the grid from the origin (the last
  cube along an axis may be shorter), and are visited in raster order of the
  cube grid; within a cube, tokens in raster order;
* the permutation lists the tokens s < S in that visiting order:
  perm[i] = the token at position i of the grouped sequence.

Defined here as a sort: key of token s = (cube index along t, y, x, then
t, y, x), stable lexicographic order of the keys.  Pinned by
tests/test_oracle_grouping.py (a hand-enumerated case, closed-form
properties: bijection, cubes contiguous and compact, identities at the two
extreme cube sizes).
"""
import numpy as np


def cube_permutation(S: int, grid, cube) -> np.ndarray:
    """perm (int64 [S]) grouping the tokens of a T x H x W raster grid
    (truncated to S tokens) into ct x ch x cw cubes."""
    T, Hg, W = (int(a) for a in grid)
    ct, ch, cw = (int(a) for a in cube)
    if min(T, Hg, W, ct, ch, cw) < 1 or T * Hg * W < S or S < 0:
        raise ValueError("bad grid / cube")
    s = np.arange(S, dtype=np.int64)
    t, rem = np.divmod(s, Hg * W)
    y, x = np.divmod(rem, W)
    # np.lexsort sorts by the last key first
    return np.lexsort((x, y, t, x // cw, y // ch, t // ct)).astype(np.int64)


"""Pins of the static spatiotemporal-cube grouping (oracle/grouping.py) and of
the pipeline with a given permutation, from the definition and closed-form
properties."""
import numpy as np
import pytest

from oracle import attention, grouping, pipeline


def test_hand_enumerated_case():
    # grid T=2, H=2, W=4 (raster s = 8t + 4y + x), cubes 1 x 2 x 2: per time
    # step the left 2x2 square (x 0-1), then the right one (x 2-3)
    got = grouping.cube_permutation(16, (2, 2, 4), (1, 2, 2))
    want = [0, 1, 4, 5, 2, 3, 6, 7, 8, 9, 12, 13, 10, 11, 14, 15]
    assert got.tolist() == want
    # cubes 2 x 1 x 2: the two frames of each 1 x 2 strip together
    got = grouping.cube_permutation(16, (2, 2, 4), (2, 1, 2))
    want = [0, 1, 8, 9, 2, 3, 10, 11, 4, 5, 12, 13, 6, 7, 14, 15]
    assert got.tolist() == want


def test_truncated_grid_and_ragged_cubes():
    # T=1, H=3, W=3, cubes 1 x 2 x 2, only 8 of the 9 positions hold tokens
    got = grouping.cube_permutation(8, (1, 3, 3), (1, 2, 2))
    # cube (0,0): 0 1 3 4; cube (0,1): 2 5; cube (1,0): 6 7; cube (1,1): (8 absent)
    assert got.tolist() == [0, 1, 3, 4, 2, 5, 6, 7]


@pytest.mark.parametrize("grid,cube,S", [((20, 48, 34), (2, 8, 8), 32626),
                                         ((5, 12, 10), (2, 4, 4), 600),
                                         ((3, 7, 5), (2, 3, 2), 100)])
def test_bijection_and_compact_cubes(grid, cube, S):
    perm = grouping.cube_permutation(S, grid, cube)
    assert np.array_equal(np.sort(perm), np.arange(S))
    T, Hg, W = grid
    t, rem = np.divmod(perm, Hg * W)
    y, x = np.divmod(rem, W)
    key = (t // cube[0]) * 10**8 + (y // cube[1]) * 10**4 + (x // cube[2])
    # cube index never decreases, and each cube's tokens are one contiguous run
    cube_id = (t // cube[0], y // cube[1], x // cube[2])
    lin = (cube_id[0] * ((Hg + cube[1] - 1) // cube[1]) + cube_id[1]) * ((W + cube[2] - 1) // cube[2]) + cube_id[2]
    assert np.all(np.diff(lin) >= 0)
    assert len(np.unique(key)) == np.count_nonzero(np.diff(lin)) + 1
    # within a cube, raster order
    same = np.diff(lin) == 0
    assert np.all(np.diff(perm)[same] > 0)


def test_full_cubes_fill_whole_blocks():
    # grid dims multiples of a 2 x 8 x 8 = 128-token cube, no truncation: each
    # 128-token block is exactly one cube (extent 2 x 8 x 8 in t, y, x)
    grid = (4, 16, 24)
    S = 4 * 16 * 24
    perm = grouping.cube_permutation(S, grid, (2, 8, 8))
    for j in range(0, S, 128):
        blk = perm[j:j + 128]
        t, rem = np.divmod(blk, 16 * 24)
        y, x = np.divmod(rem, 24)
        assert np.ptp(t) == 1 and np.ptp(y) == 7 and np.ptp(x) == 7
        assert len(set(zip(t.tolist(), y.tolist(), x.tolist()))) == 128


def test_identity_cases():
    S = 5 * 6 * 7
    assert np.array_equal(grouping.cube_permutation(S, (5, 6, 7), (1, 1, 1)), np.arange(S))
    assert np.array_equal(grouping.cube_permutation(S, (5, 6, 7), (5, 6, 7)), np.arange(S))
    # cubes spanning whole rows (1 x 1 x W): raster order again
    assert np.array_equal(grouping.cube_permutation(S - 3, (5, 6, 7), (1, 1, 7)), np.arange(S - 3))


def test_bad_arguments():
    with pytest.raises(ValueError):
        grouping.cube_permutation(100, (2, 3, 4), (1, 1, 1))     # grid too small
    with pytest.raises(ValueError):
        grouping.cube_permutation(10, (2, 3, 4), (0, 1, 1))


def test_pipeline_with_a_given_permutation():
    """A given permutation takes the same route as the k-means one: with the
    k-means permutation passed in, every output is identical; with a cube
    permutation O stays in query order (its error against FP64 dense
    attention is that of the quantized path, not of a row shuffle)."""
    rng = np.random.default_rng(5)
    S, D = 300, 64
    q, k, v = (rng.standard_normal((S, D)).astype(np.float32) for _ in range(3))
    km = pipeline.smoothed_attention_head(q, k, v, kmeans_kt=(4, 2))
    given = pipeline.smoothed_attention_head(q, k, v, perm=km["perm"])
    for name in ("q_codes", "k_codes", "v_codes", "k_scale", "v_scale", "k_mean", "v_mean",
                 "O", "lse2"):
        np.testing.assert_array_equal(given[name], km[name], err_msg=name)
    perm = grouping.cube_permutation(S, (3, 10, 10), (1, 4, 4))
    out = pipeline.smoothed_attention_head(q, k, v, perm=perm)
    ref_o, ref_l = attention.dense_attention(q, k, v, pipeline.default_scale(D))
    e = pipeline.error_report(out["O"], ref_o)["rel_l2"]
    e_seq = pipeline.error_report(pipeline.smoothed_attention_head(q, k, v)["O"], ref_o)["rel_l2"]
    e_shuf = pipeline.error_report(out["O"][perm], ref_o)["rel_l2"]
    assert e < 1.5 * e_seq and e_shuf > 10 * e, (e, e_seq, e_shuf)
    assert np.array_equal(out["perm"], perm)
    with pytest.raises(ValueError):
        pipeline.smoothed_attention_head(q, k, v, perm=np.zeros(S, dtype=np.int64))
    with pytest.raises(ValueError):
        pipeline.smoothed_attention_head(q, k, v, perm=perm, kmeans_kt=(4, 2))

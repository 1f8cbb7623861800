"""Pins of the QK Hadamard rotation (oracle/smoothing.hadamard_rows_f32) and
of the pipeline with it, from the definition of the Sylvester matrix and the
algebra of the rotation."""
import math

import numpy as np
import pytest

from oracle import attention, pipeline, smoothing


def _sylvester(D):
    h = np.array([[1.0]])
    while h.shape[0] < D:
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    return h


@pytest.mark.parametrize("D", [2, 8, 64, 128])
def test_butterfly_equals_the_kronecker_definition(D):
    rng = np.random.default_rng(D)
    # small integers: every partial sum is exact in float32
    x = rng.integers(-50, 50, size=(37, D)).astype(np.float32)
    np.testing.assert_array_equal(smoothing.hadamard_rows_f32(x), x.astype(np.float64) @ _sylvester(D))
    # unit vectors give the rows of H
    np.testing.assert_array_equal(smoothing.hadamard_rows_f32(np.eye(D, dtype=np.float32)), _sylvester(D))


def test_orthogonality_and_float32_error():
    D = 128
    H = _sylvester(D)
    np.testing.assert_array_equal(H @ H.T, D * np.eye(D))
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, D)).astype(np.float32)
    twice = smoothing.hadamard_rows_f32(smoothing.hadamard_rows_f32(x)).astype(np.float64)
    np.testing.assert_allclose(twice, D * x.astype(np.float64), rtol=0, atol=1e-3)
    # 7 rounded stages: within 7 float32 half-ulps of the row's magnitude sum
    exact = x.astype(np.float64) @ H
    bound = 7 * 2.0 ** -24 * np.abs(x).sum(axis=1, keepdims=True) * 2
    assert np.all(np.abs(smoothing.hadamard_rows_f32(x) - exact) <= bound)


def test_rotation_leaves_the_score_product_unchanged():
    """(q H / D)(k H)^T = q k^T: the rotated, centred operands give the same
    scores, so FP64 attention on them equals attention on the originals."""
    rng = np.random.default_rng(2)
    S, D = 200, 64
    q, k, v = (rng.standard_normal((S, D)) for _ in range(3))
    H = _sylvester(D)
    o1, l1 = attention.dense_attention(q, k, v, 1.0 / math.sqrt(D))
    o2, l2 = attention.dense_attention(q @ H / D, k @ H, v, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-11)


def test_prescaled_queries_fold_one_over_d_into_c():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((10, 128)).astype(np.float32)
    c = smoothing.score_constant(np.float32(1 / math.sqrt(128)))
    got = smoothing.hadamard_prescale_queries(q, c)
    want = smoothing.hadamard_rows_f32(q) * np.float32(c / np.float32(128))
    np.testing.assert_array_equal(got, want.astype(np.float32))
    with pytest.raises(ValueError):
        smoothing.hadamard_rows_f32(np.zeros((2, 96), dtype=np.float32))


def test_pipeline_with_the_rotation_stays_close_to_dense():
    """End to end the rotation only moves the quantization error (the pages:
    at most 0.1-0.3 dB PSNR); a dropped 1/D or a rotation of Q alone would
    change the scores by far more."""
    rng = np.random.default_rng(4)
    S, D = 256, 128
    q, k, v = (rng.standard_normal((S, D)).astype(np.float32) for _ in range(3))
    k += 3.0 * rng.standard_normal(D).astype(np.float32)
    ref, ref_l = attention.dense_attention(q, k, v, pipeline.default_scale(D))
    base = pipeline.smoothed_attention_head(q, k, v)
    rot = pipeline.smoothed_attention_head(q, k, v, qk_hadamard=True)
    eb = pipeline.error_report(base["O"], ref)["rel_l2"]
    er = pipeline.error_report(rot["O"], ref)["rel_l2"]
    assert er < 2 * eb and eb < 2 * er, (eb, er)
    np.testing.assert_allclose(rot["lse2"], ref_l, rtol=0, atol=0.05)
    # the rotated codes differ from the plain ones
    assert not np.array_equal(rot["k_codes"], base["k_codes"])

"""Pins of the oracle's statistics and per-block quantizers."""
from fractions import Fraction
import json
import os

import numpy as np
import torch

from oracle import e4m3, smoothing

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages.json")))


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def test_exact_mean_is_the_rational_mean_rounded_once():
    rng = np.random.default_rng(0)
    x = _bf16(rng.standard_normal((37, 5)) * 2.0 ** rng.integers(-20, 20, (37, 5)))
    got = smoothing.exact_mean_f32(x)
    for d in range(5):
        exact = sum(Fraction(float(t)) for t in x[:, d]) / 37
        assert got[d] == np.float32(float(exact))


def test_block_means_cover_ragged_last_block():
    rng = np.random.default_rng(1)
    v = _bf16(rng.standard_normal((300, 8)))
    bm = smoothing.v_block_means(v)
    assert bm.shape == (3, 8)
    np.testing.assert_array_equal(bm[2], smoothing.exact_mean_f32(v[256:300]))
    np.testing.assert_array_equal(bm[0], smoothing.exact_mean_f32(v[:128]))


def test_zero_block_uses_unit_scale():
    x = np.zeros((130, 16), dtype=np.float32)
    x[128:] = 1.0
    codes, scale = smoothing.quantize_blocks(x)
    assert scale[0] == 1.0 and np.all(codes[:128] == 0)
    # amax 1 -> scale 2^-8 (1 <= 448/256 and 1 > 448/512): code of 256
    assert scale[1] == 2.0 ** -8 and np.all(codes[128:130] == 0x78)


def test_centring_removes_the_sequence_mean():
    rng = np.random.default_rng(3)
    k = _bf16(rng.standard_normal((1000, 32)) + 3.0 * rng.standard_normal(32))
    mu = smoothing.k_seq_mean(k)
    kc = smoothing.centre(k, mu)
    # residual mean is at float32 rounding level of the data, far below its spread
    assert np.all(np.abs(kc.astype(np.float64).mean(axis=0)) < 1e-5)


def test_smoothing_reduces_quantization_error_direction():
    """TeleFuser PR #40's accuracy table reports lower quantized-K MSE, lower
    dequantized-V MSE and a far lower dequantized-V-mean MSE with smoothing.
    Synthetic K/V with channel offsets and outlier rows must show the same
    direction (the magnitudes are not comparable)."""
    g = GOLDEN["smoothing_accuracy_direction"]
    assert g["quanted_k_mse"][1] < g["quanted_k_mse"][0]
    rng = np.random.default_rng(4)
    S, D = 2048, 64
    k = _bf16(rng.standard_normal((S, D)) + 3.0 * rng.standard_normal(D))
    v = rng.standard_normal((S, D)) + 2.0 * rng.standard_normal(D)
    v[rng.choice(S, 10, replace=False)] *= 20
    v = _bf16(v)

    def k_err(x, mean):
        codes, sc = smoothing.quantize_blocks(x)
        rec = smoothing.dequantize_blocks(codes, sc, S) + (0 if mean is None else mean)
        return np.mean((rec - k) ** 2)
    mu = smoothing.k_seq_mean(k)
    assert k_err(smoothing.centre(k, mu), mu.astype(np.float64)) < k_err(k, None)

    bm = smoothing.v_block_means(v)
    rcodes, rsc = smoothing.quantize_blocks(smoothing.residual_blocks(v, bm))
    rec_s = smoothing.dequantize_blocks(rcodes, rsc, S) + bm[np.arange(S) // 128]
    vcodes, vsc = smoothing.quantize_blocks(v)
    rec_u = smoothing.dequantize_blocks(vcodes, vsc, S)
    assert np.mean((rec_s - v) ** 2) < np.mean((rec_u - v) ** 2)
    # the mean the attention sees: smoothed, the FP32 block mean carried
    # outside the FP8 codes; unsmoothed, the mean of the dequantized values
    true_means = np.stack([v[j:j + 128].astype(np.float64).mean(0) for j in range(0, S, 128)])
    err_mean_s = np.mean((bm - true_means) ** 2)
    err_mean_u = np.mean((np.stack([rec_u[j:j + 128].mean(0) for j in range(0, S, 128)]) - true_means) ** 2)
    assert err_mean_s < 1e-6 * err_mean_u


def test_q_log2_offset_is_the_row_shift_of_centring():
    rng = np.random.default_rng(5)
    q = _bf16(rng.standard_normal((7, 16)))
    k = _bf16(rng.standard_normal((50, 16)) + 2.0)
    mu = smoothing.k_seq_mean(k)
    c = smoothing.score_constant(0.25)
    off = smoothing.q_log2_offset(q, mu, c)
    z = float(c) * (q.astype(np.float64) @ k.T.astype(np.float64))
    zc = float(c) * (q.astype(np.float64) @ (k.astype(np.float64) - mu.astype(np.float64)).T)
    np.testing.assert_allclose(z - zc, np.repeat(off[:, None], 50, axis=1), rtol=0, atol=1e-12)


def test_pow2_scale_is_the_smallest_fitting_power_of_two():
    """Block scale 2^e: the smallest power of two with amax <= 448 2^e, the
    block maximum's code in (224, 448], every value within half an E4M3 step,
    padding rows code 0."""
    rng = np.random.default_rng(6)
    for amax in [1e-30, 0.3, 1.0, 447.0, 448.0, 448.5, 896.0, 897.0, 3e5]:
        e = smoothing.pow2_exponent(np.float32(amax))
        assert amax <= 448 * 2.0 ** e and (e == -126 or amax > 448 * 2.0 ** (e - 1))
    assert smoothing.pow2_exponent(0.0) == 0
    x = (rng.standard_normal((300, 32)) * rng.uniform(0.01, 50, (300, 1))).astype(np.float32)
    codes, scale = smoothing.quantize_blocks(x)
    for j in range(3):
        xb = x[j * 128:min(300, (j + 1) * 128)]
        e = np.log2(float(scale[j]))
        assert e == np.round(e)                                    # a power of two
        m = np.abs(e4m3.decode(codes[j * 128:j * 128 + len(xb)])).max()
        assert 224 < m <= 448                                      # the max lands in (224, 448]
        assert scale[j] == np.float32(2.0 ** smoothing.pow2_exponent(np.abs(xb).max()))
        rec = e4m3.decode(codes[j * 128:j * 128 + len(xb)]) * float(scale[j])
        y = np.abs(xb.astype(np.float64)) / float(scale[j])
        assert np.all(np.abs(rec - xb) <= e4m3.ulp_half(y) * float(scale[j]) * 1.0000001)
    assert np.all(codes[300:] == 0)

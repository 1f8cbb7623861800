"""Pins of the oracle's rotary embedding (VC-Attention summary, Key
Contribution 3: the rotation belongs to the fused prologue): the bf16
rounding against PyTorch's own float32 -> bfloat16 conversion, the rotation
against its definition as complex multiplication, the special angles, the
relative-position property of the rotated dot products, and the pipeline
with the rotation fused equal to the pipeline on pre-rotated inputs."""
import math

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, pipeline, smoothing


def test_bf16_rounding_equals_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-30, 30, 200000)).astype(np.float32)
    # exact ties between two bf16 values (both parities of the kept bit)
    base = rng.standard_normal(2000).astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1.0, 3.0e38])])
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(smoothing.round_bf16(x), want)


def _tables(S, D, seed=1):
    rng = np.random.default_rng(seed)
    ang = rng.uniform(-50, 50, (S, D // 2))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32), ang


def test_rotation_is_complex_multiplication_within_rounding():
    """(y_2i + i y_2i+1) = (x_2i + i x_2i+1) (cos + i sin): the oracle's
    bf16 result is within half a bf16 step of the exact float64 rotation of
    the same inputs and tables (plus the float32 rounding of the products)."""
    S, D = 500, 128
    rng = np.random.default_rng(2)
    x = smoothing.round_bf16(rng.standard_normal((S, D)).astype(np.float32) * 3)
    c, s, _ = _tables(S, D)
    z = (x[:, 0::2].astype(np.float64) + 1j * x[:, 1::2]) * (c.astype(np.float64) + 1j * s)
    exact = np.empty((S, D))
    exact[:, 0::2], exact[:, 1::2] = z.real, z.imag
    y = smoothing.rope_rows_bf16(x, c, s).astype(np.float64)
    # float32 rounding of the two products and of their sum, relative to the
    # products (they may cancel), then half a bf16 step of the result
    a, b = np.abs(x[:, 0::2]).astype(np.float64), np.abs(x[:, 1::2]).astype(np.float64)
    ac, as_ = np.abs(c).astype(np.float64), np.abs(s).astype(np.float64)
    f32err = np.empty((S, D))
    f32err[:, 0::2] = f32err[:, 1::2] = 3 * 2.0 ** -24 * (a * np.maximum(ac, as_) + b * np.maximum(ac, as_))
    mag = np.maximum(np.abs(y), np.abs(exact)).astype(np.float32)
    half_bf16 = np.spacing(mag).astype(np.float64) * 2 ** 15
    assert np.all(np.abs(y - exact) <= half_bf16 + f32err)
    # and the rotation really rotates: pair norms kept to bf16 precision
    n0 = x[:, 0::2].astype(np.float64) ** 2 + x[:, 1::2].astype(np.float64) ** 2
    n1 = y[:, 0::2] ** 2 + y[:, 1::2] ** 2
    np.testing.assert_allclose(n1, n0, rtol=2 * 2.0 ** -8, atol=1e-30)


def test_special_angles():
    S, D = 64, 64
    rng = np.random.default_rng(3)
    x = smoothing.round_bf16(rng.standard_normal((S, D)).astype(np.float32))
    one, zero = np.ones((S, D // 2), np.float32), np.zeros((S, D // 2), np.float32)
    np.testing.assert_array_equal(smoothing.rope_rows_bf16(x, one, zero), x)     # angle 0
    y = smoothing.rope_rows_bf16(x, zero, one)                                   # angle pi/2
    np.testing.assert_array_equal(y[:, 0::2], -x[:, 1::2])
    np.testing.assert_array_equal(y[:, 1::2], x[:, 0::2])


def test_rotated_scores_depend_on_relative_position():
    """1D RoPE: the dot product of query position m and key position n
    depends on m - n only (to bf16 precision of the rotated vectors)."""
    D, L = 64, 40
    inv = 10000.0 ** (-np.arange(D // 2) * 2.0 / D)
    pos = np.arange(L)
    ang = pos[:, None] * inv[None, :]
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    rng = np.random.default_rng(4)
    qv = smoothing.round_bf16(rng.standard_normal(D).astype(np.float32))
    kv = smoothing.round_bf16(rng.standard_normal(D).astype(np.float32))
    qr = smoothing.rope_rows_bf16(np.repeat(qv[None], L, 0), c, s).astype(np.float64)
    kr = smoothing.rope_rows_bf16(np.repeat(kv[None], L, 0), c, s).astype(np.float64)
    for d in (0, 3, 11):
        vals = [qr[m] @ kr[m - d] for m in range(d, L)]
        assert np.ptp(vals) < 0.1 * np.sqrt(D) * 2 ** -6 * D ** 0.5
    assert abs(qr[20] @ kr[20] - qr[20] @ kr[9]) > 0.05            # positions matter


@pytest.mark.parametrize("D", [64, 128])
def test_pipeline_with_rope_equals_pipeline_on_rotated_inputs(D):
    """Rotation fused (rope=...) equals the same pipeline on inputs the
    oracle rotated beforehand, output for output (the rotation comes first
    and yields bf16 values either way)."""
    S = 700
    grid = (2, 16, 24)
    cos, sin = (t.numpy() for t in workloads.rope_tables_3d(S, D, grid))
    rng = np.random.default_rng(5)
    q = smoothing.round_bf16(rng.standard_normal((S, D)).astype(np.float32))
    k = smoothing.round_bf16((rng.standard_normal((S, D)) + 2.0).astype(np.float32))
    v = smoothing.round_bf16(rng.standard_normal((S, D)).astype(np.float32))
    rows = pipeline.sample_rows(S, 64)
    a = pipeline.smoothed_attention_head(q, k, v, rows=rows, rope=(cos, sin))
    b = pipeline.smoothed_attention_head(smoothing.rope_rows_bf16(q, cos, sin),
                                         smoothing.rope_rows_bf16(k, cos, sin), v, rows=rows)
    for key in ("O", "lse2", "q_codes", "k_codes", "k_mean", "q_off"):
        np.testing.assert_array_equal(a[key], b[key])
    # and it is attention of the rotated operands
    qr, kr = smoothing.rope_rows_bf16(q, cos, sin), smoothing.rope_rows_bf16(k, cos, sin)
    ref, _ = attention.dense_attention(qr[rows], kr, v, 1.0 / math.sqrt(D))
    assert pipeline.error_report(a["O"], ref)["rel_l2"] < 0.1

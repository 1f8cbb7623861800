"""Pins of the E2M1 codec and the MXFP4 block quantizer (oracle/fp4.py), from
the OCP format definition: exhaustive over the 16 codes and every midpoint."""
import numpy as np
import pytest

from oracle import fp4


def test_decode_table_from_the_format():
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert fp4.DECODE[:8].tolist() == want
    assert fp4.DECODE[8:].tolist() == [-v for v in want]
    assert np.signbit(fp4.DECODE[8])


def test_every_code_round_trips():
    for c in range(16):
        got = int(fp4.encode(fp4.DECODE[c]))
        assert got == c, (c, got)


def test_midpoints_round_to_the_even_code():
    vals = fp4.DECODE[:8]
    for i in range(7):
        mid = 0.5 * (vals[i] + vals[i + 1])
        even = i if i % 2 == 0 else i + 1
        assert int(fp4.encode(mid)) == even, mid
        assert int(fp4.encode(-mid)) == even + 8
        assert int(fp4.encode(np.nextafter(mid, 0))) == i
        assert int(fp4.encode(np.nextafter(mid, 10))) == i + 1


def test_saturation_and_nearest_by_brute_force():
    assert int(fp4.encode(7.0)) == 7 and int(fp4.encode(1e30)) == 7 and int(fp4.encode(-9.0)) == 15
    rng = np.random.default_rng(0)
    x = rng.uniform(-7, 7, 5000)
    c = fp4.encode(x)
    err = np.abs(fp4.decode(c) - np.clip(x, -6, 6))
    best = np.min(np.abs(np.abs(np.clip(x, -6, 6))[:, None] - fp4.DECODE[:8][None, :]), axis=1)
    np.testing.assert_allclose(err, best, rtol=0, atol=0)


def test_group_exponent_is_the_smallest_fitting_power_of_two():
    for amax in [6.0, 6.0000001, 3.0, 5.99, 0.75, 1e-30, 1e30]:
        e = fp4.group_exponent(amax)
        assert amax <= 6 * 2.0 ** e and (e == -127 or amax > 6 * 2.0 ** (e - 1))
    assert fp4.group_exponent(0.0) == 0
    assert fp4.group_exponent(6.0) == 0 and fp4.group_exponent(6.01) == 1


def test_block_quantizer_groups_error_and_padding():
    rng = np.random.default_rng(1)
    S, D = 300, 64
    r = (rng.standard_normal((S, D)) * rng.uniform(0.1, 10, D)).astype(np.float32)
    codes, exps = fp4.quantize_mxfp4(r)
    assert codes.shape == (384, D) and exps.shape == (12, D)
    assert np.all(codes[S:] == 0)
    deq = fp4.dequantize_mxfp4(codes, exps, S)
    for g in range(12):
        sl = slice(32 * g, min(S, 32 * g + 32))
        if sl.start >= S:
            continue
        amax = np.abs(r[sl]).max(axis=0)
        scale = 2.0 ** exps[g]
        # each group's largest entry lies in (3, 6] times its scale
        assert np.all(amax <= 6 * scale) and np.all((amax > 3 * scale) | (amax == 0))
        # error at most half the widest step (2 at the top of the range) times the scale
        assert np.all(np.abs(deq[sl] - r[sl]) <= scale * 1.0 + 1e-30)


def test_pipeline_with_mxfp4_v():
    """The MXFP4 V path: the same Q/K codes as the E4M3 path, V error of the
    4-bit order (well above E4M3's, well below no smoothing at all with a
    large V offset), and block demeaning helps it more than it helps E4M3."""
    from oracle import attention, pipeline
    rng = np.random.default_rng(2)
    S, D = 512, 64
    q, k = (rng.standard_normal((S, D)).astype(np.float32) for _ in range(2))
    v = (rng.standard_normal((S, D)) + 4.0 * rng.standard_normal(D)).astype(np.float32)
    ref, _ = attention.dense_attention(q, k, v, pipeline.default_scale(D))
    e8 = pipeline.smoothed_attention_head(q, k, v)
    f4 = pipeline.smoothed_attention_head(q, k, v, v_format="mxfp4")
    f4u = pipeline.smoothed_attention_head(q, k, v, v_format="mxfp4", smooth=False)
    np.testing.assert_array_equal(f4["k_codes"], e8["k_codes"])
    r8 = pipeline.error_report(e8["O"], ref)["rel_l2"]
    r4 = pipeline.error_report(f4["O"], ref)["rel_l2"]
    r4u = pipeline.error_report(f4u["O"], ref)["rel_l2"]
    assert r8 < r4 < r4u, (r8, r4, r4u)
    assert f4["v_exps"].shape == (16, D)
    with pytest.raises(ValueError):
        pipeline.smoothed_attention_head(q, k, v, v_format="nvfp4")

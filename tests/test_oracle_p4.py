"""Pins of the oracle's 4-bit probability tile (pcast "mxfp4"): the grouping
against a per-element brute force, a closed-form row, the cast's error
bound, and the identities the E4M3 cast also keeps (mean-restore shift, lse2
independent of the cast)."""
import math

import numpy as np
import pytest

from oracle import attention, e4m3, fp4, pipeline, smoothing


def test_group_exponents_match_the_scalar_rule():
    rng = np.random.default_rng(0)
    pow2 = 6.0 * 2.0 ** np.arange(-130, 12)
    a = np.concatenate([rng.random(3000) * 1e3, rng.random(500) * 1e-38, pow2,
                        np.nextafter(pow2, np.inf), np.nextafter(pow2, 0.0),
                        [0.0, 2.0 ** -149, 3.0, 6.0, 256.0]])
    got = fp4.group_exponents(a)
    want = np.array([fp4.group_exponent(x) for x in a])
    np.testing.assert_array_equal(got, want)


def _brute_mxfp4(p8):
    """Per row, per group of 32 consecutive keys, per element: scalar rule."""
    R, n = p8.shape
    vals = np.zeros((R, n))
    codes = np.zeros((R, n), dtype=np.uint8)
    for i in range(R):
        for g0 in range(0, n, 32):
            grp = [float(p8[i, t]) for t in range(g0, min(n, g0 + 32))]
            e = fp4.group_exponent(max(grp))
            for t, x in enumerate(grp):
                c = int(fp4.encode(np.array([x * 2.0 ** -e]))[0])
                codes[i, g0 + t] = c
                vals[i, g0 + t] = float(fp4.DECODE[c]) * 2.0 ** e
    return codes, vals


@pytest.mark.parametrize("n", [1, 31, 32, 33, 100, 128])
def test_probability_groups_match_a_per_element_brute_force(n):
    rng = np.random.default_rng(n)
    p8 = np.exp2(rng.uniform(-20, 8, (6, n))).astype(np.float32).astype(np.float64)
    p8[0, :] = 0.0                                   # an all-zero row
    codes, exps, vals = attention.mxfp4_probabilities(p8)
    bc, bv = _brute_mxfp4(p8)
    np.testing.assert_array_equal(codes, bc)
    np.testing.assert_array_equal(vals, bv)
    assert exps.shape == (6, (n + 31) // 32)


def test_closed_form_row():
    """One query, D = 1 keys k_t = s_t and q = 1 (c = 1): the row maximum is
    0, so p 2^8 = 2^(s + 8).  Group 0 holds 256, 128, 64, 32, 16, 8 (e = 6:
    256 <= 6 2^6, 256 > 6 2^5): in units of 2^6 they are 4, 2, 1, 0.5, 0.25
    (a tie between codes 0 and 1: the even code, 0) and 0.125 (0), so P~ 2^8
    = 256, 128, 64, 32, 0, 0.  Group 1 holds 2^-3 alone with zeros (e = -5,
    value 4 exactly).  O = sum P~ v / sum p (the float32 p before the cast)."""
    s = np.full(64, -np.inf)
    s[:6] = [0, -1, -2, -3, -4, -5]
    s[40] = -11
    valid = np.isfinite(s)
    k = np.where(valid, s, -1000.0)[:, None]        # exp2 underflows to 0 there
    v = np.arange(64, dtype=np.float64)[:, None] + 1.0
    o, lse2 = attention.tiled_attention(np.ones((1, 1)), 1.0, np.pad(k, ((0, 64), (0, 0))),
                                        np.ones(1), np.pad(v, ((0, 64), (0, 0))), np.ones(1),
                                        64, 1.0, pcast="mxfp4", fp32=False)
    p = np.where(valid, np.exp2(np.where(valid, s, 0.0)), 0.0)
    pt = np.zeros(64)
    pt[:4] = [1.0, 0.5, 0.25, 0.125]
    pt[40] = 2.0 ** -11
    np.testing.assert_allclose(o[0, 0], (pt * v[:, 0]).sum() / p.sum(), rtol=1e-14)
    np.testing.assert_allclose(lse2[0], math.log2(p.sum()), rtol=0, atol=1e-14)
    codes, exps, vals = attention.mxfp4_probabilities(np.exp2(np.where(valid, s, -1000.0) + 8)[None])
    assert list(exps[0]) == [6, -5]
    assert list(codes[0, :6]) == [6, 4, 2, 1, 0, 0] and codes[0, 40] == 6


def test_cast_error_bound():
    """Per element |P~ - p| 2^8 <= 2^e max(1/4, p 2^8 2^-e / 4) (half the E2M1
    spacing), so with exact operands each output channel moves by at most
    max|v| (1/4 + (8/3) sum_g amax_g / sum p 2^8) -- 2^e < amax_g / 3."""
    rng = np.random.default_rng(7)
    S, D = 500, 32
    q = rng.standard_normal((12, D)) * 2
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, D))
    scale = 1.0 / math.sqrt(D)
    c = scale / math.log(2.0)
    nb = (S + 127) // 128
    pad = nb * 128 - S
    kp, vp = np.pad(k, ((0, pad), (0, 0))), np.pad(v, ((0, pad), (0, 0)))
    o4, _, tr = attention.tiled_attention(q, 1.0, kp, np.ones(nb), vp, np.ones(nb), S, c,
                                          pcast="mxfp4", fp32=False, return_trace=True)
    od, _ = attention.dense_attention(q, k, v, scale)
    # rebuild each tile's p 2^8 from the traced maxima and check the per-element bound
    s_all = (q @ k.T) * c
    mfinal = tr["m"][-1]
    bound_terms = np.zeros(len(q))
    for j in range(nb):
        lo, hi = 128 * j, min(S, 128 * (j + 1))
        p8 = np.exp2(s_all[:, lo:hi] - tr["m"][j][:, None] + 8.0)
        codes, exps, vals = attention.mxfp4_probabilities(p8)
        e = np.repeat(exps, 32, axis=1)[:, :hi - lo]
        assert np.all(np.abs(vals - p8) <= np.exp2(e) * np.maximum(0.25, p8 * np.exp2(-e) / 4)
                      + 1e-12)
        amax = np.pad(p8, ((0, 0), (0, 32 * exps.shape[1] - (hi - lo)))).reshape(
            len(q), -1, 32).max(axis=2)
        bound_terms += (amax * np.exp2(tr["m"][j] - mfinal)[:, None]).sum(axis=1)
    l8 = np.exp2(s_all - mfinal[:, None] + 8.0).sum(axis=1)
    err = np.abs(o4 - od)
    vmax = np.abs(v).max(axis=0)
    bound = (0.25 + (8.0 / 3.0) * bound_terms / l8)[:, None] * vmax[None, :]
    assert np.all(err <= bound + 1e-12)
    assert np.all(err.max(axis=1) > 0)


def _case(seed, S, D):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, D)).astype(np.float32) * 2
    k = rng.standard_normal((S, D)).astype(np.float32)
    v = rng.standard_normal((S, D)).astype(np.float32) + 3.0
    c = smoothing.score_constant(np.float32(1.0 / math.sqrt(D)))
    bm = smoothing.v_block_means(v)
    qc, qs = smoothing.quantize_blocks(smoothing.prescale_queries(q, c))
    kcodes, ks = smoothing.quantize_blocks(smoothing.centre(k, smoothing.k_seq_mean(k)))
    vcodes, vs = smoothing.quantize_blocks(smoothing.residual_blocks(v, bm))
    rows = np.arange(0, S, 11)
    args = (e4m3.decode(qc[rows]), qs[rows // 128], e4m3.decode(kcodes), ks, e4m3.decode(vcodes),
            vs, S, 1.0)
    return rng, args, bm, rows


def test_mean_restore_follows_a_shift_of_the_block_means():
    rng, args, bm, rows = _case(21, 450, 32)
    u = rng.standard_normal(bm.shape[1]) * 5
    o1, _ = attention.tiled_attention(*args, v_mean=bm, vmean_mode="block", pcast="mxfp4")
    o2, _ = attention.tiled_attention(*args, v_mean=bm + u[None, :], vmean_mode="block",
                                      pcast="mxfp4")
    np.testing.assert_allclose(o2 - o1, np.repeat(u[None], len(rows), 0), rtol=0, atol=1e-12)


def test_lse2_does_not_depend_on_the_4bit_cast():
    _, args, bm, _ = _case(22, 400, 64)
    o4, l4 = attention.tiled_attention(*args, v_mean=bm, vmean_mode="block", pcast="mxfp4")
    o8, l8 = attention.tiled_attention(*args, v_mean=bm, vmean_mode="block", pcast="e4m3")
    np.testing.assert_array_equal(l4, l8)
    assert np.max(np.abs(o4 - o8)) > 1e-3


def test_pipeline_p_format():
    rng = np.random.default_rng(23)
    S, D = 300, 64
    q, k, v = (rng.standard_normal((S, D)).astype(np.float32) for _ in range(3))
    a = pipeline.smoothed_attention_head(q, k, v, p_format="mxfp4", rows=np.arange(0, S, 7))
    b = pipeline.smoothed_attention_head(q, k, v, pcast="mxfp4", rows=np.arange(0, S, 7))
    np.testing.assert_array_equal(a["O"], b["O"])
    od, _ = attention.dense_attention(q[::7].astype(np.float64), k.astype(np.float64),
                                      v.astype(np.float64), 1.0 / math.sqrt(D))
    e8 = pipeline.smoothed_attention_head(q, k, v, rows=np.arange(0, S, 7))
    rel = np.linalg.norm(a["O"] - od) / np.linalg.norm(od)
    rel8 = np.linalg.norm(e8["O"] - od) / np.linalg.norm(od)
    # coarser than the E4M3 tile on these unit-variance inputs, still close
    assert rel8 < rel < 0.3, (rel8, rel)
    with pytest.raises(ValueError):
        pipeline.smoothed_attention_head(q, k, v, p_format="mxfp4", expcast=True)

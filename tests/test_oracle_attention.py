"""Pins of the oracle's attention: brute force, exact invariances, the E4M3
probability cast and the ExpCast-FP8 bound (Proposition 3.1)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, e4m3, smoothing

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages.json")))


def _brute_dense(q, k, v, scale):
    """Softmax attention with Python loops and math.exp (tiny shapes)."""
    R, S = q.shape[0], k.shape[0]
    out = np.zeros((R, v.shape[1]))
    lse2 = np.zeros(R)
    for i in range(R):
        z = [scale * float(np.dot(q[i].astype(np.float64), k[t].astype(np.float64))) for t in range(S)]
        zm = max(z)
        w = [math.exp(x - zm) for x in z]
        den = sum(w)
        for t in range(S):
            out[i] += (w[t] / den) * v[t].astype(np.float64)
        lse2[i] = (zm + math.log(den)) / math.log(2.0)
    return out, lse2


def _no_cast(q, k, v, S, scale, **kw):
    """tiled_attention with raw float64 operands, unit scales, no P cast."""
    nb = (S + 127) // 128
    pad = nb * 128 - S
    kp = np.pad(k, ((0, pad), (0, 0)))
    vp = np.pad(v, ((0, pad), (0, 0)))
    c = scale / math.log(2.0)
    return attention.tiled_attention(q, 1.0, kp, np.ones(nb), vp, np.ones(nb), S, c,
                                     pcast="none", fp32=False, **kw)


@pytest.mark.parametrize("S", [1, 7, 128, 129, 300])
@pytest.mark.parametrize("D", [64, 128])
def test_dense_and_tiled_match_brute_force(S, D):
    rng = np.random.default_rng(S * 1000 + D)
    q = rng.standard_normal((5, D)) * 1.5
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, D))
    scale = 1.0 / math.sqrt(D)
    ob, lb = _brute_dense(q, k, v, scale)
    od, ld = attention.dense_attention(q, k, v, scale)
    np.testing.assert_allclose(od, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ld, lb, rtol=0, atol=1e-12)
    ot, lt = _no_cast(q, k, v, S, scale)
    np.testing.assert_allclose(ot, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lt, lb, rtol=0, atol=1e-12)


def test_k_centring_is_exact_for_softmax():
    rng = np.random.default_rng(1)
    S, D = 300, 64
    q = rng.standard_normal((9, D))
    k = rng.standard_normal((S, D)) + 5.0 * rng.standard_normal(D)
    v = rng.standard_normal((S, D))
    scale = 1.0 / math.sqrt(D)
    od, ld = attention.dense_attention(q, k, v, scale)
    mu = k.mean(axis=0)
    q_off = (scale / math.log(2.0)) * (q @ mu)
    ot, lt = _no_cast(q, k - mu, v, S, scale, q_off=q_off)
    np.testing.assert_allclose(ot, od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lt, ld, rtol=0, atol=1e-12)
    # without the offset the lse2 is that of the centred logits, not the original
    _, lt0 = _no_cast(q, k - mu, v, S, scale)
    assert np.max(np.abs(lt0 - ld)) > 1e-3


@pytest.mark.parametrize("mode", ["block", "seq"])
def test_v_mean_restore_identity(mode):
    """P(V - mu) + mu 1^T-weighted by the row sums = PV."""
    rng = np.random.default_rng(2)
    S, D = 300, 32
    q = rng.standard_normal((6, D))
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, D)) + 4.0 + np.linspace(0, 3, S)[:, None]
    scale = 1.0 / math.sqrt(D)
    od, _ = attention.dense_attention(q, k, v, scale)
    if mode == "block":
        means = np.stack([v[j:j + 128].mean(0) for j in range(0, S, 128)])
        r = v - means[np.arange(S) // 128]
    else:
        means = v.mean(0)
        r = v - means
    ot, _ = _no_cast(q, k, r, S, scale, v_mean=means, vmean_mode=mode)
    np.testing.assert_allclose(ot, od, rtol=0, atol=1e-12)
    # dropping the restore term is visibly wrong
    on, _ = _no_cast(q, k, r, S, scale)
    assert np.max(np.abs(on - od)) > 1.0


def test_joint_permutation_invariance():
    rng = np.random.default_rng(3)
    S, D = 300, 64
    q = rng.standard_normal((8, D))
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, D))
    perm = rng.permutation(S)
    scale = 1.0 / math.sqrt(D)
    o1, l1 = _no_cast(q, k, v, S, scale)
    o2, l2 = _no_cast(q, k[perm], v[perm], S, scale)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)
    # permuting only K is not invariant
    o3, _ = _no_cast(q, k[perm], v, S, scale)
    assert np.max(np.abs(o3 - o1)) > 1e-2


def _quantized_case(rng, S, D, q, k, v, smooth=True):
    """Quantized operands as the pipeline forms them: c folded into Q, so the
    score constant handed to the recurrence is 1."""
    c = smoothing.score_constant(np.float32(1.0 / math.sqrt(D)))
    kc = smoothing.centre(k, smoothing.k_seq_mean(k)) if smooth else k
    bm = smoothing.v_block_means(v)
    r = smoothing.residual_blocks(v, bm) if smooth else v
    qc, qs = smoothing.quantize_blocks(smoothing.prescale_queries(q, c))
    kcodes, ks = smoothing.quantize_blocks(kc)
    vcodes, vs = smoothing.quantize_blocks(r)
    return 1.0, qc, qs, kcodes, ks, vcodes, vs, bm


def test_constant_v_is_returned_exactly_with_block_mean_restore():
    rng = np.random.default_rng(4)
    S, D = 300, 64
    q = rng.standard_normal((S, D)).astype(np.float32)
    k = rng.standard_normal((S, D)).astype(np.float32)
    const = rng.standard_normal(D).astype(np.float32) * 3
    v = np.repeat(const[None, :], S, axis=0)
    c, qc, qs, kcodes, ks, vcodes, vs, bm = _quantized_case(rng, S, D, q, k, v)
    assert np.all(vcodes == 0)
    rows = np.arange(0, S, 17)
    o, _ = attention.tiled_attention(e4m3.decode(qc[rows]), qs[rows // 128], e4m3.decode(kcodes), ks,
                                     e4m3.decode(vcodes), vs, S, c, v_mean=bm, vmean_mode="block")
    np.testing.assert_allclose(o, np.repeat(const[None].astype(np.float64), len(rows), 0), rtol=0, atol=1e-12)


def test_equal_scores_give_the_mean_of_dequantized_v():
    """All keys identical: every score of a row equals the row maximum, so
    every p is exactly 1, every code is 0x78, O is the plain average of the
    dequantized V rows, and lse2 = s + log2 S exactly (the row sum adds the
    float32 p, here all 1)."""
    rng = np.random.default_rng(5)
    S, D = 300, 64
    q = rng.standard_normal((S, D)).astype(np.float32)
    k = np.repeat(rng.standard_normal((1, D)).astype(np.float32), S, axis=0)
    v = (rng.standard_normal((S, D)) * 2 + 1).astype(np.float32)
    c, qc, qs, kcodes, ks, vcodes, vs, bm = _quantized_case(rng, S, D, q, k, v, smooth=False)
    rows = np.arange(0, S, 13)
    o, lse2, tr = attention.tiled_attention(e4m3.decode(qc[rows]), qs[rows // 128], e4m3.decode(kcodes), ks,
                                            e4m3.decode(vcodes), vs, S, c, return_trace=True)
    for codes in tr["codes"]:
        assert np.all(codes == 0x78)
    srow = np.array([float(np.float32(sum(float(a) * float(b) for a, b in
                                          zip(e4m3.decode(qc[i]), e4m3.decode(kcodes[0])))
                                      * float(qs[i // 128]) * float(ks[0]))) for i in rows])
    deq = smoothing.dequantize_blocks(vcodes, vs, S)
    np.testing.assert_allclose(o, np.repeat(deq.mean(0)[None], len(rows), 0), rtol=1e-14, atol=0)
    np.testing.assert_allclose(lse2, srow + math.log2(S), rtol=0, atol=1e-12)


def test_score_is_the_exact_dot_product():
    """The recurrence's float64 score of decoded E4M3 operands equals the
    rational sum of the products (Fraction arithmetic), over codes spanning
    the whole E4M3 range, subnormals included; with fp32 it is that value
    rounded once to float32."""
    from fractions import Fraction
    rng = np.random.default_rng(11)
    D = 128
    codes = np.arange(256)
    finite = codes[~np.isnan(e4m3.DECODE)]
    qc = rng.choice(finite, size=(4, D)).astype(np.uint8)
    kc = rng.choice(finite, size=(128, D)).astype(np.uint8)
    qv, kv = e4m3.decode(qc), e4m3.decode(kc)
    _, _, tr = attention.tiled_attention(qv, 1.0, kv, np.ones(1), np.zeros((128, 1)), np.ones(1),
                                         128, 1.0, pcast="none", fp32=False, return_trace=True)
    exact = np.array([[float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv[i], kv[t])))
                       for t in range(128)] for i in range(4)])
    got = qv @ kv.T
    assert np.array_equal(got, exact)
    # the traced row maximum is the maximum of those exact scores
    np.testing.assert_array_equal(tr["m"][0], exact.max(axis=1))
    _, _, tr32 = attention.tiled_attention(qv, 1.0, kv, np.ones(1), np.zeros((128, 1)), np.ones(1),
                                           128, 1.0, pcast="none", fp32=True, return_trace=True)
    np.testing.assert_array_equal(tr32["m"][0], exact.max(axis=1).astype(np.float32))


def test_row_maximum_gets_code_0x78():
    """The running maximum is the row maximum itself: in the tile holding a
    row's largest score that key has p = 1 exactly, i.e. E4M3(2^8) = 0x78,
    and no code of the row exceeds 0x78."""
    rng = np.random.default_rng(12)
    S, D = 700, 64
    q = rng.standard_normal((S, D)).astype(np.float32) * 2
    k = rng.standard_normal((S, D)).astype(np.float32)
    v = rng.standard_normal((S, D)).astype(np.float32)
    c, qc, qs, kcodes, ks, vcodes, vs, bm = _quantized_case(rng, S, D, q, k, v)
    rows = np.arange(0, S, 7)
    _, _, tr = attention.tiled_attention(e4m3.decode(qc[rows]), qs[rows // 128], e4m3.decode(kcodes), ks,
                                         e4m3.decode(vcodes), vs, S, c, v_mean=bm,
                                         vmean_mode="block", return_trace=True)
    codes = attention.p_codes_row_major(tr, S)
    qd = e4m3.decode(qc[rows]) * qs[rows // 128, None].astype(np.float64)
    sc = qd @ smoothing.dequantize_blocks(kcodes, ks, S).T
    arg = sc.argmax(axis=1)
    assert np.all(codes[np.arange(len(rows)), arg] == 0x78)
    assert codes.max() == 0x78


def test_lse2_does_not_depend_on_the_e4m3_cast():
    """The row sum adds the float32 p before the cast (ExpCast off), so the
    lse2 with the E4M3 cast equals that with no cast bit for bit, while O
    differs."""
    rng = np.random.default_rng(13)
    S, D = 500, 64
    q = rng.standard_normal((S, D)).astype(np.float32) * 2
    k = rng.standard_normal((S, D)).astype(np.float32)
    v = rng.standard_normal((S, D)).astype(np.float32)
    c, qc, qs, kcodes, ks, vcodes, vs, bm = _quantized_case(rng, S, D, q, k, v)
    rows = np.arange(0, S, 5)
    args = (e4m3.decode(qc[rows]), qs[rows // 128], e4m3.decode(kcodes), ks, e4m3.decode(vcodes),
            vs, S, c)
    o1, l1 = attention.tiled_attention(*args, v_mean=bm, vmean_mode="block", pcast="e4m3")
    o0, l0 = attention.tiled_attention(*args, v_mean=bm, vmean_mode="block", pcast="none")
    np.testing.assert_array_equal(l1, l0)
    assert np.max(np.abs(o1 - o0)) > 1e-4


@pytest.mark.parametrize("pcast", ["e4m3", "expcast"])
def test_mean_restore_follows_a_shift_of_the_block_means(pcast):
    """The rank-one term and l take the same tile row sum, so shifting every
    block mean by a vector u (residuals unchanged) shifts O by exactly u,
    whatever the probability cast."""
    rng = np.random.default_rng(14)
    S, D = 600, 32
    q = rng.standard_normal((S, D)).astype(np.float32) * 2
    k = rng.standard_normal((S, D)).astype(np.float32)
    v = rng.standard_normal((S, D)).astype(np.float32) + 3.0
    c, qc, qs, kcodes, ks, vcodes, vs, bm = _quantized_case(rng, S, D, q, k, v)
    rows = np.arange(0, S, 9)
    args = (e4m3.decode(qc[rows]), qs[rows // 128], e4m3.decode(kcodes), ks, e4m3.decode(vcodes),
            vs, S, c)
    u = rng.standard_normal(D) * 5
    o1, _ = attention.tiled_attention(*args, v_mean=bm, vmean_mode="block", pcast=pcast)
    o2, _ = attention.tiled_attention(*args, v_mean=bm + u[None, :], vmean_mode="block",
                                      pcast=pcast)
    np.testing.assert_allclose(o2 - o1, np.repeat(u[None], len(rows), 0), rtol=0, atol=1e-12)


def test_e4m3_p_cast_error_is_bounded_by_the_values():
    """With exact operands, the E4M3 P cast (2^8 scale) changes each p by at
    most 2^-4 of itself (p >= 2^-14; below that by at most 2^-18), and O is
    sum_t P~_t v_t / sum_t p_t (the row sum adds the p before the cast, and
    the row maximum has p = 1), so each output channel moves by at most
    (2^-4 + S 2^-18) max_t |v_t|."""
    rng = np.random.default_rng(6)
    S, D = 700, 64
    q = rng.standard_normal((20, D)) * 2
    k = rng.standard_normal((S, D))
    v = rng.standard_normal((S, D))
    scale = 1.0 / math.sqrt(D)
    od, _ = attention.dense_attention(q, k, v, scale)
    nb = (S + 127) // 128
    pad = nb * 128 - S
    c = scale / math.log(2.0)
    oc, _ = attention.tiled_attention(q, 1.0, np.pad(k, ((0, pad), (0, 0))), np.ones(nb),
                                      np.pad(v, ((0, pad), (0, 0))), np.ones(nb), S, c,
                                      pcast="e4m3", fp32=False)
    err = np.abs(oc - od)
    vmax = np.abs(v).max(axis=0)
    assert np.all(err <= (2.0 ** -4 + S * 2.0 ** -18) * vmax[None, :])
    assert np.all(err.max(axis=1) > 0)          # the cast really happened


def test_golden_expcast_bound_matches_closed_form():
    g = GOLDEN["expcast_tv_bound"]
    assert abs(attention.EXPCAST_TV_BOUND - g["value"]) <= g["rounding"]
    # centring over the continuous mantissa instead would give 3.66%
    f = 1.0 / math.log(2.0) - 1.0
    sig_cont = 0.5 * (math.log2(1 + f) - f)
    e = sig_cont + 1 / 16
    assert abs((2 ** e - 1) / (2 ** e + 1) - g["value"]) > g["rounding"]
    assert abs(attention.K0 - (120 - 8 * attention.SIGMA)) < 1e-12
    assert attention.DELTA.argmax() == 4 and attention.DELTA.argmin() == 0


def _expcast_row(s):
    """ExpCast probabilities of one row of log2 scores through the oracle."""
    S = s.size
    D = 1
    nb = (S + 127) // 128
    assert nb == 1
    # encode scores as q.k with q = 1 and unit scales; c = 1 (log2 units)
    q = np.ones((1, D))
    k = np.pad(s[:, None], ((0, 128 - S), (0, 0)))
    v = np.zeros((128, D))
    _, _, tr = attention.tiled_attention(q, 1.0, k, np.ones(1), v, np.ones(1), S, 1.0,
                                         pcast="expcast", fp32=False, return_trace=True)
    codes = tr["codes"][0][0]
    return codes


def test_expcast_tv_bound_on_random_rows():
    """Proposition 3.1: TV(p, p_hat) <= 3.64% + mass of the entries cast to 0."""
    rng = np.random.default_rng(7)
    worst = 0.0
    for _ in range(400):
        S = int(rng.integers(2, 129))
        s = rng.standard_normal(S) * rng.uniform(0.1, 8)
        codes = _expcast_row(s)
        p = np.exp2(s - s.max())
        p /= p.sum()
        ph = e4m3.decode(codes)
        ph = ph / ph.sum()
        tail = p[codes == 0].sum()
        tv = attention.total_variation(p, ph)
        assert tv <= attention.EXPCAST_TV_BOUND + tail + 1e-12
        worst = max(worst, tv - tail)
        # per element: log2 error within sigma + 1/16 where the code is normal
        # (codes are relative to the row maximum)
        nz = codes != 0
        err = np.log2(e4m3.decode(codes[nz]) / 256.0) - (s[nz] - s.max())
        assert np.all(np.abs(err) <= attention.EXPCAST_LOG2_ERR + 1e-12)
    assert worst > 0.005


def test_expcast_two_point_row_attains_the_bound():
    """A row whose entries sit at the two extremes of the per-element error,
    with mass ratio 1/(2^e + 1), reaches the 3.64% bound."""
    e = attention.EXPCAST_LOG2_ERR
    K0 = attention.K0
    # group A: t = c - 1/2 with c = 116 (mantissa 4): rounds (half to even) to 116
    # group B: t = c + 1/2 with c = 112 (mantissa 0): rounds to 112
    xa = (116 - 0.5 - K0) / 8.0
    xb = (112 + 0.5 - K0) / 8.0
    ca = attention.expcast_codes(np.array([8 * xa + K0]))[0]
    cb = attention.expcast_codes(np.array([8 * xb + K0]))[0]
    assert (ca, cb) == (116, 112)
    pa, pb = 2.0 ** xa, 2.0 ** xb
    qa, qb = e4m3.decode([ca])[0] / 256, e4m3.decode([cb])[0] / 256
    assert abs(math.log2(qa / pa) - e) < 1e-12 and abs(math.log2(qb / pb) + e) < 1e-12
    # weights na, nb of the two groups plus the exact row max (p = 1, error 0)
    a = 1.0 / (2.0 ** e + 1.0)
    big = 1e12
    na, nb = big * a / pa, big * (1 - a) / pb
    Z = na * pa + nb * pb + 1.0
    Zh = na * qa + nb * qb + 1.0
    tv = 0.5 * (na * abs(pa / Z - qa / Zh) + nb * abs(pb / Z - qb / Zh) + abs(1 / Z - 1 / Zh))
    assert abs(tv - attention.EXPCAST_TV_BOUND) < 1e-8


def test_expcast_underflow_and_clip():
    t = np.array([-50.0, 0.0, 7.4, 7.5, 8.5, 9.5, 119.66, 125.6, 126.5, 300.0])
    codes = attention.expcast_codes(t)
    np.testing.assert_array_equal(codes, [0, 0, 0, 8, 8, 10, 120, 126, 126, 126])


def test_expcast_output_bound_by_value_diameter():
    """Proposition 3.1's output form: |o_hat - o| <= (TV bound + tail) *
    (max_t v_t - min_t v_t) per channel."""
    rng = np.random.default_rng(8)
    for _ in range(50):
        S, D = 128, 16
        s = rng.standard_normal(S) * rng.uniform(0.5, 6)
        v = rng.standard_normal((S, D)) * 3
        codes = _expcast_row(s)
        p = np.exp2(s - s.max())
        p /= p.sum()
        ph = e4m3.decode(codes)
        ph /= ph.sum()
        tail = p[codes == 0].sum()
        diam = v.max(0) - v.min(0)
        assert np.all(np.abs(ph @ v - p @ v) <= (attention.EXPCAST_TV_BOUND + tail) * diam + 1e-12)


def test_score_constant_folded_into_q_gives_log2_scores():
    """Q quantized as c Q (c = softmax_scale log2 e) and the recurrence run
    with c = 1 is softmax attention of the dequantized operands in log2 units:
    exactly dense attention of (deq Q, deq K) at scale ln 2 when P is not
    cast; applying c a second time (or not at all) is far off."""
    rng = np.random.default_rng(8)
    S, D = 300, 64
    q = rng.standard_normal((S, D)).astype(np.float32) * 2
    k = rng.standard_normal((S, D)).astype(np.float32)
    v = rng.standard_normal((S, D)).astype(np.float32)
    c1, qc, qs, kcodes, ks, vcodes, vs, _ = _quantized_case(rng, S, D, q, k, v, smooth=False)
    assert c1 == 1.0
    rows = np.arange(0, S, 11)
    qd = e4m3.decode(qc[rows]) * qs[rows // 128, None].astype(np.float64)
    kd = smoothing.dequantize_blocks(kcodes, ks, S)
    vd = smoothing.dequantize_blocks(vcodes, vs, S)
    od, ld = attention.dense_attention(qd, kd, vd, math.log(2.0))
    ot, lt = attention.tiled_attention(e4m3.decode(qc[rows]), qs[rows // 128], e4m3.decode(kcodes),
                                       ks, e4m3.decode(vcodes), vs, S, 1.0, pcast="none", fp32=False)
    np.testing.assert_allclose(ot, od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lt, ld, rtol=0, atol=1e-12)
    # and it approximates attention of the original operands at 1/sqrt(D)
    o0, _ = attention.dense_attention(q[rows], k, v, 1.0 / math.sqrt(D))
    rel = lambda o: np.linalg.norm(o - o0) / np.linalg.norm(o0)  # noqa: E731
    assert rel(ot) < 0.1
    c = float(smoothing.score_constant(np.float32(1.0 / math.sqrt(D))))
    o2, _ = attention.tiled_attention(e4m3.decode(qc[rows]), qs[rows // 128], e4m3.decode(kcodes),
                                      ks, e4m3.decode(vcodes), vs, S, c, pcast="none", fp32=False)
    assert rel(o2) > 10 * rel(ot)

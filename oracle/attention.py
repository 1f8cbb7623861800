"""Attention: FP64 dense reference and the tiled online-softmax recurrence.

Test infrastructure (see ``oracle/__init__``).

``dense_attention`` is the definition softmax(Q K^T * scale) V with its log2
normalizer, in float64 on the unquantized inputs: the accuracy reference
(TeleFuser PR #40, "Smooth Attention Kernel Accuracy", measures against dense
attention; FastVideo PR #2048, "Test Results", reports the output and the
log2-LSE).

``tiled_attention`` walks the keys in 128-token tiles in the FlashAttention
order that VC-Attention builds on (summary, abstract and "Methodology in Plain
English": an online softmax that keeps the running row maximum and the row
sum, the scores taken after subtracting that maximum).  Per tile j, with the
scores s in log2 units:

    s_t  = (Q~ . K~_t) s_Q s_K,j c       exact dot product of the E4M3 operands
    m'   = max(m, max_t s_t)             running row maximum, once per tile
    p_t  = 2^(s_t - m')                  the FP32 exponential
    P~   = cast of p to E4M3 (see below)
    l_j  = sum_t p_t                     the row sum the recurrence keeps
    l    = 2^(m - m') l + l_j
    acc  = 2^(m - m') acc + s_V,j (P~ . R~_j) + l_j mu_V,j
    m    = m'

and O = acc / l, lse2 = m + log2 l + qmu.  The last term of ``acc`` is the
rank-one restore of the block's V mean from the tile row sum (VC-Attention
summary, Key Contribution 1: the mean is restored inside the online-softmax
recurrence from the row sum it already accumulates).

Readings:

* Scores.  The pages put QK^T on low-bit matrix cores without fixing how the
  products are added, so the score is the dot product itself: the sum of the
  exact products of the decoded E4M3 values, times the block scales and the
  score constant.  Products of two E4M3 values carry at most 8 significant
  bits and lie between 2^-18 and 2^18, so a float64 sum of 128 of them is
  exact in any order.  With ``fp32`` the score is then rounded once to
  float32 (the pages fix FP32 for the softmax that consumes it).
* Row sum (ExpCast off).  l_j is the sum of the float32 probabilities p
  before their cast to E4M3: the row sum a FlashAttention recurrence
  accumulates, which the mean restore reuses.  The restored output is then
  mu + sum_t P~_t (v_t - mu) / sum_t p_t, so the probability cast's error
  multiplies the residual V - mu, not V itself.
* Row sum (ExpCast on).  No float32 p exists, so l_j is the sum of the
  decoded codes, 2^-8 sum_t decode(code_t): the normalizer of the ExpCast
  probability vector that Proposition 3.1 bounds (Key Contribution 4).
  Either way the rank-one term and l use the same l_j.

Probability casts (``pcast``):

* ``"e4m3"``: P~ = E4M3(p 2^8) 2^-8.  Reading: the pages do not fix P's
  scale; 2^8 is a power of two (exact), maps p = 1 (the row maximum) to 256
  (code 0x78) and keeps p >= 2^-14 normal.
* ``"expcast"``: ExpCast-FP8 (VC-Attention summary, Key Contribution 2 and
  Methodology): the E4M3 byte is an affine function of log2 of its value, so
  the code is formed from the log-domain score by one multiply-add and one
  integer conversion:  code = rint(8 (s - m') + K0), codes below 8 (the
  subnormals) become 0 (underflow maps to zero), codes above 126 are
  clipped (the codes stay in the normal E4M3 range), and the byte is used
  as an E4M3 value as is.  With the same 2^8 offset, an exact mapping would be
  code = 8 log2(p) + 120 - 8 delta(M), delta(M) = log2(1 + M/8) - M/8 over
  the eight mantissas M; delta ranges over [0, log2(1.5) - 1/2].  The pages
  centre that one remaining error term minimax: sigma = half that range,
  K0 = 120 - 8 sigma.  rint rounds half to even.
* ``"mxfp4"``: a 4-bit P tile (VC-Attention summary, Future Directions,
  first item: an on-the-fly 4-bit probability needs a per-block scale on
  the softmax path; Main Findings: the 4-bit kernels).  Reading: the pages'
  NVFP4 (E4M3 scale per 16) becomes gfx950's native OCP MXFP4: per query
  row, each group of 32 consecutive keys of a tile (the MX block along the
  PV contraction) takes the E8M0 exponent of its largest p 2^8 (the same
  rule as the MXFP4 V residual, ``fp4.group_exponent``) and E2M1 codes of
  p 2^8 2^-e, nearest with ties to the even code.  P~ = decode 2^(e-8).
  The row sum stays that of the float32 p.
* ``"none"``: no cast (P~ = p), for the exactness pins.

Precision (``fp32=True``): the pages fix the exponential (and K centring) at
FP32 and the operands at E4M3.  Each quantity that decides a code is a
float32 value obtained by rounding the exact (float64) result of its formula
once:

    s_t   = f32(S_t * f32(f32(s_Q s_K,j) c))      S_t the exact dot product
    m'    = max(m, max_t s_t)                     (float32 values)
    e4m3:    p8_t = f32(2^(s_t - m' + 8)),  P~ code = E4M3(p8_t),
             l_j = 2^-8 sum_t p8_t
    expcast: t_t = f32(8 (s_t - m') + f32(K0)),   code = rint(t_t) ...

and l, acc and the rescale factors are float64.  With ``fp32=False``
everything is float64 and K0 is exact.

Pinned by tests/test_oracle_attention.py: brute-force dense attention on
tiny shapes (S in {1, 7, 128, 129, 300}, D in {64, 128}) with no cast; the
K-centring invariance; the V-mean restore identity (block and sequence mean);
joint K/V permutation invariance; the exactness of the float64 score; the
row maximum's code 0x78; lse2 independent of the E4M3 cast; constant-V and
equal-score cases with the cast; the cast's error bound against the residual;
the ExpCast total-variation bound of Proposition 3.1 (3.64% plus the
underflow tail) and its two-point extremal row; the MXFP4 cast against a
per-element brute force, its closed-form group cases and its error bound.
"""
import numpy as np

from . import e4m3, fp4

BLOCK = 128

# ExpCast constants (see module docstring)
DELTA = np.array([np.log2(1.0 + m / 8.0) - m / 8.0 for m in range(8)])
SIGMA = 0.5 * (DELTA.max() - DELTA.min())          # 0.0424812...
K0 = 120.0 - 8.0 * SIGMA                          # 119.6601...
K0_F32 = np.float32(K0)
#: per-element log2 error bound of ExpCast: half a code step plus sigma
EXPCAST_LOG2_ERR = SIGMA + 1.0 / 16.0
#: Proposition 3.1: worst-case TV distance for that per-element bound
EXPCAST_TV_BOUND = (2.0 ** EXPCAST_LOG2_ERR - 1.0) / (2.0 ** EXPCAST_LOG2_ERR + 1.0)


def dense_attention(q, k, v, softmax_scale):
    """float64 softmax(q k^T * scale) v and log2 sum_t 2^(c q.k_t), c = scale*log2 e.

    q [R, D], k [S, D], v [S, D] (any float dtype, used exactly).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = (q @ k.T) * (float(softmax_scale) / np.log(2.0))   # logits in log2 units
    zmax = z.max(axis=1, keepdims=True)
    w = np.exp2(z - zmax)
    den = w.sum(axis=1, keepdims=True)
    out = (w @ v) / den
    lse2 = zmax[:, 0] + np.log2(den[:, 0])
    return out, lse2


def expcast_codes(t):
    """E4M3 codes from ExpCast pre-codes t = 8 (s - m') + K0 (float array)."""
    code = np.rint(np.asarray(t, dtype=np.float64))
    code = np.where(code < 8.0, 0.0, np.minimum(code, 126.0))
    return code.astype(np.uint8)


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def tiled_attention(q_hat, q_scale, k_hat, k_scale, v_hat, v_scale, S, c, *,
                    v_mean=None, vmean_mode="none", q_off=None, pcast="e4m3",
                    fp32=True, block=BLOCK, return_trace=False):
    """One head, R query rows, the recurrence of the module docstring.

    q_hat   [R, D]   query rows (decoded E4M3 codes, or raw values)
    q_scale [R]      s_Q of each row's block (1 for raw values)
    k_hat   [nb*block or more, D]  key rows (decoded codes or raw values)
    k_scale [nb]     s_K per key block
    v_hat   [nb*block or more, D]  residual V rows (decoded codes or raw)
    v_scale [nb]     s_V per key block
    S       number of valid keys; keys >= S are masked
    c       score constant softmax_scale * log2 e (float32 when fp32)
    v_mean  [nb, D] (vmean_mode "block") or [D] ("seq") or None ("none")
    q_off   [R] log2 offset added to lse2 (qmu), or None
    Returns (O [R, D] float64, lse2 [R] float64) and, with return_trace, a
    dict of per-tile P codes (e4m3/expcast), row sums and running maxima.
    """
    q_hat = np.asarray(q_hat, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    R, D = q_hat.shape
    nb = (S + block - 1) // block
    rnd = _f32 if fp32 else (lambda x: np.asarray(x, dtype=np.float64))
    c = float(c)
    q_scale = np.broadcast_to(np.asarray(q_scale, dtype=np.float64), (R,))
    k0 = float(K0_F32) if fp32 else K0

    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, D))
    trace = {"codes": [], "ell": [], "m": []} if return_trace else None
    for j in range(nb):
        lo, hi = j * block, min(S, (j + 1) * block)
        n = hi - lo
        kb = k_hat[lo:lo + block]
        vb = v_hat[lo:lo + block]
        cj = rnd(rnd(q_scale * float(k_scale[j])) * c)      # [R]
        s = rnd((q_hat @ kb[:n].T) * cj[:, None])           # [R, n]
        m_new = np.maximum(m, s.max(axis=1))
        if pcast == "expcast":
            t = rnd(8.0 * (s - m_new[:, None]) + k0)
            codes = expcast_codes(t)
            p_tilde = e4m3.decode(codes) * 2.0 ** -8
            ell = p_tilde.sum(axis=1)
        else:
            p8 = rnd(np.exp2(s - m_new[:, None] + 8.0))
            if pcast == "e4m3":
                codes = e4m3.encode(p8)
                p_tilde = e4m3.decode(codes) * 2.0 ** -8
            elif pcast == "mxfp4":
                codes, exps, vals = mxfp4_probabilities(p8)
                p_tilde = vals * 2.0 ** -8
            elif pcast == "none":
                codes = None
                p_tilde = p8 * 2.0 ** -8
            else:
                raise ValueError(pcast)
            ell = p8.sum(axis=1) * 2.0 ** -8
        alpha = np.exp2(m - m_new)          # 0 on the first tile (m = -inf)
        l = alpha * l + ell
        acc = alpha[:, None] * acc + float(v_scale[j]) * (p_tilde @ vb[:n])
        if vmean_mode == "block":
            acc += ell[:, None] * np.asarray(v_mean, dtype=np.float64)[j][None, :]
        m = m_new
        if return_trace:
            trace["codes"].append(codes)
            trace["ell"].append(ell)
            trace["m"].append(m.copy())
    out = acc / l[:, None]
    if vmean_mode == "seq":
        out = out + np.asarray(v_mean, dtype=np.float64)[None, :]
    lse2 = m + np.log2(l)
    if q_off is not None:
        lse2 = lse2 + np.asarray(q_off, dtype=np.float64)
    if return_trace:
        return out, lse2, trace
    return out, lse2


def mxfp4_probabilities(p8):
    """MXFP4 of one tile's probabilities in units of 2^-8, p8 float [R, n]:
    each row's keys in groups of 32 consecutive keys of the tile (the last
    group of a ragged tile padded with zeros), per group the E8M0 exponent
    e = fp4.group_exponent(group max) and E2M1 codes of p8 2^-e.  Returns
    (codes uint8 [R, n], exponents int64 [R, ceil(n/32)], values float64
    [R, n] = decode(code) 2^e)."""
    p8 = np.asarray(p8, dtype=np.float64)
    R, n = p8.shape
    G = (n + fp4.GROUP - 1) // fp4.GROUP
    pad = np.zeros((R, G * fp4.GROUP))
    pad[:, :n] = p8
    grp = pad.reshape(R, G, fp4.GROUP)
    exps = fp4.group_exponents(grp.max(axis=2))
    scale = np.exp2(exps.astype(np.float64))[..., None]
    codes = fp4.encode(grp / scale)
    vals = fp4.decode(codes) * scale
    return (codes.reshape(R, -1)[:, :n], exps, vals.reshape(R, -1)[:, :n])


def p_codes_row_major(trace, S):
    """The traced P codes of every tile concatenated in key order: [R, S]."""
    return np.concatenate([c for c in trace["codes"]], axis=1)[:, :S]


def total_variation(p, q) -> np.ndarray:
    """Row-wise total-variation distance between two normalized rows."""
    return 0.5 * np.abs(np.asarray(p) - np.asarray(q)).sum(axis=-1)

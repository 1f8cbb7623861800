"""V-Smooth grouping: integer k-means on V, stable label sort, joint K/V gather.

Test infrastructure (see ``oracle/__init__``).

The pages say tokens are grouped by a lightweight online k-means over the
value tokens of a head, the labels are sorted into a permutation, and keys and
values are permuted together by it, which leaves attention unchanged: the
same reordering hits the columns of the probability matrix and the rows of
V, and their product does not see it (VC-Attention summary, Key Contribution 1 and
"Methodology in Plain English").  They fix neither the precision, the
initialisation nor the tie rules.  The reading used here makes the grouping an
integer computation, so that any implementation of it gets the same labels:

1. codes: one power-of-two scale per head, 2^e with e the smallest integer
   such that max|V| <= 127 * 2^e; codes = rint(V * 2^-e) (round half to
   even), int8 in [-127, 127].  The scaling is exact.
2. initial centroids: the codes of tokens floor(j * S / k), j = 0..k-1.
3. ``iters`` Lloyd passes.  Assign: label = argmin_j (|c_j|^2 - 2 v.c_j),
   ties to the lowest j (the same argmin as |v - c_j|^2).  Update: c_j =
   round-half-away-from-zero(sum_j / count_j) in integer arithmetic; an empty
   cluster keeps its centroid.  The labels returned are those of the last
   assignment.
4. perm = stable sort of the labels (ascending label, original order within a
   label); K'[i] = K[perm[i]], V'[i] = V[perm[i]].

Pinned by tests/test_oracle_kmeans.py (brute force with explicit Python loops
on tiny heads, invariants, exact recovery of a separated mixture).
"""
import numpy as np


def code_exponent(v) -> int:
    """Smallest integer e with max|v| <= 127 * 2^e (0 when V is all zero)."""
    amax = float(np.max(np.abs(np.asarray(v, dtype=np.float64))))
    if amax == 0.0:
        return 0
    e = int(np.ceil(np.log2(amax / 127.0)))
    while amax > 127.0 * 2.0 ** e:
        e += 1
    while amax <= 127.0 * 2.0 ** (e - 1):
        e -= 1
    return e


def int8_codes(v):
    """(codes int64 [S, D] in [-127, 127], e) for one head."""
    e = code_exponent(v)
    codes = np.rint(np.asarray(v, dtype=np.float64) * 2.0 ** (-e)).astype(np.int64)
    return codes, e


def initial_centroids(codes, k: int):
    S = codes.shape[0]
    idx = (np.arange(k, dtype=np.int64) * S) // k
    return codes[idx].copy()


def assign(codes, centroids):
    """label[t] = argmin_j |c_j|^2 - 2 v_t . c_j, first index on ties.

    The products are integers of magnitude < 2^22, so the float64 matrix
    product below is exact.
    """
    c = centroids.astype(np.float64)
    dots = codes.astype(np.float64) @ c.T
    dist = (c * c).sum(axis=1)[None, :] - 2.0 * dots
    return np.argmin(dist, axis=1).astype(np.int64)


def update(codes, labels, centroids):
    """Integer centroid update, round half away from zero; empty keeps old."""
    k = centroids.shape[0]
    onehot = np.zeros((k, codes.shape[0]), dtype=np.float64)
    onehot[labels, np.arange(codes.shape[0])] = 1.0
    sums = np.rint(onehot @ codes.astype(np.float64)).astype(np.int64)  # exact, < 2^31
    cnt = np.bincount(labels, minlength=k).astype(np.int64)
    new = centroids.copy()
    nz = cnt > 0
    mag = (2 * np.abs(sums[nz]) + cnt[nz, None]) // (2 * cnt[nz, None])
    new[nz] = np.sign(sums[nz]) * mag
    return new


def lloyd_labels(codes, k: int, iters: int):
    """Labels after ``iters`` (assign, update) passes from the fixed init."""
    if iters < 1:
        raise ValueError("iters must be >= 1")
    cent = initial_centroids(codes, k)
    labels = None
    for _ in range(iters):
        labels = assign(codes, cent)
        cent = update(codes, labels, cent)
    return labels


def stable_perm(labels):
    """perm[i]: original index of the i-th token in (label, index) order."""
    return np.argsort(labels, kind="stable").astype(np.int64)


def kmeans_permute_head(k_head, v_head, n_clusters: int, iters: int):
    """One head: (labels, perm, K', V') with K' = K[perm], V' = V[perm]."""
    codes, _ = int8_codes(v_head)
    labels = lloyd_labels(codes, n_clusters, iters)
    perm = stable_perm(labels)
    return labels, perm, k_head[perm], v_head[perm]


def block_energy_removed(v_ordered, block: int = 128) -> float:
    """1 - |V - blockmean(V)|_F^2 / |V|_F^2 for tokens in the given order.

    The pages report this share for sequence order, a static cube order and
    k-means order (VC-Attention summary, Main Findings, second bullet); they
    do not define it, this is the plain reading.
    """
    v = np.asarray(v_ordered, dtype=np.float64)
    S = v.shape[0]
    tot = float((v * v).sum())
    res = 0.0
    for j in range(0, S, block):
        vb = v[j:j + block]
        r = vb - vb.mean(axis=0)
        res += float((r * r).sum())
    return 1.0 - res / tot if tot > 0 else 0.0

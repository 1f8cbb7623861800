"""Pins of the oracle's integer k-means, stable sort and gather."""
import numpy as np
import torch

from oracle import kmeans


def _bf16(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def _brute_force_labels(v, k, iters):
    """The same reading with explicit Python loops and ints (no numpy math)."""
    rows = [[float(x) for x in r] for r in v]
    amax = max(abs(x) for r in rows for x in r)
    e = 0
    if amax > 0:
        e = -200
        while amax > 127 * 2.0 ** e:
            e += 1
    codes = [[int(round(x * 2.0 ** -e)) for x in r] for r in rows]   # round() is half-even
    S = len(codes)
    cent = [list(codes[(j * S) // k]) for j in range(k)]
    labels = None
    for _ in range(iters):
        labels = []
        for r in codes:
            best = None
            for j, cj in enumerate(cent):
                d = sum((a - b) * (a - b) for a, b in zip(r, cj))
                if best is None or d < best[0]:
                    best = (d, j)
            labels.append(best[1])
        for j in range(k):
            members = [codes[t] for t in range(S) if labels[t] == j]
            if not members:
                continue
            n = len(members)
            new = []
            for dim in range(len(cent[j])):
                s = sum(m[dim] for m in members)
                mag = (2 * abs(s) + n) // (2 * n)
                new.append(mag if s >= 0 else -mag)
            cent[j] = new
    return np.array(labels)


def test_code_exponent_is_the_smallest_fitting_power():
    for amax in [1e-3, 0.5, 1.0, 126.9, 127.0, 127.5, 254.0, 254.1, 3e4]:
        v = np.array([[amax, -0.1 * amax]], dtype=np.float64)
        e = kmeans.code_exponent(v)
        assert amax <= 127 * 2.0 ** e
        assert amax > 127 * 2.0 ** (e - 1)
    assert kmeans.code_exponent(np.zeros((3, 3))) == 0


def test_codes_are_exact_power_of_two_roundings():
    rng = np.random.default_rng(0)
    v = _bf16(rng.standard_normal((200, 16)) * 3)
    codes, e = kmeans.int8_codes(v)
    assert codes.min() >= -127 and codes.max() <= 127
    assert np.abs(codes).max() >= 64     # the scale is tight
    np.testing.assert_array_equal(codes, np.rint(v.astype(np.float64) / 2.0 ** e))


def test_lloyd_matches_brute_force_on_tiny_heads():
    rng = np.random.default_rng(1)
    for S, D, k, iters in [(50, 8, 4, 3), (37, 5, 7, 2), (64, 16, 3, 5), (10, 4, 12, 2)]:
        v = _bf16(rng.standard_normal((S, D)) * 2 + rng.integers(-3, 3, (S, 1)))
        codes, _ = kmeans.int8_codes(v)
        got = kmeans.lloyd_labels(codes, k, iters)
        want = _brute_force_labels(v, k, iters)
        np.testing.assert_array_equal(got, want)


def test_argmin_ties_go_to_the_lowest_cluster():
    codes = np.array([[0, 0], [2, 0], [-2, 0], [1, 0]], dtype=np.int64)
    cent = np.array([[2, 0], [-2, 0], [2, 0]], dtype=np.int64)
    lab = kmeans.assign(codes, cent)
    # token 0 is equidistant from all three: lowest index wins
    assert lab[0] == 0 and lab[1] == 0 and lab[2] == 1 and lab[3] == 0


def test_update_rounds_half_away_and_keeps_empty():
    codes = np.array([[1, -1], [2, -2], [5, 5]], dtype=np.int64)
    labels = np.array([0, 0, 2])
    cent = np.array([[0, 0], [9, 9], [0, 0]], dtype=np.int64)
    new = kmeans.update(codes, labels, cent)
    np.testing.assert_array_equal(new[0], [2, -2])       # 1.5 -> 2, -1.5 -> -2
    np.testing.assert_array_equal(new[1], [9, 9])        # empty keeps
    np.testing.assert_array_equal(new[2], [5, 5])


def test_invariants_on_random_head():
    rng = np.random.default_rng(2)
    S, D, k, iters = 2000, 32, 16, 4
    v = _bf16(rng.standard_normal((S, D)))
    kk = _bf16(rng.standard_normal((S, D)))
    labels, perm, kp, vp = kmeans.kmeans_permute_head(kk, v, k, iters)
    assert sorted(perm.tolist()) == list(range(S))          # bijection
    sl = labels[perm]
    assert np.all(np.diff(sl) >= 0)                          # sorted by label
    same = np.diff(sl) == 0
    assert np.all(np.diff(perm)[same] > 0)                   # stable
    np.testing.assert_array_equal(kp, kk[perm])
    np.testing.assert_array_equal(vp, v[perm])
    # the returned labels are argmins against the centroids of the previous update
    codes, _ = kmeans.int8_codes(v)
    cent = kmeans.initial_centroids(codes, k)
    for _ in range(iters - 1):
        cent = kmeans.update(codes, kmeans.assign(codes, cent), cent)
    d = (codes[:, None, :] - cent[None, :, :]) ** 2
    d = d.sum(-1)
    assert np.all(d[np.arange(S), labels] == d.min(axis=1))


def test_separated_mixture_is_recovered():
    rng = np.random.default_rng(3)
    S, D, k = 4096, 64, 8
    means = rng.standard_normal((k, D)) * 6
    truth = np.repeat(np.arange(k), S // k)        # every component seeds a centroid
    rng.shuffle(truth)
    # the init tokens floor(j S / k) get one component each, so every
    # component seeds one centroid and recovery is exact
    truth[(np.arange(k) * S) // k] = np.arange(k)
    v = _bf16(means[truth] + 0.3 * rng.standard_normal((S, D)))
    codes, _ = kmeans.int8_codes(v)
    lab = kmeans.lloyd_labels(codes, k, 5)
    # a one-to-one map between found and true labels
    pairs = set(zip(lab.tolist(), truth.tolist()))
    assert len(pairs) == k


def test_block_energy_rises_after_grouping():
    rng = np.random.default_rng(4)
    S, D = 4096, 32
    means = rng.standard_normal((16, D)) * 3
    lab = rng.integers(0, 16, S)
    v = _bf16(means[lab] + 0.5 * rng.standard_normal((S, D)))
    seq = kmeans.block_energy_removed(v)
    labels, perm, _, vp = kmeans.kmeans_permute_head(v, v, 16, 8)
    grouped = kmeans.block_energy_removed(vp)
    assert grouped > seq + 0.3


def test_all_zero_v_gives_label_zero():
    v = np.zeros((100, 8), dtype=np.float32)
    codes, e = kmeans.int8_codes(v)
    assert e == 0
    assert np.all(kmeans.lloyd_labels(codes, 5, 3) == 0)

"""Pins of the oracle's E4M3 codec against the format definition (exhaustive
over the 256 codes) and against PyTorch's independent float8_e4m3fn cast."""
import numpy as np
import torch

from oracle import e4m3


def test_decode_anchor_codes():
    d = e4m3.DECODE
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    assert d[0x01] == 2.0 ** -9          # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert d[0x08] == 2.0 ** -6          # smallest normal
    assert d[0x38] == 1.0
    assert d[0x78] == 256.0
    assert d[0x7E] == 448.0              # largest finite
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert d[0xFE] == -448.0


def test_decode_counts_and_monotone():
    d = e4m3.DECODE
    finite = d[~np.isnan(d)]
    assert finite.size == 254
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0)                 # codes 0..126 increase
    assert np.array_equal(d[0x80:0xFF], -pos)       # sign-magnitude


def test_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3.encode(e4m3.decode(codes)), codes)


def _nearest_brute(x):
    """Nearest finite E4M3 value by scanning all codes; ties to even code."""
    best = None
    for c in range(0x7F):
        v = e4m3.DECODE[c]
        dist = abs(abs(x) - v)
        if best is None or dist < best[0] or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    c = best[1]
    return c | 0x80 if np.signbit(x) else c


def test_encode_matches_brute_force_scan():
    rng = np.random.default_rng(0)
    pos = e4m3.DECODE[:0x7F]
    mids = 0.5 * (pos[1:] + pos[:-1])
    xs = np.concatenate([
        mids, -mids,
        np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
        rng.uniform(-448, 448, 2000),
        rng.standard_normal(2000) * 2.0 ** rng.integers(-12, 8, 2000),
        [0.0, -0.0, 447.9, 448.0, -448.0],
    ])
    got = e4m3.encode(xs)
    want = np.array([_nearest_brute(x) for x in xs], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_midpoints_round_to_even_code():
    pos = e4m3.DECODE[:0x7F]
    mids = 0.5 * (pos[1:] + pos[:-1])
    got = e4m3.encode(mids).astype(int)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)


def test_saturation():
    xs = np.array([448.0, 449.0, 463.9, 464.0, 1e6, np.float32(3e38), np.inf])
    assert np.all(e4m3.encode(xs) == 0x7E)
    assert np.all(e4m3.encode(-xs) == 0xFE)
    assert e4m3.encode(np.array([np.nan]))[0] == 0x7F


def test_negative_values_rounding_to_zero_keep_sign():
    assert e4m3.encode(np.array([-1e-9]))[0] == 0x80
    assert e4m3.encode(np.array([1e-9]))[0] == 0x00


def test_matches_torch_float8_e4m3fn_in_range():
    """PyTorch's float8_e4m3fn cast is an independent RNE implementation of
    the same format; it does not saturate, so compare on |x| <= 448."""
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-14, 9, 20000),
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(x)
    assert np.array_equal(got, want)

"""OCP MX FP4 (E2M1) codec and the MXFP4 block quantization of the V residual.

Test infrastructure (see ``oracle/__init__``).

VC-Attention summary (Key Contributions; Main Findings on 4-bit kernels):
V-Smooth also runs with 4-bit operands, where quantizing only the block
residual matters most.  The pages' 4-bit path is NVFP4 on NVIDIA hardware;
gfx950's matrix core takes the OCP MX formats instead, so the reading here
is MXFP4 for the V residual only (Q, K and the probabilities stay E4M3):

* E2M1 nibble = s ee m, exponent bias 1: e == 0 gives (m / 2) (0 or 0.5),
  e >= 1 gives (1 + m / 2) * 2^(e - 1); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  no infinity or NaN.  Encoding rounds to nearest, ties to the even code,
  saturating at 6, sign kept (-0 is nibble 8).
* one E8M0 scale 2^e per 32 consecutive tokens of a 128-token block and per
  channel (the MX block lies along the PV reduction), e the smallest integer
  >= -127 with amax <= 6 * 2^e (e = 0 when the group is all zero), codes =
  E2M1(r * 2^-e).  The same power-of-two rule as the E4M3 block scales, with
  6 in place of 448.

Pinned by tests/test_oracle_fp4.py (exhaustive over the 16 codes, every
midpoint, saturation, the scale rule and the reconstruction error bound).
"""
import numpy as np

GROUP = 32
BLOCK = 128
MAX_FINITE = 6.0


def _decode_one(code: int) -> float:
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = (m / 2.0) if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


#: DECODE[c] is the value of nibble c
DECODE = np.array([_decode_one(c) for c in range(16)], dtype=np.float64)
_POS = DECODE[:8]          # increasing: 0, 0.5, 1, 1.5, 2, 3, 4, 6


def decode(codes) -> np.ndarray:
    return DECODE[np.asarray(codes, dtype=np.uint8) & 15]


def encode(x) -> np.ndarray:
    """E2M1 nibbles (uint8 0..15) of x: nearest value, ties to the even code
    (mantissa bit 0), saturating at 6, sign kept."""
    x = np.asarray(x, dtype=np.float64)
    mag = np.minimum(np.abs(x), MAX_FINITE)
    # nearest candidate by brute force over the 8 magnitudes
    d = np.abs(mag[..., None] - _POS)
    best = d.min(axis=-1, keepdims=True)
    tie = d == best
    # among tied candidates take the even code (codes 0, 2, 4, 6 are even)
    even = tie & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), tie.argmax(axis=-1))
    sign = np.signbit(x)
    return (idx + 8 * sign).astype(np.uint8)


def group_exponent(amax) -> int:
    """Smallest integer e >= -127 with amax <= 6 * 2^e (0 for amax == 0)."""
    a = float(amax)
    if a == 0.0:
        return 0
    e = int(np.floor(np.log2(a))) - 2
    while a > MAX_FINITE * 2.0 ** e:
        e += 1
    while e > -127 and a <= MAX_FINITE * 2.0 ** (e - 1):
        e -= 1
    return max(e, -127)


def group_exponents(amax) -> np.ndarray:
    """group_exponent of every entry of an array (int64, same shape)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    e[nz] = np.floor(np.log2(a[nz])).astype(np.int64) - 2
    while True:
        up = nz & (a > MAX_FINITE * np.exp2(e.astype(np.float64)))
        if not up.any():
            break
        e[up] += 1
    while True:
        dn = nz & (e > -127) & (a <= MAX_FINITE * np.exp2(e.astype(np.float64) - 1))
        if not dn.any():
            break
        e[dn] -= 1
    return np.where(nz, np.maximum(e, -127), 0)


def quantize_mxfp4(r):
    """MXFP4 codes of a float32 [S, D] residual: (codes uint8 [nb*128, D],
    exps int32 [nb*4, D]) -- group g covers tokens 32g .. 32g+31, padding
    tokens past S are 0 (code 0)."""
    r = np.asarray(r, dtype=np.float32)
    S, D = r.shape
    nb = (S + BLOCK - 1) // BLOCK
    pad = np.zeros((nb * BLOCK, D), dtype=np.float32)
    pad[:S] = r
    codes = np.zeros((nb * BLOCK, D), dtype=np.uint8)
    exps = np.zeros((nb * BLOCK // GROUP, D), dtype=np.int32)
    for g in range(nb * BLOCK // GROUP):
        blk = pad[g * GROUP:(g + 1) * GROUP]
        for d in range(D):
            e = group_exponent(np.max(np.abs(blk[:, d])))
            exps[g, d] = e
            codes[g * GROUP:(g + 1) * GROUP, d] = encode(blk[:, d].astype(np.float64) * 2.0 ** -e)
    return codes, exps


def dequantize_mxfp4(codes, exps, S: int) -> np.ndarray:
    """float64 [S, D] values of MXFP4 codes."""
    scale = np.repeat(2.0 ** np.asarray(exps, dtype=np.float64), GROUP, axis=0)
    return decode(codes[:S]) * scale[:S]

"""OCP FP8 E4M3 ("E4M3FN") codec, written from the format definition.

Test infrastructure (see ``oracle/__init__``).

The pages quantize to "E4M3" (TeleFuser PR #40, Changes; VC-Attention summary,
Key Contributions 2 and Methodology, where the byte's exponent field is the
integer part of log2 of the value plus a bias and the mantissa approximates
the fractional part).  The variant is the OCP one that NVIDIA's FP8 tensor
cores and AMD gfx950 both use:

    byte = s eeee mmm, exponent bias 7
    e == 0      : subnormal, value = (-1)^s * (m / 8) * 2^-6
    1 <= e <= 15: normal,    value = (-1)^s * (1 + m / 8) * 2^(e - 7)
    e == 15, m == 7 : NaN (0x7F, 0xFF); there is no infinity
    largest finite magnitude 448 (0x7E), smallest normal 2^-6 (0x08),
    smallest subnormal 2^-9 (0x01).

Encoding is round-to-nearest, ties to the even code (even mantissa LSB), with
saturation: every finite magnitude >= 448 encodes to 448.  The sign bit is
kept, so a negative value that rounds to zero gives -0 (0x80).  NaN encodes to
0x7F.

Pinned by tests/test_oracle_e4m3.py: exhaustive over all 256 codes.
"""
import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def _decode_one(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


#: decode table: DECODE[c] is the float64 value of byte c (NaN for 0x7F/0xFF)
DECODE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)

# non-negative finite magnitudes in increasing order with their codes; the
# codes 0x00..0x7E are already increasing in value
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = DECODE[:0x7F].copy()


def decode(codes) -> np.ndarray:
    """float64 values of an array of E4M3 bytes."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(x) -> np.ndarray:
    """E4M3 bytes of ``x`` (any float dtype; its exact value is used).

    Round to nearest, ties to even code, saturating at +-448; sign kept.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    nan = np.isnan(x)
    neg = np.signbit(x)
    mag = np.minimum(np.abs(np.where(nan, 0.0, x)), MAX_FINITE)
    # index of the first table value >= mag: the upper neighbour
    hi = np.searchsorted(_POS_VALUES, mag, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    v_hi = _POS_VALUES[hi]
    v_lo = _POS_VALUES[lo]
    d_hi = v_hi - mag
    d_lo = mag - v_lo
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    exact = v_hi == mag
    code = np.where(exact | pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(neg, code | 0x80, code)
    out[...] = code.astype(np.uint8)
    out[nan] = NAN_CODE
    return out


def ulp_half(mag) -> np.ndarray:
    """Half the spacing of the E4M3 grid at magnitude ``mag`` (<= 448).

    Spacing is 2^-9 in the subnormal binade and (1/8)*2^E in the binade
    [2^E, 2^(E+1)).  Used by the quantizer error bound.
    """
    mag = np.asarray(mag, dtype=np.float64)
    e = np.floor(np.log2(np.maximum(mag, 2.0 ** -6)))
    return 0.5 * np.where(mag < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))

"""Exact K/V statistics and the per-block E4M3 quantizers (one head at a time).

Test infrastructure (see ``oracle/__init__``).

Arrays are per head: ``x[S, D]``, float32 arrays that hold bf16 values
exactly (the inputs are bf16).  Blocks are 128 consecutive tokens; the last
block of a ragged sequence holds S mod 128 valid tokens.

Sources
-------
* K centring: K minus its sequence mean, computed in FP32 before E4M3
  quantization, is exact for softmax because q . mu_K is the same for every
  key of a row (TeleFuser PR #40, "Changes", first bullet).
* "Exact" K/V statistics in one fused reduction (same list, third bullet):
  the means here are the exact means (float64 sums of the bf16 values,
  rounded once to float32).
* V-Smooth block demeaning: each hardware block subtracts its mean and only
  the residual is quantized (VC-Attention summary, Key Contribution 1 and
  "Methodology in Plain English").  The sequence-mean variant is TeleFuser's
  "centralize V, restore its sequence mean after attention".
* Block quantization scale: one scale per block set by the block's largest
  entry (VC-Attention abstract: the largest entries of a block decide its
  scale).  Reading, for Q, centred K and the V residual alike:
  the scale is the power of two 2^e with e the smallest integer such that
  amax <= 448 * 2^e over the block's valid tokens and all channels (e >=
  -126; e = 0 when amax == 0), and codes = E4M3(x * 2^-e), round to nearest
  even.  A power-of-two block scale (the E8M0 block scale of MX formats) is
  applied by the FP8 matrix core itself, exactly, in both products; it leaves
  every value's relative precision unchanged (E4M3 is a floating-point
  format) and only lets the block maximum land in (224, 448] instead of at
  448.
* Score constant folded into Q: the scores are kept in log2 units (the
  exponential is exp2), so Q is multiplied by c = softmax_scale * log2(e) in
  FP32 before its quantization, as SageAttention-style FP8 attention does
  with its softmax scale.  Reading: the pages leave open where the scale is
  applied; with power-of-two Q and K block scales this makes the matrix
  core's output the log2-domain score itself.

Pinned by tests/test_oracle_quant.py (the smallest fitting power of two,
the block maximum in (224, 448], reconstruction error within half an E4M3
step, padding, exact centring, mean error of the dequantized V) and
tests/test_oracle_hadamard.py (the butterfly against the Kronecker
definition of H_D, orthogonality, the score product unchanged).
"""
import numpy as np

from . import e4m3

BLOCK = 128
LOG2E_F32 = np.float32(1.4426950408889634)


def n_blocks(S: int, block: int = BLOCK) -> int:
    return (S + block - 1) // block


def score_constant(softmax_scale) -> np.float32:
    """c = softmax_scale * log2(e), in float32: scores are kept in log2 units
    so the exponential is exp2 (FlashAttention-style online softmax)."""
    return np.float32(np.float32(softmax_scale) * LOG2E_F32)


def exact_mean_f32(x) -> np.ndarray:
    """Mean over axis 0 of the values in ``x``: float64 sum, float64 divide,
    rounded once to float32."""
    x = np.asarray(x, dtype=np.float64)
    return (x.sum(axis=0) / np.float64(x.shape[0])).astype(np.float32)


def k_seq_mean(k) -> np.ndarray:
    """mu_K[d]: mean of K over all S tokens (float32)."""
    return exact_mean_f32(k)


def v_seq_mean(v) -> np.ndarray:
    """mu_V^seq[d]: mean of V over all S tokens (float32)."""
    return exact_mean_f32(v)


def v_block_means(v, block: int = BLOCK) -> np.ndarray:
    """mu_V^blk[j, d]: mean of V over the valid tokens of block j (float32)."""
    S = v.shape[0]
    nb = n_blocks(S, block)
    out = np.empty((nb, v.shape[1]), dtype=np.float32)
    for j in range(nb):
        out[j] = exact_mean_f32(v[j * block:min(S, (j + 1) * block)])
    return out


def centre(x, mean) -> np.ndarray:
    """float32 x - mean (one float32 subtraction per element)."""
    return (np.asarray(x, dtype=np.float32) - np.asarray(mean, dtype=np.float32)).astype(np.float32)


def residual_blocks(v, block_means, block: int = BLOCK) -> np.ndarray:
    """float32 V - mu_V^blk[block of the token]."""
    S = v.shape[0]
    idx = np.arange(S) // block
    return (np.asarray(v, dtype=np.float32) - block_means[idx]).astype(np.float32)


def pow2_exponent(amax) -> int:
    """Smallest integer e >= -126 with amax <= 448 * 2^e (0 for amax == 0)."""
    a = float(amax)
    if a == 0.0:
        return 0
    e = int(np.floor(np.log2(a))) - 8
    while a > 448.0 * 2.0 ** e:
        e += 1
    while e > -126 and a <= 448.0 * 2.0 ** (e - 1):
        e -= 1
    return max(e, -126)


def quantize_blocks(x, block: int = BLOCK):
    """Per-block E4M3 quantization of a float32 [S, D] array with the
    power-of-two block scale (reading above).

    Returns (codes uint8 [nb*block, D], scale float32 [nb]).  Rows past S are
    padding and get code 0.  Dequantized value = decode(code) * scale.
    """
    x = np.asarray(x, dtype=np.float32)
    S, D = x.shape
    nb = n_blocks(S, block)
    codes = np.zeros((nb * block, D), dtype=np.uint8)
    scale = np.empty(nb, dtype=np.float32)
    for j in range(nb):
        xb = x[j * block:min(S, (j + 1) * block)]
        e = pow2_exponent(np.float32(np.max(np.abs(xb))))
        scale[j] = np.float32(2.0 ** e)
        codes[j * block:j * block + xb.shape[0]] = e4m3.encode(xb.astype(np.float64) * 2.0 ** -e)
    return codes, scale


def prescale_queries(q, c) -> np.ndarray:
    """float32 q * c (one float32 rounding): Q in log2-score units."""
    return (np.asarray(q, dtype=np.float32) * np.float32(c)).astype(np.float32)


def hadamard_rows_f32(x) -> np.ndarray:
    """Each row of a float32 [S, D] array (D a power of two) times the
    Sylvester Hadamard matrix H_D (entries +-1, H H^T = D I), in float32.

    VC-Attention summary, Key Contribution 3 (a QK Hadamard rotation is part
    of the fused preprocessing chain) and Main Findings (rotating Q and K
    moves PSNR by at most 0.1-0.3 dB).  Reading: the unnormalized transform
    is applied to K (after centring) and to Q with the 1/D folded into Q's
    score constant, so (Q H / D)(K H)^T = Q K^T exactly in real arithmetic
    and every scale stays a power of two.  Precision: the transform is the
    butterfly (a, b) -> (a + b, a - b) over channel bit 0, then bit 1, ...,
    each sum and difference rounded to float32 -- fixed so that the codes it
    leads to are decided identically wherever it is computed.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    S, D = y.shape
    if D & (D - 1):
        raise ValueError("D must be a power of two")
    h = 1
    while h < D:
        v = y.reshape(S, D // (2 * h), 2, h)
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        h *= 2
    return y


def round_bf16(x) -> np.ndarray:
    """float32 values rounded to the nearest bf16 (ties to the even
    mantissa), returned as float32: the upper 16 bits of the float32 after
    adding 0x7FFF plus the lowest kept bit (finite inputs)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def rope_rows_bf16(x, cos, sin) -> np.ndarray:
    """Rotary position embedding of each row of a float32 [S, D] array of
    bf16 values, as a model applies it to its bf16 activations: channel
    pair i = (2i, 2i + 1) of token s is rotated by the angle whose cosine
    and sine are cos[s, i], sin[s, i] (float32 [S, D/2]),

        y_2i   = f32(f32(x_2i cos) - f32(x_2i+1 sin))
        y_2i+1 = f32(f32(x_2i sin) + f32(x_2i+1 cos))

    (each product and the sum rounded to float32), then rounded to bf16.

    VC-Attention summary, Key Contribution 3: the rotary embedding is part
    of the fused preprocessing before the quantizers.  Reading: fusing it
    must give what the model's own rotation gives on its bf16 tensors, so
    the result is a bf16 value -- which also keeps every statistic an exact
    float64 sum of bf16 values.
    """
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    a, b = x[:, 0::2], x[:, 1::2]
    y = np.empty_like(x)
    y[:, 0::2] = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    y[:, 1::2] = (a * s).astype(np.float32) + (b * c).astype(np.float32)
    return round_bf16(y)


def hadamard_prescale_queries(q, c) -> np.ndarray:
    """float32 (q H_D) * f32(c / D): the rotated Q in log2-score units (the
    1/D of the rotation is a power of two folded into c, one rounding)."""
    q = np.asarray(q, dtype=np.float32)
    D = q.shape[1]
    cd = np.float32(np.float32(c) * np.float32(1.0 / D))
    return (hadamard_rows_f32(q) * cd).astype(np.float32)


def dequantize_blocks(codes, scale, S: int, block: int = BLOCK) -> np.ndarray:
    """float64 [S, D]: decode(code) * scale of the code's block."""
    idx = np.arange(S) // block
    return e4m3.decode(codes[:S]) * scale[idx].astype(np.float64)[:, None]


def q_log2_offset(q, k_mean, c) -> np.ndarray:
    """qmu[s] = c * (q_s . mu_K), float64, from the unquantized (bf16) q.

    Adding it to the log2-LSE of the centred logits gives the log2-LSE of the
    original logits, because centring K shifts every logit of row s by
    -c * q_s . mu_K (TeleFuser PR #40, Changes, first bullet).
    """
    return np.float64(c) * (np.asarray(q, dtype=np.float64) @ np.asarray(k_mean, dtype=np.float64))

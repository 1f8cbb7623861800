"""The whole hot path for one head, in the pages' order.

Test infrastructure (see ``oracle/__init__``).

0. optional rotary embedding of Q and K (``smoothing.rope_rows_bf16``), as
   the model would apply it before the call;
1. optional V-Smooth grouping: integer k-means on V, stable label sort,
   K and V permuted together (``kmeans``), or a given permutation (a static
   cube grouping, ``grouping``, or one reused from an earlier call);
2. exact statistics: mu_K over the sequence, mu_V per 128-token block (or
   over the sequence) (``smoothing``);
3. per-block E4M3 quantization (power-of-two scales) of c Q, of K - mu_K
   and of the V residual, and qmu = c q.mu_K from the bf16 q (``smoothing``);
   optionally Q and the centred K rotated by a Hadamard matrix first;
4. the tiled recurrence with the rank-one mean restore and the chosen P cast
   (``attention``).

Q, O and lse2 stay in the original token order; only K and V are permuted
(VC-Attention summary, Methodology: one reordering applied to the keys and
the values reorders the probability matrix's columns and V's rows alike,
which leaves their product unchanged).

parity unpinned: the end result (O, lse2) of the quantized pipeline is not
pinned beyond the oracle itself, because the pages print no worked example
and the captured activations they measure on are not available.  Every step
above is pinned on its own (see the per-module docstrings); the pipeline
itself is checked for the direction of the smoothing effect against FP64
dense attention (tests/test_oracle_pipeline.py).
"""
import numpy as np

from . import attention, e4m3, fp4, kmeans, smoothing

BLOCK = 128


def default_scale(D: int) -> np.float32:
    return np.float32(1.0 / np.sqrt(np.float64(D)))


def smoothed_attention_head(q, k, v, *, rows=None, softmax_scale=None,
                            smooth=True, vmean_mode="block", kmeans_kt=None, perm=None,
                            qk_hadamard=False, v_format="e4m3", expcast=False, pcast=None,
                            fp32=True, trace=False, rope=None, p_format="e4m3"):
    """Run the hot path on one head.

    q, k, v: float32 [S, D] holding bf16 values.  rows: query rows to
    evaluate (default all).  kmeans_kt: (k, iters) or None.  perm: a given
    permutation of the keys and values instead (a static cube grouping or a
    permutation reused from an earlier call), or None.  qk_hadamard: Q and
    the centred K rotated by H_D before quantization (smoothing docstring).
    v_format: "e4m3" (per-block power-of-two scale) or "mxfp4" (E2M1 codes
    with an E8M0 scale per 32 tokens and channel, ``fp4``).  smooth: K
    centring and V mean removal on/off (off = the unsmoothed baseline).
    rope: (cos, sin) float32 [S, D/2] tables: Q and K rotated first (token s
    by row s of the tables, before any permutation).
    p_format: "e4m3" (the probability tile as E4M3, or ExpCast with
    ``expcast``) or "mxfp4" (4-bit P: E2M1 codes with an E8M0 exponent per
    32 keys of a tile and query row, ``attention.mxfp4_probabilities``).
    trace: also return the E4M3 probability codes of the evaluated rows
    ("p_codes", [R, S], key order of the (permuted) K) and the running max
    per tile.
    Returns a dict with O, lse2 and every intermediate the GPU path also
    produces.
    """
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    if rope is not None:
        q = smoothing.rope_rows_bf16(q, *rope)
        k = smoothing.rope_rows_bf16(k, *rope)
    S, D = q.shape
    if rows is None:
        rows = np.arange(S)
    rows = np.asarray(rows, dtype=np.int64)
    if softmax_scale is None:
        softmax_scale = default_scale(D)
    c = smoothing.score_constant(softmax_scale)
    out = {"rows": rows, "c": c}

    if kmeans_kt is not None and perm is not None:
        raise ValueError("k-means grouping and a given permutation are exclusive")
    if kmeans_kt is not None:
        labels, perm, kp, vp = kmeans.kmeans_permute_head(k, v, *kmeans_kt)
        out["labels"], out["perm"] = labels, perm
    elif perm is not None:
        perm = np.asarray(perm, dtype=np.int64)
        if not np.array_equal(np.sort(perm), np.arange(S)):
            raise ValueError("perm is not a permutation of the tokens")
        kp, vp = k[perm], v[perm]
        out["perm"] = perm
    else:
        kp, vp = k, v
    out["k_perm"], out["v_perm"] = kp, vp

    if smooth:
        k_mean = smoothing.k_seq_mean(kp)
        kc = smoothing.centre(kp, k_mean)
        if vmean_mode == "block":
            v_mean = smoothing.v_block_means(vp)
            vr = smoothing.residual_blocks(vp, v_mean)
        elif vmean_mode == "seq":
            v_mean = smoothing.v_seq_mean(vp)
            vr = smoothing.centre(vp, v_mean)
        else:
            v_mean, vr = None, vp
        q_off = smoothing.q_log2_offset(q[rows], k_mean, c)
    else:
        k_mean, kc, v_mean, vr, q_off = None, kp, None, vp, None
        vmean_mode = "none"
    out.update(k_mean=k_mean, v_mean=v_mean, vmean_mode=vmean_mode,
               v_block_means=smoothing.v_block_means(vp) if smooth else None)

    if qk_hadamard:
        qpre = smoothing.hadamard_prescale_queries(q, c)
        kc = smoothing.hadamard_rows_f32(kc)
    else:
        qpre = smoothing.prescale_queries(q, c)
    q_codes, q_scale = smoothing.quantize_blocks(qpre)
    k_codes, k_scale = smoothing.quantize_blocks(kc)
    if v_format == "mxfp4":
        v_codes, v_exps = fp4.quantize_mxfp4(vr)
        v_scale = None
        v_hat = fp4.dequantize_mxfp4(v_codes, v_exps, v_codes.shape[0])
        v_hat_scale = np.ones(smoothing.n_blocks(S), dtype=np.float32)
        out["v_exps"] = v_exps
    elif v_format == "e4m3":
        v_codes, v_scale = smoothing.quantize_blocks(vr)
        v_hat, v_hat_scale = e4m3.decode(v_codes), v_scale
    else:
        raise ValueError(f"unknown v_format {v_format!r}")
    out.update(q_codes=q_codes, q_scale=q_scale, k_codes=k_codes,
               k_scale=k_scale, v_codes=v_codes, v_scale=v_scale, q_off=q_off)

    if p_format not in ("e4m3", "mxfp4"):
        raise ValueError(f"unknown p_format {p_format!r}")
    if p_format == "mxfp4" and (expcast or pcast not in (None, "mxfp4")):
        raise ValueError("the 4-bit P tile is its own probability cast")
    if pcast is None:
        pcast = "mxfp4" if p_format == "mxfp4" else ("expcast" if expcast else "e4m3")
    res = attention.tiled_attention(
        e4m3.decode(q_codes[rows]), q_scale[rows // BLOCK],
        e4m3.decode(k_codes), k_scale, v_hat, v_hat_scale, S, 1.0,
        v_mean=v_mean, vmean_mode=vmean_mode, q_off=q_off, pcast=pcast,
        fp32=fp32, return_trace=trace)
    out["O"], out["lse2"] = res[0], res[1]
    if trace and pcast != "none":
        out["p_codes"] = attention.p_codes_row_major(res[2], S)
        out["tile_max"] = np.stack(res[2]["m"], axis=1)
    return out


def sample_rows(S: int, n: int) -> np.ndarray:
    """n evenly spaced query rows, always with row 0, row S-1 and a row of the
    last (possibly ragged) block (TeleFuser PR #40 measures on evenly spaced
    query positions)."""
    if n >= S:
        return np.arange(S)
    r = np.unique(np.linspace(0, S - 1, n).round().astype(np.int64))
    last_block = ((S - 1) // BLOCK) * BLOCK
    extra = [0, S - 1, last_block + (S - 1 - last_block) // 2]
    return np.unique(np.concatenate([r, np.asarray(extra, dtype=np.int64)]))


def error_report(o, ref) -> dict:
    """MSE, cosine, relative L2 and SQNR (dB) of ``o`` against ``ref``, plus
    max-abs and RMSE (the metrics of TeleFuser PR #40's accuracy table and of
    FastVideo PR #2048's error table)."""
    o = np.asarray(o, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    d = o - ref
    mse = float(np.mean(d * d))
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    cos = float(o @ ref / max(np.linalg.norm(o) * np.linalg.norm(ref), 1e-300))
    sqnr = float(10.0 * np.log10(max(np.sum(ref * ref), 1e-300) / max(np.sum(d * d), 1e-300)))
    return {"mse": mse, "cos": cos, "rel_l2": rel, "sqnr_db": sqnr,
            "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
            "rmse": float(np.sqrt(mse))}

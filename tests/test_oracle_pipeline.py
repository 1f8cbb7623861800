"""Oracle pipeline: direction of the smoothing effect against FP64 dense
attention (TeleFuser PR #40's accuracy table), on small synthetic heads."""
import numpy as np
import torch

import workloads
from oracle import attention, kmeans, pipeline


def _head(w, h, S=None):
    q, k, v = workloads.generate(w)
    q, k, v = workloads.head_slices(q, k, v, 0, h)
    if S is not None:
        q, k, v = q[:S], k[:S], v[:S]
    return q, k, v


def test_smoothing_lowers_output_error_on_the_tiny_workload():
    errs = {True: [], False: []}
    for h in range(2):
        q, k, v = _head("tiny", h)
        rows = pipeline.sample_rows(q.shape[0], 64)
        ref, _ = attention.dense_attention(q[rows], k, v, pipeline.default_scale(q.shape[1]))
        for smooth in (True, False):
            r = pipeline.smoothed_attention_head(q, k, v, rows=rows, smooth=smooth)
            errs[smooth].append(pipeline.error_report(r["O"], ref)["rel_l2"])
    assert np.mean(errs[True]) < np.mean(errs[False])


def test_lse2_tracks_dense_lse2():
    q, k, v = _head("tiny", 0)
    rows = pipeline.sample_rows(q.shape[0], 32)
    _, lse_ref = attention.dense_attention(q[rows], k, v, pipeline.default_scale(q.shape[1]))
    err = {}
    for smooth in (True, False):
        r = pipeline.smoothed_attention_head(q, k, v, rows=rows, smooth=smooth)
        err[smooth] = np.max(np.abs(r["lse2"] - lse_ref))
    # K centring removes the offset's quantization error from the scores
    assert err[True] < 0.05 and err[True] < 0.5 * err[False]


def test_grouping_pipeline_stays_close_to_dense_and_raises_block_energy():
    w = workloads.Workload("g", 1, 2048, 2, 128, 11, "mixture", kmeans=(16, 8),
                           extra=dict(n_comp=16, comp_std=3.0, noise=0.5))
    q, k, v = workloads.generate(w)
    qh, kh, vh = workloads.head_slices(q, k, v, 0, 0)
    rows = pipeline.sample_rows(2048, 48)
    ref, lse_ref = attention.dense_attention(qh[rows], kh, vh, pipeline.default_scale(128))
    r = pipeline.smoothed_attention_head(qh, kh, vh, rows=rows, kmeans_kt=(16, 8))
    rep = pipeline.error_report(r["O"], ref)
    assert rep["rel_l2"] < 0.05
    assert kmeans.block_energy_removed(r["v_perm"]) > kmeans.block_energy_removed(vh) + 0.3
    r0 = pipeline.smoothed_attention_head(qh, kh, vh, rows=rows, kmeans_kt=None)
    assert rep["rel_l2"] < pipeline.error_report(r0["O"], ref)["rel_l2"]


def test_expcast_pipeline_error_is_bounded():
    q, k, v = _head("tiny", 1)
    rows = pipeline.sample_rows(q.shape[0], 32)
    ref, _ = attention.dense_attention(q[rows], k, v, pipeline.default_scale(q.shape[1]))
    r1 = pipeline.smoothed_attention_head(q, k, v, rows=rows, expcast=True)
    r0 = pipeline.smoothed_attention_head(q, k, v, rows=rows, expcast=False)
    e1 = pipeline.error_report(r1["O"], ref)["rel_l2"]
    e0 = pipeline.error_report(r0["O"], ref)["rel_l2"]
    # ExpCast adds at most its weight error (Proposition 3.1, total
    # variation <= 3.64% plus the underflow tail) on top of the E4M3 cast;
    # on one small head either may come out ahead
    assert e0 < 0.2 and e1 < e0 + 2 * attention.EXPCAST_TV_BOUND


def test_sample_rows_cover_edges():
    r = pipeline.sample_rows(32626, 256)
    assert r[0] == 0 and r[-1] == 32625
    assert np.any(r >= 32512)
    assert np.all(np.diff(r) > 0)

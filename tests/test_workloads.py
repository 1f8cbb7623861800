"""The seeded synthetic workloads: determinism, shapes and structure."""
import numpy as np
import torch

import workloads


def test_same_seed_same_bytes():
    a = workloads.generate("tiny")
    b = workloads.generate("tiny")
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (1, 1024, 2, 64)
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_tiny_structure_offsets_and_outliers():
    q, k, v = workloads.generate("tiny")
    kf = k.float()[0]
    # a shared per-channel offset of std 3: channel means spread far beyond 1/sqrt(S)
    assert kf.mean(dim=0).std() > 1.5
    # round(0.005 * 1024) = 5 outlier rows x20 per head
    for h in range(2):
        norms = v.float()[0, :, h, :].norm(dim=-1)
        assert int((norms > 5 * norms.median()).sum()) == 5


def test_rope_rows_keep_rms_one():
    w = workloads.Workload("r", 1, 640, 2, 128, 9, "rope_drift",
                           extra=dict(grid=(1, 20, 32), out_frac=0.0, out_mult=1.0))
    q, k, v = workloads.generate(w, dtype=torch.float32)
    rms = q.pow(2).mean(-1).sqrt()
    assert torch.allclose(rms, torch.ones_like(rms), atol=1e-4)


def test_workload_table_matches_the_five_configs():
    shapes = [(w.S, w.H, w.D, w.seed) for w in (workloads.WORKLOADS[n] for n in workloads.ORDER)]
    assert shapes == [(1024, 2, 64, 0), (8192, 8, 128, 1), (32626, 56, 128, 2),
                      (32760, 40, 128, 3), (115328, 56, 128, 4)]
    assert workloads.WORKLOADS["grouped"].kmeans == (16, 8)
    assert workloads.WORKLOADS["long"].kmeans == (32, 4) and workloads.WORKLOADS["long"].expcast
    assert abs(workloads.WORKLOADS["live"].flops - 3.052e13) / 3.052e13 < 1e-3

"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times: inputs generated on the GPU, the whole path run on all heads,
then sampled heads compared with the oracle (statistics, every code, the
k-means labels and permutation in full; O and lse2 on evenly spaced rows
that include the first row, the last row and a row of the ragged last block),
and properties checked on every head."""
import numpy as np
import pytest
import torch

import workloads
from oracle import pipeline
from gpu_util import check_attn, check_intermediates, dev, oracle_head, plan_head

pytestmark = pytest.mark.gpu


def _run(name, expcast=None, opts=None):
    import bit_attention_video_smooth_amd as vs
    w = workloads.WORKLOADS[name]
    d = dev()
    opts = dict(opts or {})
    print(f"[full] {name} S={w.S} H={w.H} D={w.D} kmeans={w.kmeans} expcast={expcast} "
          f"{opts}", flush=True)
    rope = opts.pop("rope", False)
    # rope: Q and K generated before their 3D rotary embedding, which the
    # statistics pass and the quantizers apply from the tables
    q, k, v = workloads.generate(w, device=d, rotate=not rope)
    tables = None
    if rope:
        tables = workloads.rope_tables_3d(w.S, w.D, w.extra["grid"], device=d)
        opts["rope"] = tables
    ec = w.expcast if expcast is None else expcast
    kmeans = None if "cube" in opts else w.kmeans
    plan = vs.Plan((w.B, w.S, w.H, w.D), d, kmeans=kmeans, expcast=ec, **opts)
    plan.run(q, k, v)
    torch.cuda.synchronize(d)
    # properties on every head
    assert torch.isfinite(plan.out).all() and torch.isfinite(plan.lse2).all()
    if plan.perm is not None:
        srt = torch.sort(plan.perm, dim=-1).values
        assert torch.equal(srt, torch.arange(w.S, device=d, dtype=srt.dtype).expand_as(srt))
        if plan.labels is not None:
            lab_sorted = torch.gather(plan.labels, -1, plan.perm.long())
            assert bool((lab_sorted[..., 1:] >= lab_sorted[..., :-1]).all())
    plan.tables = None if tables is None else tuple(t.cpu().numpy() for t in tables)
    return w, q, k, v, plan, ec


LIVE_CUBE = ((20, 48, 34), (2, 8, 8))


CASES = [
    ("mid", None, (0, 7), 64, None),
    ("live", None, (0, 27, 55), 32, None),
    ("grouped", None, (0, 39), 32, None),
    ("long", True, (0, 55), 24, None),
    ("long", False, (31,), 24, None),
    ("live", None, (13,), 32, {"qk_hadamard": True}),
    ("live", None, (41,), 32, {"v_format": "mxfp4"}),
    ("grouped", None, (7,), 32, {"v_format": "mxfp4"}),
    ("live", None, (50,), 32, {"cube": LIVE_CUBE}),
    ("mid", None, (3,), 64, {"mma": "bf16"}),
    ("live", None, (0, 55), 32, {"mma": "bf16"}),
    ("grouped", None, (0, 39), 32, {"mma": "bf16"}),
    ("long", True, (0,), 24, {"mma": "bf16"}),
    ("live", None, (0, 27, 55), 32, {"rope": True}),
    ("live", None, (9,), 32, {"rope": True, "mma": "bf16"}),
    ("live", None, (20,), 32, {"rope": True, "cube": LIVE_CUBE}),
    ("long", True, (0, 55), 24, {"rope": True}),
]


def _case_id(c):
    name, expcast, _, _, opts = c
    parts = [name] + (["expcast"] if expcast else []) + [
        k if v is True else f"{k}_{v}" if isinstance(v, str) else k for k, v in (opts or {}).items()]
    return "-".join(parts)


@pytest.mark.parametrize("name,expcast,heads,nrows,opts", CASES, ids=[_case_id(c) for c in CASES])
def test_full_size(name, expcast, heads, nrows, opts):
    w, q, k, v, plan, ec = _run(name, expcast, opts)
    rows = pipeline.sample_rows(w.S, nrows)
    opts = dict(opts or {})
    kw = {"qk_hadamard": opts.get("qk_hadamard", False),
          "v_format": opts.get("v_format", "e4m3"), "rope": plan.tables}
    if "cube" in opts:
        from oracle import grouping
        kw["perm"] = grouping.cube_permutation(w.S, *opts["cube"])
    else:
        kw["kmeans_kt"] = w.kmeans
    for h in heads:
        print(f"[full] {name} head {h}: oracle", flush=True)
        ref = oracle_head(q, k, v, 0, h, rows, expcast=ec, **kw)
        got = plan_head(plan, 0, h, rows)
        if "perm" in kw:
            np.testing.assert_array_equal(plan.perm[0, h].cpu().numpy(), kw["perm"])
        check_intermediates(got, ref, w.S, label=f"{name} h{h}")
        np.testing.assert_allclose(got["q_mu"][rows], ref["q_off"], rtol=1e-5, atol=1e-5)
        check_attn(got["O"], got["lse2"], ref, label=f"{name} ec={ec} h{h}")

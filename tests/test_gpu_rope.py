"""GPU parity of the rotary embedding fused into the statistics pass and the
Q/K quantizers (vs_smooth_stats_ex, vs_quantize_residual_ex with cos / sin
tables) against the oracle, which rotates Q and K first
(``smoothing.rope_rows_bf16``) and then runs the same pipeline.

Bars: the rotated K's mean, every scale and code (or bf16 operand)
bit-exact; O and log2-LSE to the parity bars (with FP8 products the
relative-L2 bar, max-abs and lse2 reported, as for every input outside the
five workloads); and the fused path
bit-identical to the unfused library path fed the oracle's rotated Q and K
(the same quantized operands reach the same attention kernel).
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import grouping, smoothing
from gpu_util import check_attn, check_intermediates, dev, oracle_head, plan_head

pytestmark = pytest.mark.gpu

# small video-like workloads of the live recipe (unit-norm Q/K rows, drifting
# V with outliers) on token grids whose raster order covers S exactly; the
# last 128-token block is ragged in both
SMALL = {
    "d128": workloads.Workload("rope_d128", 1, 1500, 2, 128, 7, "rope_drift",
                               extra=dict(grid=(3, 20, 25), out_frac=0.005, out_mult=25.0)),
    "d64": workloads.Workload("rope_d64", 2, 900, 2, 64, 8, "rope_drift",
                              extra=dict(grid=(1, 30, 30), out_frac=0.005, out_mult=25.0)),
}


def _inputs(w, d):
    q, k, v = workloads.generate(w, rotate=False)
    cos, sin = workloads.rope_tables_3d(w.S, w.D, w.extra["grid"])
    return q, k, v, cos, sin


def _rotated_bf16(x, cos, sin):
    """The oracle's rotation of every head of a bf16 [B, S, H, D] tensor."""
    B, S, H, D = x.shape
    out = torch.empty_like(x)
    c, s = cos.numpy(), sin.numpy()
    for b in range(B):
        for h in range(H):
            r = smoothing.rope_rows_bf16(x[b, :, h, :].float().numpy(), c, s)
            out[b, :, h, :] = torch.from_numpy(r).to(torch.bfloat16)   # exact: bf16 values
    return out


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("case", ["d128", "d64"])
def test_rotated_k_mean(case, layout):
    """vs_smooth_stats_ex: the mean of the rotated K, bit-exact, in both token
    layouts; the V means equal vs_smooth_stats' (V is not rotated)."""
    import bit_attention_video_smooth_amd as vs
    w = SMALL[case]
    d = dev()
    print(f"[rope stats] {case} layout {layout}", flush=True)
    q, k, v, cos, sin = _inputs(w, d)
    B, S, H, D = w.B, w.S, w.H, w.D
    kk, vv = (k, v) if layout == 0 else (k.transpose(1, 2).contiguous(), v.transpose(1, 2).contiguous())
    nb = (S + 127) // 128
    e = lambda *s: torch.full(s, float("nan"), device=d)  # noqa: E731
    km, vbm, vsm = e(B, H, D), e(B, H, nb, D), e(B, H, D)
    km0, vbm0, vsm0 = e(B, H, D), e(B, H, nb, D), e(B, H, D)
    ws = torch.empty(vs.vs_smooth_stats_workspace_bytes(B, S, H, D), dtype=torch.uint8, device=d)
    shape = (B, S, H, D)
    vs.vs_smooth_stats_ex(kk.to(d), vv.to(d), shape, layout, cos.to(d), sin.to(d), km, vbm, vsm, ws)
    vs.vs_smooth_stats(kk.to(d), vv.to(d), shape, layout, km0, vbm0, vsm0, ws)
    torch.cuda.synchronize(d)
    for b in range(B):
        for h in range(H):
            kr = smoothing.rope_rows_bf16(k[b, :, h, :].float().numpy(), cos.numpy(), sin.numpy())
            np.testing.assert_array_equal(km[b, h].cpu().numpy(), smoothing.k_seq_mean(kr))
    assert torch.equal(vbm, vbm0) and torch.equal(vsm, vsm0)
    # the rotation changes the mean (the test would not see a skipped rotation otherwise)
    assert not torch.equal(km, km0)


OPTS = [
    ("plain", {}),
    ("hadamard", {"qk_hadamard": True}),
    ("cube", {"cube": True}),
    ("kmeans", {"kmeans": (8, 3)}),
    ("seq_mean", {"vmean": "seq"}),
    ("unsmoothed", {"smooth": False}),
]


@pytest.mark.parametrize("mma", ["fp8", "bf16"])
@pytest.mark.parametrize("opt", [o[0] for o in OPTS])
@pytest.mark.parametrize("case", ["d128", "d64"])
def test_fused_rope_path(case, opt, mma):
    """The whole path on unrotated Q, K with the tables: intermediates
    bit-exact and O, lse2 within the bars against the oracle with rope, on
    every query row of every head."""
    import bit_attention_video_smooth_amd as vs
    w = SMALL[case]
    d = dev()
    kw = dict(dict(OPTS)[opt])
    print(f"[rope path] {case} {opt} {mma}", flush=True)
    q, k, v, cos, sin = _inputs(w, d)
    okw = {"qk_hadamard": kw.get("qk_hadamard", False), "kmeans_kt": kw.get("kmeans"),
           "vmean_mode": kw.get("vmean", "block"), "smooth": kw.get("smooth", True)}
    if kw.pop("cube", False):
        cube = (w.extra["grid"], (1, 4, 4) if w.extra["grid"][0] < 2 else (2, 4, 4))
        kw["cube"] = cube
        okw["perm"] = grouping.cube_permutation(w.S, *cube)
    plan = vs.Plan((w.B, w.S, w.H, w.D), d, mma=mma, rope=(cos.to(d), sin.to(d)), **kw)
    plan.run(q.to(d), k.to(d), v.to(d))
    torch.cuda.synchronize(d)
    rows = np.arange(w.S)
    tables = (cos.numpy(), sin.numpy())
    for b in range(w.B):
        for h in range(w.H):
            ref = oracle_head(q, k, v, b, h, rows, rope=tables, **okw)
            got = plan_head(plan, b, h, rows)
            check_intermediates(got, ref, w.S, label=f"rope {case} {opt} b{b}h{h}")
            if ref["q_off"] is not None:
                np.testing.assert_allclose(got["q_mu"][rows], ref["q_off"], rtol=1e-5, atol=1e-5)
            # FP8 products on these small inputs: the relative-L2 bar, max-abs
            # and lse2 reported (the policy of the parity tests outside the
            # five workloads); bf16 products: all three bars
            check_attn(got["O"], got["lse2"], ref, label=f"rope {case} {opt} {mma} b{b}h{h}",
                       strict=(mma == "bf16"))


@pytest.mark.parametrize("mma", ["fp8", "bf16"])
def test_fused_equals_unfused_at_live_size(mma):
    """At the live shape (S = 32626 over a 20 x 48 x 34 grid, 56 heads,
    D = 128): the fused rotation gives bit-for-bit the codes, means, O and
    lse2 of the unfused path run on the oracle's rotated Q and K."""
    import bit_attention_video_smooth_amd as vs
    w = workloads.WORKLOADS["live"]
    d = dev()
    print(f"[rope live] {mma}: inputs", flush=True)
    q, k, v = workloads.generate(w, device=d, rotate=False)
    cos, sin = workloads.rope_tables_3d(w.S, w.D, w.extra["grid"], device=d)
    qr = _rotated_bf16(q.cpu(), cos.cpu(), sin.cpu()).to(d)
    kr = _rotated_bf16(k.cpu(), cos.cpu(), sin.cpu()).to(d)
    shape = (w.B, w.S, w.H, w.D)
    print(f"[rope live] {mma}: fused and unfused runs", flush=True)
    fused = vs.Plan(shape, d, mma=mma, rope=(cos, sin))
    fused.run(q, k, v)
    plain = vs.Plan(shape, d, mma=mma)
    plain.run(qr, kr, v)
    torch.cuda.synchronize(d)
    # every buffer in full: the quantizers also write the padding rows and
    # tokens of the ragged last block (as zero codes)
    for name in ["k_mean", "v_mean", "q_mu", "q8", "q_scale", "k8", "k_scale", "v8", "v_scale",
                 "out", "lse2"]:
        a, b = getattr(fused, name), getattr(plain, name)
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), name

"""Helpers of the GPU parity tests (host-side layout handling and checks)."""
import numpy as np
import torch

import workloads
from oracle import e4m3, fp4, pipeline

# token held at position p of a V block row (the layout vsmooth.h documents)
V_TOKEN_OF_POS = np.array([64 * (p // 64) + 32 * ((p % 32) // 16) + 8 * ((p % 16) // 4)
                           + 4 * ((p % 64) // 32) + p % 4 for p in range(128)])

TOL_MAX_ABS = 2e-3
TOL_REL_L2 = 5e-3
TOL_LSE2 = 1e-4


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test without a GPU")
    return torch.device("cuda:0")


# token held at position p of a bf16 V block row (the VS_BF16_MMA layout
# vsmooth.h documents): bits 2 and 3 of p swapped (an involution)
V16_TOKEN_OF_POS = np.array([(p & ~12) | (((p >> 3) & 1) << 2) | (((p >> 2) & 1) << 3)
                             for p in range(128)])


def v16_rows(v16_head):
    """[nb, D, 128] bf16 V values (as float) -> [nb*128, D] in token order."""
    nb, D, _ = v16_head.shape
    out = np.zeros((nb * 128, D), dtype=np.float64)
    for j in range(nb):
        out[j * 128 + V16_TOKEN_OF_POS, :] = v16_head[j].T
    return out


# token held at position p of a V block row for the 4-bit probability tile
# (VS_P_MXFP4): bits 4 and 5 of p swapped
P4_TOKEN_OF_POS = np.array([(p & ~48) | (((p >> 4) & 1) << 5) | (((p >> 5) & 1) << 4)
                            for p in range(128)])


def v8_rows(v8_head, token_of_pos=None):
    """[nb, D, 128] block-transposed V codes -> [nb*128, D] in token order."""
    order = V_TOKEN_OF_POS if token_of_pos is None else token_of_pos
    nb, D, _ = v8_head.shape
    out = np.zeros((nb * 128, D), dtype=np.uint8)
    for j in range(nb):
        out[j * 128 + order, :] = v8_head[j].T
    return out


def run_plan(q, k, v, **kw):
    """Run the GPU path on CPU bf16 tensors; returns the Plan (buffers on GPU)."""
    import bit_attention_video_smooth_amd as vs
    d = dev()
    plan = vs.Plan(tuple(q.shape), d, **kw)
    plan.run(q.to(d), k.to(d), v.to(d))
    torch.cuda.synchronize(d)
    return plan


def oracle_head(q, k, v, b, h, rows, **kw):
    qh, kh, vh = workloads.head_slices(q, k, v, b, h)
    return pipeline.smoothed_attention_head(qh, kh, vh, rows=rows, **kw)


def attn_errors(o_gpu, lse_gpu, ref):
    o = np.asarray(o_gpu, dtype=np.float64)
    d = np.abs(o - ref["O"])
    return {"max_abs": float(d.max()),
            "rel_l2": float(np.linalg.norm(d) / max(np.linalg.norm(ref["O"]), 1e-30)),
            "lse2": float(np.abs(np.asarray(lse_gpu, dtype=np.float64) - ref["lse2"]).max()),
            # the distribution of |O - O_oracle| (the largest few come from single
            # probability codes one step from the oracle's)
            "p50": float(np.quantile(d, 0.5)), "p99": float(np.quantile(d, 0.99)),
            "p9999": float(np.quantile(d, 0.9999))}


def check_attn(o_gpu, lse_gpu, ref, label="", strict=True):
    """O and lse2 against the oracle.  strict: all three bars.  Not strict
    (the FP8 matrix core's products on inputs outside the five workloads,
    where its truncated accumulation moves single probability codes next to
    large V rows): the relative-L2 bar only; max-abs and lse2 are reported."""
    e = attn_errors(o_gpu, lse_gpu, ref)
    tag = "" if strict else " (fp8 products: rel-L2 bar only)"
    print(f"{label}: max_abs {e['max_abs']:.3e} rel_l2 {e['rel_l2']:.3e} lse2 {e['lse2']:.3e} "
          f"|dO| p50 {e['p50']:.1e} p99 {e['p99']:.1e} p99.99 {e['p9999']:.1e}{tag}", flush=True)
    assert e["rel_l2"] <= TOL_REL_L2, e
    if strict:
        assert e["max_abs"] <= TOL_MAX_ABS, e
        assert e["lse2"] <= TOL_LSE2, e
    return e


def v4_rows(v8_head, vsc_head):
    """MXFP4 V of one head: ([nb, D, 64] nibble tiles, [nb, D, 4] E8M0 bytes)
    -> (codes [nb*128, D], exponents [nb*4, D]) in token order (the layout
    vsmooth.h documents for VS_V_MXFP4)."""
    nb, D, _ = v8_head.shape
    codes = np.zeros((nb * 128, D), dtype=np.uint8)
    q = np.arange(32)
    u = 8 * ((q % 16) // 4) + 4 * (q // 16) + q % 4
    for j in range(nb):
        for g in range(4):
            byts = v8_head[j, :, 16 * g:16 * g + 16]          # [D, 16]
            nib = np.stack([byts & 15, byts >> 4], axis=-1).reshape(D, 32)
            codes[j * 128 + 32 * g + u, :] = nib.T
    exps = vsc_head.astype(np.int32).transpose(0, 2, 1).reshape(nb * 4, D) - 127
    return codes, exps


def plan_head(plan, b, h, rows):
    """GPU outputs of one head: O rows, lse2 rows and the intermediates."""
    S = plan.shape[1]
    g = lambda t: None if t is None else t[b, h].cpu().numpy()  # noqa: E731
    qk16 = getattr(plan, "mma", "fp8") == "bf16"
    out = {"O": plan.out[b, :, h, :].float().cpu().numpy()[rows],
           "lse2": plan.lse2[b, h].cpu().numpy()[rows],
           "q_codes": None if qk16 else g(plan.q8), "k_codes": None if qk16 else g(plan.k8),
           "q16": plan.q8[b, h].float().cpu().numpy() if qk16 else None,
           "k16": plan.k8[b, h].float().cpu().numpy() if qk16 else None,
           "q_scale": g(plan.q_scale), "k_scale": g(plan.k_scale), "v_scale": g(plan.v_scale),
           "k_mean": g(plan.k_mean), "v_mean": g(plan.v_mean),
           "q_mu": None if plan.q_mu is None else plan.q_mu[b, h].cpu().numpy()}
    if qk16:
        out["v16"] = v16_rows(plan.v8[b, h].float().cpu().numpy())
        out["v_codes"] = None
        if getattr(plan, "v_format", "e4m3") == "mxfp4":
            out["v_exps"] = plan.v_scale[b, h].cpu().numpy().astype(np.int32).transpose(0, 2, 1)
            out["v_exps"] = out["v_exps"].reshape(-1, out["v_exps"].shape[-1]) - 127
            out["v_scale"] = None
    elif getattr(plan, "v_format", "e4m3") == "mxfp4":
        out["v_codes"], out["v_exps"] = v4_rows(g(plan.v8), g(plan.v_scale))
        out["v_scale"] = None
    elif getattr(plan, "p_format", "e4m3") == "mxfp4":
        # the 4-bit probability tile's V layout: position p holds token p with
        # bits 4 and 5 swapped
        out["v_codes"] = v8_rows(g(plan.v8), P4_TOKEN_OF_POS)
    else:
        out["v_codes"] = v8_rows(g(plan.v8))
    if plan.labels is not None:
        out["labels"] = g(plan.labels)
        out["perm"] = g(plan.perm)
        if plan.k_perm is not None:
            out["k_perm"] = plan.k_perm[b, h].view(torch.int16).cpu().numpy()
            out["v_perm"] = plan.v_perm[b, h].view(torch.int16).cpu().numpy()
    assert out["O"].shape[0] == len(rows) and S >= len(rows)
    return out


def check_intermediates(gpu, ref, S, label=""):
    """Statistics and codes bit-exact; q_mu to float32 summation error."""
    np.testing.assert_array_equal(gpu["q_scale"], ref["q_scale"], err_msg=label + " q_scale")
    np.testing.assert_array_equal(gpu["k_scale"], ref["k_scale"], err_msg=label + " k_scale")
    if ref.get("v_exps") is not None:
        np.testing.assert_array_equal(gpu["v_exps"], ref["v_exps"], err_msg=label + " v_exps")
    else:
        np.testing.assert_array_equal(gpu["v_scale"], ref["v_scale"], err_msg=label + " v_scale")
    if gpu.get("q16") is not None:
        # bf16 operands: the oracle's E4M3 values times their block scales, exactly
        for name, codes, sc in (("q16", ref["q_codes"], ref["q_scale"]),
                                ("k16", ref["k_codes"], ref["k_scale"])):
            want = e4m3.decode(codes) * np.repeat(sc.astype(np.float64), 128)[:, None]
            np.testing.assert_array_equal(gpu[name].astype(np.float64), want,
                                          err_msg=label + " " + name)
        # and V: the oracle's residual codes' values times their scales
        nb = len(ref["q_scale"])
        if ref.get("v_exps") is not None:
            want = fp4.dequantize_mxfp4(ref["v_codes"], ref["v_exps"], nb * 128)
        else:
            want = e4m3.decode(ref["v_codes"]) * np.repeat(ref["v_scale"].astype(np.float64), 128)[:, None]
        np.testing.assert_array_equal(gpu["v16"], want[:nb * 128], err_msg=label + " v16")
    else:
        np.testing.assert_array_equal(gpu["q_codes"], ref["q_codes"], err_msg=label + " q codes")
        np.testing.assert_array_equal(gpu["k_codes"], ref["k_codes"], err_msg=label + " k codes")
        np.testing.assert_array_equal(gpu["v_codes"], ref["v_codes"], err_msg=label + " v codes")
    if ref["k_mean"] is not None:
        np.testing.assert_array_equal(gpu["k_mean"], ref["k_mean"], err_msg=label + " k_mean")
        np.testing.assert_array_equal(gpu["v_mean"], ref["v_mean"], err_msg=label + " v_mean")
    if "labels" in ref:
        np.testing.assert_array_equal(gpu["labels"], ref["labels"], err_msg=label + " labels")
        np.testing.assert_array_equal(gpu["perm"], ref["perm"], err_msg=label + " perm")


def pcode_flips(gpu_codes, ref_codes, label="", expcast=False):
    """Compare the kernel's E4M3 probability codes ([R, S], from
    Plan.attn_pcodes) with the oracle's: returns per-row counts of differing
    codes, and checks that each differs by one code step (a rounding boundary
    crossed, not a wrong value).  Steps count the codes the cast can produce:
    every code for E4M3; 0 and 8..126 for ExpCast, whose pre-codes below 8
    become 0 (so 8 and 0 are neighbours)."""
    g = np.asarray(gpu_codes).astype(np.int64)
    r = np.asarray(ref_codes).astype(np.int64)
    diff = g != r
    per_row = diff.sum(axis=1)
    if expcast:
        assert not np.any((g > 0) & (g < 8)), f"{label}: an ExpCast code below 8 and not 0"
        g, r = np.where(g == 0, 7, g), np.where(r == 0, 7, r)
    step = np.abs(g - r).max() if diff.any() else 0
    print(f"{label}: P codes differing {int(diff.sum())} of {diff.size} "
          f"({diff.mean():.2e}); per row max {int(per_row.max())} mean {per_row.mean():.2f}; "
          f"largest step {int(step)}", flush=True)
    assert step <= 1, f"{label}: a code differs by {step} steps"
    return per_row

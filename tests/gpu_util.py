"""Helpers of the GPU parity tests (host-side layout handling and checks)."""
import numpy as np
import torch

import workloads
from oracle import pipeline

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


def v8_rows(v8_head):
    """[nb, D, 128] block-transposed V codes -> [nb*128, D] in token order."""
    nb, D, _ = v8_head.shape
    out = np.zeros((nb * 128, D), dtype=np.uint8)
    for j in range(nb):
        out[j * 128 + V_TOKEN_OF_POS, :] = v8_head[j].T
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
    d = o - ref["O"]
    return {"max_abs": float(np.abs(d).max()),
            "rel_l2": float(np.linalg.norm(d) / max(np.linalg.norm(ref["O"]), 1e-30)),
            "lse2": float(np.abs(np.asarray(lse_gpu, dtype=np.float64) - ref["lse2"]).max())}


def check_attn(o_gpu, lse_gpu, ref, label=""):
    e = attn_errors(o_gpu, lse_gpu, ref)
    print(f"{label}: max_abs {e['max_abs']:.3e} rel_l2 {e['rel_l2']:.3e} lse2 {e['lse2']:.3e}",
          flush=True)
    assert e["max_abs"] <= TOL_MAX_ABS, e
    assert e["rel_l2"] <= TOL_REL_L2, e
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
    out = {"O": plan.out[b, :, h, :].cpu().numpy()[rows],
           "lse2": plan.lse2[b, h].cpu().numpy()[rows],
           "q_codes": g(plan.q8), "k_codes": g(plan.k8),
           "q_scale": g(plan.q_scale), "k_scale": g(plan.k_scale), "v_scale": g(plan.v_scale),
           "k_mean": g(plan.k_mean), "v_mean": g(plan.v_mean),
           "q_mu": None if plan.q_mu is None else plan.q_mu[b, h].cpu().numpy()}
    if getattr(plan, "v_format", "e4m3") == "mxfp4":
        out["v_codes"], out["v_exps"] = v4_rows(g(plan.v8), g(plan.v_scale))
        out["v_scale"] = None
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
    np.testing.assert_array_equal(gpu["q_codes"], ref["q_codes"], err_msg=label + " q codes")
    np.testing.assert_array_equal(gpu["k_codes"], ref["k_codes"], err_msg=label + " k codes")
    np.testing.assert_array_equal(gpu["v_codes"], ref["v_codes"], err_msg=label + " v codes")
    if ref["k_mean"] is not None:
        np.testing.assert_array_equal(gpu["k_mean"], ref["k_mean"], err_msg=label + " k_mean")
        np.testing.assert_array_equal(gpu["v_mean"], ref["v_mean"], err_msg=label + " v_mean")
    if "labels" in ref:
        np.testing.assert_array_equal(gpu["labels"], ref["labels"], err_msg=label + " labels")
        np.testing.assert_array_equal(gpu["perm"], ref["perm"], err_msg=label + " perm")

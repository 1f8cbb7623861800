"""Seeded synthetic inputs for the five attention workloads.

This module holds input generation only; it contains none of the method's
arithmetic and is shared by the tests, the benchmark and the smoke check.
Both the GPU path and the CPU oracle consume the same bf16 tensors.

The captured MiniMax-H3 activations that TeleFuser PR #40 measures on
("Smooth Attention Kernel Accuracy": post-QK-norm, post-RoPE Q/K/V at live
shape (1, 32626, 56, 128)) are not available; these generators stand in for
them with the shapes, value distributions and structure described below.
Readings where the workload descriptions are loose:

* "N(0, s)" means standard deviation s.
* "unit-norm rows (post-QK-norm)": RMS-normalized rows, |row|_2 = sqrt(D),
  so the logits q.k/sqrt(D) are about N(0, 1) before RoPE mixing.
* 3D RoPE: D split 44/42/42 over (t, h, w), interleaved pairs, base 10000,
  positions in raster order over a T x 48 x 34 grid truncated to S
  (T = 20 for S = 32626, T = 71 for S = 115328).
* V drift: A sin(2 pi f s / S + phi) per (head, channel), A ~ U(0.5, 2),
  f ~ U(0.5, 4), phi ~ U(0, 2 pi).
* outliers: round(frac * S) whole V rows per head, chosen uniformly without
  replacement, multiplied by the factor.
* the long-context workload uses the live-shape recipe (RMS-normalized
  RoPE'd Q/K, drifting V, 0.05% outliers x25).
* the grouping workload's Q is N(0, 1); its V is a 16-component mixture
  per head (means ~ N(0, 3^2 I), sigma 0.5, labels uniform at random), and
  K = V W_h + N(0, 1) with W_h orthogonal (QR of a Gaussian matrix).

All draws come from one ``torch.Generator`` seeded per workload, in float32,
then cast to bf16 (round to nearest even).  Layout [B, S, H, D].  The
generator lives on the device asked for: the same seed gives the same bytes
on a given device type (CPU and GPU streams differ), and both the library and
the oracle always consume one generated copy.
"""
from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    H: int
    D: int
    seed: int
    recipe: str
    kmeans: tuple = None          # (k, iters) or None
    expcast: bool = False
    smooth: bool = True
    extra: dict = field(default_factory=dict)

    @property
    def flops(self) -> float:
        """Attention FLOPs, 4 * B * S^2 * D * H (QK^T and PV)."""
        return 4.0 * self.B * self.S * self.S * self.D * self.H


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1024, 2, 64, 0, "offsets",
                     extra=dict(k_off=3.0, k_off_shared=True, v_off=0.0,
                                out_frac=0.005, out_mult=20.0)),
    "mid": Workload("mid", 1, 8192, 8, 128, 1, "offsets",
                    extra=dict(k_off=4.0, k_off_shared=False, v_off=2.0,
                               out_frac=0.001, out_mult=30.0)),
    "live": Workload("live", 1, 32626, 56, 128, 2, "rope_drift",
                     extra=dict(grid=(20, 48, 34), out_frac=0.0005, out_mult=25.0)),
    "grouped": Workload("grouped", 1, 32760, 40, 128, 3, "mixture",
                        kmeans=(16, 8),
                        extra=dict(n_comp=16, comp_std=3.0, noise=0.5)),
    "long": Workload("long", 1, 115328, 56, 128, 4, "rope_drift",
                     kmeans=(32, 4), expcast=True,
                     extra=dict(grid=(71, 48, 34), out_frac=0.0005, out_mult=25.0)),
}
ORDER = ["tiny", "mid", "live", "grouped", "long"]


def _rms_normalize(x):
    return x * torch.rsqrt((x * x).mean(dim=-1, keepdim=True))


def _rope_3d(x, grid, base=10000.0, split=(44, 42, 42)):
    """Rotate interleaved channel pairs of x [B, S, H, D] by 3D positions."""
    B, S, H, D = x.shape
    assert sum(split) == D
    T, GH, GW = grid
    s = torch.arange(S, dtype=torch.float64, device=x.device)
    pos = [torch.div(s, GH * GW, rounding_mode="floor"),
           torch.remainder(torch.div(s, GW, rounding_mode="floor"), GH),
           torch.remainder(s, GW)]
    out = x.clone()
    off = 0
    for axis, part in enumerate(split):
        half = part // 2
        inv = base ** (-torch.arange(half, dtype=torch.float64, device=x.device) * 2.0 / part)
        ang = (pos[axis][:, None] * inv[None, :]).to(torch.float32)       # [S, half]
        cos = torch.cos(ang)[None, :, None, :]
        sin = torch.sin(ang)[None, :, None, :]
        a = x[..., off:off + part:2]
        b = x[..., off + 1:off + part:2]
        out[..., off:off + part:2] = a * cos - b * sin
        out[..., off + 1:off + part:2] = a * sin + b * cos
        off += part
    return out


def rope_split(D):
    """Channel split of the 3D rotary embedding over (t, h, w): even parts,
    44/42/42 at D = 128 (scaled for other D)."""
    return (44, 42, 42) if D == 128 else (D - 2 * (D // 3 // 2 * 2), D // 3 // 2 * 2, D // 3 // 2 * 2)


def rope_tables_3d(S, D, grid, base=10000.0, split=None, device="cpu"):
    """cos, sin float32 [S, D/2] of a 3D rotary embedding over a T x GH x GW
    token grid in raster order (token s at (s // (GH GW), (s // GW) % GH,
    s % GW)); pair i covers channels 2i, 2i + 1, and the pairs of each axis'
    part of the channels rotate by position * base^(-2k / part).  Input
    data for both the library's fused rotation and the oracle's."""
    split = split or rope_split(D)
    assert sum(split) == D and all(p % 2 == 0 for p in split)
    T, GH, GW = grid
    s = torch.arange(S, dtype=torch.float64, device=device)
    pos = [torch.div(s, GH * GW, rounding_mode="floor"),
           torch.remainder(torch.div(s, GW, rounding_mode="floor"), GH),
           torch.remainder(s, GW)]
    angs = []
    for axis, part in enumerate(split):
        half = part // 2
        inv = base ** (-torch.arange(half, dtype=torch.float64, device=device) * 2.0 / part)
        angs.append(pos[axis][:, None] * inv[None, :])
    ang = torch.cat(angs, dim=1).to(torch.float32)
    return torch.cos(ang).contiguous(), torch.sin(ang).contiguous()


def _outliers(v, frac, mult, g):
    B, S, H, D = v.shape
    n = int(round(frac * S))
    for b in range(B):
        for h in range(H):
            idx = torch.randperm(S, generator=g, device=v.device)[:n]
            v[b, idx, h, :] *= mult
    return v


def generate(w, *, dtype=torch.bfloat16, device="cpu", rotate=True):
    """Return (q, k, v) tensors [B, S, H, D] of ``dtype`` on ``device`` for
    workload w (a Workload or its name).  rotate=False leaves the video
    recipes' Q and K without their 3D rotary embedding (for a rotation fused
    into the quantizers; ``rope_tables_3d`` gives its tables)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    device = torch.device(device)
    g = torch.Generator(device=device).manual_seed(w.seed)
    rn = lambda *s: torch.randn(*s, generator=g, device=device)  # noqa: E731
    ru = lambda *s: torch.rand(*s, generator=g, device=device)   # noqa: E731
    B, S, H, D = w.B, w.S, w.H, w.D
    shape = (B, S, H, D)
    e = w.extra
    if w.recipe == "offsets":
        q = rn(shape)
        k = rn(shape)
        v = rn(shape)
        if e["k_off_shared"]:
            k += e["k_off"] * rn(D)
        else:
            k += e["k_off"] * rn(1, 1, H, D)
        if e["v_off"]:
            v += e["v_off"] * rn(1, 1, H, D)
        v = _outliers(v, e["out_frac"], e["out_mult"], g)
    elif w.recipe == "rope_drift":
        q = _rms_normalize(rn(shape))
        k = _rms_normalize(rn(shape))
        if rotate:
            q = _rope_3d(q, e["grid"], split=rope_split(D))
            k = _rope_3d(k, e["grid"], split=rope_split(D))
        v = rn(shape)
        amp = 0.5 + 1.5 * ru(1, 1, H, D)
        freq = 0.5 + 3.5 * ru(1, 1, H, D)
        phase = 2.0 * math.pi * ru(1, 1, H, D)
        s = (torch.arange(S, dtype=torch.float32, device=device) / S).view(1, S, 1, 1)
        v += amp * torch.sin(2.0 * math.pi * freq * s + phase)
        v = _outliers(v, e["out_frac"], e["out_mult"], g)
    elif w.recipe == "mixture":
        q = rn(shape)
        v = torch.empty(shape, device=device)
        k = torch.empty(shape, device=device)
        for b in range(B):
            for h in range(H):
                means = e["comp_std"] * rn(e["n_comp"], D)
                lab = torch.randint(0, e["n_comp"], (S,), generator=g, device=device)
                vh = means[lab] + e["noise"] * rn(S, D)
                wq, _ = torch.linalg.qr(rn(D, D).double().cpu())
                kh = vh @ wq.float().to(device) + rn(S, D)
                v[b, :, h, :] = vh
                k[b, :, h, :] = kh
    else:
        raise ValueError(w.recipe)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def head_slices(q, k, v, b, h):
    """float32 numpy [S, D] views of one head of bf16 [B, S, H, D] tensors."""
    return tuple(t[b, :, h, :].float().cpu().numpy() for t in (q, k, v))

"""Thin PyTorch binding of libvsmooth: argument marshalling only.

Every function with a ``vs_`` name mirrors the C entry point of the same
name in include/vsmooth.h: tensors in, device pointers and sizes out, the
call issued on the current HIP stream, a non-zero status raised as VsError.
All arithmetic of the hot path runs in the library's HIP kernels.

``Plan`` preallocates every buffer of one problem size and chains the four
calls in the method's order (grouping, statistics, quantizers, attention);
``attention`` is the one-shot convenience wrapper around it.
"""
import ctypes
import math

import torch

from . import _abi
from ._abi import (VS_EXPCAST, VS_OUT_BF16, VS_BF16_MMA, VS_P_MXFP4, VS_QK_HADAMARD, VS_V_MXFP4, VS_LAYOUT_BHSD, VS_LAYOUT_BSHD, VS_VMEAN_BLOCK,
                   VS_VMEAN_BLOCK_OUT, VS_VMEAN_NONE, VS_VMEAN_SEQ, check, load)

__all__ = ["vs_smooth_stats_workspace_bytes", "vs_smooth_stats", "vs_smooth_stats_ex",
           "vs_smooth_stats_noalloc",
           "vs_quantize_residual",
           "vs_quantize_residual_perm", "vs_quantize_residual_ex",
           "vs_fp8_attn_fwd", "vs_fp8_attn_fwd_pcodes", "vs_kmeans_workspace_bytes", "vs_kmeans_permute",
           "vs_cube_permutation",
           "vs_version", "Plan", "attention"]

_VMEAN = {"none": VS_VMEAN_NONE, "block": VS_VMEAN_BLOCK, "seq": VS_VMEAN_SEQ}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libvsmooth takes device tensors")
            return t.device
    raise ValueError("no tensor given")


def vs_version():
    return load().vs_version().decode()


def vs_smooth_stats_workspace_bytes(B, S, H, D):
    n = ctypes.c_size_t(0)
    check(load().vs_smooth_stats_workspace_bytes(B, S, H, D, ctypes.byref(n)),
          "vs_smooth_stats_workspace_bytes")
    return n.value


def vs_smooth_stats(k, v, shape, layout, k_mean, v_block_mean, v_seq_mean, ws):
    B, S, H, D = shape
    dev = _dev(k, v)
    check(load().vs_smooth_stats(_p(k), _p(v), B, S, H, D, layout, _p(k_mean),
                                 _p(v_block_mean), _p(v_seq_mean), _p(ws),
                                 ws.numel() * ws.element_size() if ws is not None else 0,
                                 _stream(dev)), "vs_smooth_stats")


def vs_smooth_stats_ex(k, v, shape, layout, rope_cos, rope_sin, k_mean, v_block_mean, v_seq_mean,
                       ws):
    B, S, H, D = shape
    dev = _dev(k, v)
    check(load().vs_smooth_stats_ex(_p(k), _p(v), B, S, H, D, layout, _p(rope_cos),
                                    _p(rope_sin), _p(k_mean), _p(v_block_mean), _p(v_seq_mean),
                                    _p(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                    _stream(dev)), "vs_smooth_stats_ex")


def vs_smooth_stats_noalloc(k, v, shape, layout, k_mean, v_block_mean, v_seq_mean):
    B, S, H, D = shape
    dev = _dev(k, v)
    check(load().vs_smooth_stats_noalloc(_p(k), _p(v), B, S, H, D, layout, _p(k_mean),
                                         _p(v_block_mean), _p(v_seq_mean), _stream(dev)),
          "vs_smooth_stats_noalloc")


def vs_quantize_residual(q, k, v, kv_layout, shape, softmax_scale, k_mean, v_mean, vmean_mode,
                         q8, q_scale, k8, k_scale, v8, v_scale, q_mu):
    B, S, H, D = shape
    dev = _dev(q, k, v)
    check(load().vs_quantize_residual(_p(q), _p(k), _p(v), kv_layout, B, S, H, D,
                                      float(softmax_scale), _p(k_mean), _p(v_mean), vmean_mode,
                                      _p(q8), _p(q_scale), _p(k8), _p(k_scale), _p(v8),
                                      _p(v_scale), _p(q_mu), _stream(dev)),
          "vs_quantize_residual")


def vs_quantize_residual_perm(q, k, v, perm, shape, softmax_scale, k_mean, v_mean, vmean_mode,
                              q8, q_scale, k8, k_scale, v8, v_scale, q_mu):
    B, S, H, D = shape
    dev = _dev(q, k, v)
    check(load().vs_quantize_residual_perm(_p(q), _p(k), _p(v), _p(perm), B, S, H, D,
                                           float(softmax_scale), _p(k_mean), _p(v_mean),
                                           vmean_mode, _p(q8), _p(q_scale), _p(k8),
                                           _p(k_scale), _p(v8), _p(v_scale), _p(q_mu),
                                           _stream(dev)),
          "vs_quantize_residual_perm")


def vs_quantize_residual_ex(q, k, v, kv_layout, perm, flags, shape, softmax_scale, k_mean, v_mean,
                            vmean_mode, q8, q_scale, k8, k_scale, v8, v_scale, q_mu,
                            rope_cos=None, rope_sin=None):
    B, S, H, D = shape
    dev = _dev(q, k, v)
    check(load().vs_quantize_residual_ex(_p(q), _p(k), _p(v), kv_layout, _p(perm), int(flags),
                                         B, S, H, D, float(softmax_scale), _p(rope_cos),
                                         _p(rope_sin), _p(k_mean),
                                         _p(v_mean), vmean_mode, _p(q8), _p(q_scale), _p(k8),
                                         _p(k_scale), _p(v8), _p(v_scale), _p(q_mu),
                                         _stream(dev)),
          "vs_quantize_residual_ex")


def vs_fp8_attn_fwd(q8, q_scale, k8, k_scale, v8, v_scale, v_mean, vmean_mode, q_mu, shape,
                    flags, out, lse2):
    B, S, H, D = shape
    dev = _dev(q8, k8, v8)
    check(load().vs_fp8_attn_fwd(_p(q8), _p(q_scale), _p(k8), _p(k_scale), _p(v8), _p(v_scale),
                                 _p(v_mean), vmean_mode, _p(q_mu), B, S, H, D, int(flags),
                                 _p(out), _p(lse2), _stream(dev)), "vs_fp8_attn_fwd")


def vs_fp8_attn_fwd_pcodes(q8, q_scale, k8, k_scale, v8, v_scale, v_mean, vmean_mode, q_mu,
                           shape, flags, out, lse2, p_codes, row_stride):
    B, S, H, D = shape
    dev = _dev(q8, k8, v8)
    check(load().vs_fp8_attn_fwd_pcodes(_p(q8), _p(q_scale), _p(k8), _p(k_scale), _p(v8),
                                        _p(v_scale), _p(v_mean), vmean_mode, _p(q_mu), B, S, H,
                                        D, int(flags), _p(out), _p(lse2), _p(p_codes),
                                        int(row_stride), _stream(dev)),
          "vs_fp8_attn_fwd_pcodes")


def vs_cube_permutation(S, grid, cube):
    """Host call: int32 CPU tensor [S], the static cube grouping of a
    T x Hg x W token grid (include/vsmooth.h)."""
    T, Hg, W = (int(a) for a in grid)
    ct, ch, cw = (int(a) for a in cube)
    perm = torch.empty(max(int(S), 0), dtype=torch.int32)
    check(load().vs_cube_permutation(int(S), T, Hg, W, ct, ch, cw,
                                     _p(perm) if perm.numel() else None), "vs_cube_permutation")
    return perm


def vs_kmeans_workspace_bytes(B, S, H, D, k_clusters):
    n = ctypes.c_size_t(0)
    check(load().vs_kmeans_workspace_bytes(B, S, H, D, k_clusters, ctypes.byref(n)),
          "vs_kmeans_workspace_bytes")
    return n.value


def vs_kmeans_permute(k, v, shape, k_clusters, iters, labels, perm, k_perm, v_perm, ws):
    B, S, H, D = shape
    dev = _dev(k, v)
    check(load().vs_kmeans_permute(_p(k), _p(v), B, S, H, D, k_clusters, iters, _p(labels),
                                   _p(perm), _p(k_perm), _p(v_perm), _p(ws),
                                   ws.numel() * ws.element_size() if ws is not None else 0,
                                   _stream(dev)), "vs_kmeans_permute")


class Plan:
    """All buffers of one problem, allocated once; ``run`` launches the path.

    shape (B, S, H, D); smooth: K centring + V mean removal; vmean: "block"
    or "seq" (ignored when smooth is False); kmeans: (k, iters) or None;
    expcast: ExpCast-FP8 P cast; fused_gather (with kmeans): the quantizers
    read K and V through the permutation (vs_quantize_residual_perm) instead
    of a gathered copy (vs_kmeans_permute's k_perm / v_perm, then allocated);
    cube: ((T, Hg, W), (ct, ch, cw)) groups the tokens by the static
    spatiotemporal-cube permutation instead (formed once, here);
    qk_hadamard: Q and the centred K rotated by the Hadamard matrix before
    quantization (VS_QK_HADAMARD); v_format: "e4m3" or "mxfp4" (the V
    residual as E2M1 codes with an E8M0 scale per 32 tokens and channel,
    VS_V_MXFP4: v8 is then u8 [B,H,nb,D,64] and v_scale u8 [B,H,nb,D,4]);
    out_dtype: torch.float32 or torch.bfloat16 (VS_OUT_BF16); mma: "fp8"
    (QK^T and PV on the FP8 matrix core from the E4M3 / E2M1 codes) or
    "bf16" (VS_BF16_MMA: the quantizers write the same quantized values
    times their scales as bf16 -- q8, k8 bf16 [B,H,S_pad,D], v8 bf16
    [B,H,nb,D,128] in the bf16 PV's token order -- and both products run on
    the bf16 matrix core, float32-accurate); rope: (cos, sin) float32
    [S, D/2] device tables, or None: q and k are given before their rotary
    embedding, which the statistics pass and the Q/K quantizers apply on
    the fly (vs_smooth_stats_ex, vs_quantize_residual_ex), so the rotated
    Q and K are never written; p_format: "e4m3" or "mxfp4" (the 4-bit
    probability tile, VS_P_MXFP4: E2M1 P with an E8M0 exponent per 32 keys
    of a tile; v8 then holds V's codes in token order).
    """

    def __init__(self, shape, device, *, softmax_scale=None, smooth=True, vmean="block",
                 kmeans=None, expcast=False, fused_gather=True, cube=None, qk_hadamard=False,
                 v_format="e4m3", out_dtype=torch.float32, mma="fp8", rope=None,
                 p_format="e4m3"):
        B, S, H, D = shape
        self.shape = tuple(int(x) for x in shape)
        self.device = torch.device(device)
        self.softmax_scale = float(softmax_scale) if softmax_scale else 1.0 / math.sqrt(D)
        self.smooth = smooth
        self.vmean_mode = _VMEAN[vmean] if smooth else VS_VMEAN_NONE
        self.kmeans = kmeans
        if v_format not in ("e4m3", "mxfp4"):
            raise ValueError(f"unknown v_format {v_format!r}")
        self.v_format = v_format
        v4 = VS_V_MXFP4 if v_format == "mxfp4" else 0
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("out_dtype must be torch.float32 or torch.bfloat16")
        if mma not in ("fp8", "bf16"):
            raise ValueError(f"unknown mma {mma!r}")
        self.mma = mma
        b16 = VS_BF16_MMA if mma == "bf16" else 0
        if p_format not in ("e4m3", "mxfp4"):
            raise ValueError(f"unknown p_format {p_format!r}")
        self.p_format = p_format
        p4 = VS_P_MXFP4 if p_format == "mxfp4" else 0
        if p4 and (expcast or v4 or b16):
            raise ValueError("the 4-bit probability tile runs with E4M3 V on the FP8 "
                             "matrix core, without ExpCast")
        # with the bf16 products attention takes V as bf16 values, whatever
        # format quantized them
        self.flags = ((VS_EXPCAST if expcast else 0) | (0 if b16 else v4) | b16 | p4 |
                      (VS_OUT_BF16 if out_dtype == torch.bfloat16 else 0))
        self.quant_flags = (VS_QK_HADAMARD if qk_hadamard else 0) | v4 | b16 | p4
        nb = (S + 127) // 128
        dev = self.device
        f32, u8, i32 = torch.float32, torch.uint8, torch.int32
        e = lambda *s, dtype=f32: torch.empty(*s, dtype=dtype, device=dev)  # noqa: E731
        qkt = torch.bfloat16 if b16 else u8
        self.q8, self.k8 = e(B, H, nb * 128, D, dtype=qkt), e(B, H, nb * 128, D, dtype=qkt)
        self.q_scale, self.k_scale = e(B, H, nb), e(B, H, nb)
        if v4:
            self.v8, self.v_scale = e(B, H, nb, D, 64, dtype=u8), e(B, H, nb, D, 4, dtype=u8)
        else:
            self.v8, self.v_scale = e(B, H, nb, D, 128, dtype=u8), e(B, H, nb)
        if b16:
            self.v8 = e(B, H, nb, D, 128, dtype=torch.bfloat16)
        self.out, self.lse2 = e(B, S, H, D, dtype=out_dtype), e(B, H, S)
        self.k_mean = self.q_mu = self.v_mean = self.stats_ws = None
        if smooth:
            self.k_mean = e(B, H, D)
            self.q_mu = e(B, H, S)
            self.v_mean = e(B, H, nb, D) if self.vmean_mode == VS_VMEAN_BLOCK else e(B, H, D)
            self.stats_ws = e(vs_smooth_stats_workspace_bytes(B, S, H, D), dtype=u8)
        self.rope_cos = self.rope_sin = None
        if rope is not None:
            cos, sin = rope
            for t in (cos, sin):
                if (tuple(t.shape) != (S, D // 2) or t.dtype != torch.float32
                        or not t.is_contiguous() or t.device != dev):
                    raise ValueError(f"rope tables must be contiguous float32 [{S}, {D // 2}] "
                                     "on the plan's device")
            if kmeans is not None and not fused_gather:
                raise ValueError("rope needs the fused gather: a gathered K copy has lost "
                                 "the token positions its rotation angles depend on")
            self.rope_cos, self.rope_sin = cos, sin
        self.labels = self.perm = self.k_perm = self.v_perm = self.km_ws = None
        self.cube = cube
        self._grouped = False
        if kmeans is not None and cube is not None:
            raise ValueError("kmeans and cube grouping are exclusive")
        if cube is not None:
            grid, dims = cube
            p = vs_cube_permutation(S, grid, dims).to(dev)
            self.perm = p.expand(B, H, S).contiguous()
            self._grouped = True
        if kmeans is not None:
            kc, _ = kmeans
            self.labels, self.perm = e(B, H, S, dtype=i32), e(B, H, S, dtype=i32)
            if not fused_gather:
                self.k_perm = e(B, H, S, D, dtype=torch.bfloat16)
                self.v_perm = e(B, H, S, D, dtype=torch.bfloat16)
            self.km_ws = e(vs_kmeans_workspace_bytes(B, S, H, D, kc), dtype=u8)

    def run(self, q, k, v, regroup=True):
        """Launch the whole path on the current stream; returns (out, lse2).

        regroup=False (k-means plans with the fused gather) keeps the
        permutation of the previous call instead of clustering again (the
        pages' amortized grouping reuses it across adjacent steps)."""
        shape = self.shape
        if tuple(q.shape) != shape or tuple(k.shape) != shape or tuple(v.shape) != shape:
            raise ValueError(f"expected q, k, v of shape {shape}")
        for t in (q, k, v):
            if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.device != self.device:
                raise ValueError("q, k, v must be contiguous bf16 tensors on the plan's device")
        layout = VS_LAYOUT_BSHD
        kk, vv = k, v
        if not regroup and self.k_perm is not None:
            raise ValueError("reusing a permutation needs the fused gather")
        if self.kmeans is not None and (regroup or not self._grouped):
            kc, iters = self.kmeans
            vs_kmeans_permute(k, v, shape, kc, iters, self.labels, self.perm, self.k_perm,
                              self.v_perm, self.km_ws)
            self._grouped = True
            if self.k_perm is not None:
                kk, vv, layout = self.k_perm, self.v_perm, VS_LAYOUT_BHSD
        qmode = self.vmean_mode
        if self.smooth:
            # block means come out of the V quantizer (VS_VMEAN_BLOCK_OUT), so
            # the statistics pass reads K only; the sequence mean needs V here
            seq = self.v_mean if self.vmean_mode == VS_VMEAN_SEQ else None
            vs_smooth_stats_ex(kk, vv if seq is not None else None, shape, layout,
                               self.rope_cos, self.rope_sin, self.k_mean, None, seq,
                               self.stats_ws)
            if self.vmean_mode == VS_VMEAN_BLOCK:
                qmode = VS_VMEAN_BLOCK_OUT
        # with a permutation and no gathered copy the quantizers read K and V
        # rows through it (the K mean, permutation-invariant, came from the
        # unpermuted K)
        perm = self.perm if (self.perm is not None and self.k_perm is None) else None
        vs_quantize_residual_ex(q, kk, vv, layout, perm, self.quant_flags, shape,
                                self.softmax_scale, self.k_mean, self.v_mean, qmode, self.q8,
                                self.q_scale, self.k8, self.k_scale, self.v8, self.v_scale,
                                self.q_mu, self.rope_cos, self.rope_sin)
        self.attn()
        return self.out, self.lse2

    def attn(self):
        """The attention call alone, on the buffers the last ``run`` filled."""
        vs_fp8_attn_fwd(self.q8, self.q_scale, self.k8, self.k_scale, self.v8, self.v_scale,
                        self.v_mean, self.vmean_mode, self.q_mu, self.shape, self.flags,
                        self.out, self.lse2)

    def attn_pcodes(self, row_stride):
        """The attention call again, also returning the E4M3 probability codes
        of every row_stride-th query row: u8 [B, H, ceil(S/stride), S_pad], the
        codes of key t at column t (vs_fp8_attn_fwd_pcodes, a diagnostic)."""
        B, S, H, D = self.shape
        nb = (S + 127) // 128
        n = (S + row_stride - 1) // row_stride
        codes = torch.zeros(B, H, n, nb * 128, dtype=torch.uint8, device=self.device)
        vs_fp8_attn_fwd_pcodes(self.q8, self.q_scale, self.k8, self.k_scale, self.v8,
                               self.v_scale, self.v_mean, self.vmean_mode, self.q_mu, self.shape,
                               self.flags, self.out, self.lse2, codes, row_stride)
        return codes


def attention(q, k, v, **kw):
    """One-shot: build a Plan for q's shape and run it; returns (out, lse2)."""
    plan = Plan(tuple(q.shape), q.device, **kw)
    return plan.run(q, k, v)

"""Benchmark of the FP8 smoothed-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload live]

A step is one pass of the whole path over one batch of synthetic input that
is already resident in HBM: (k-means grouping when the workload has it) ->
exact K/V statistics -> per-block E4M3 quantizers -> FP8 attention; on the
video workloads Q and K arrive before their 3D rotary embedding, which the
statistics pass and the quantizers apply on load (--rope pre: inputs
rotated beforehand).  The
default workload is the live DiT layer shape S=32626, H=56, D=128, B=1.

Prints ONE JSON line.  ``value`` is whole-step throughput in the metric's
unit, 4*B*S^2*D*H / step time.  ``roofline`` is the attention kernel alone,
timed with HIP events on the stream it is launched on, against MI355X's
dense FP8 MFMA peak.  ``cpu_baseline`` is the NumPy oracle timed on the
host on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 smoothed-attn TFLOP/s (4·S²·D·H) and % FP8 MFMA peak, S=32626 H=56 D=128"
FP8_PEAK_TFLOPS = 5000.0          # MI355X dense FP8 MFMA, published
HBM_PEAK_GBS = 8000.0
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attn_fwd_live_traffic.json")


def _traffic(workload, expcast, v_format="e4m3", mma="fp8", p_format="e4m3"):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    record (FETCH_SIZE / WRITE_SIZE, scaled by a 1 GiB copy), or None when the
    record is for another workload or kernel variant, or the kernel sources
    changed since."""
    import hashlib
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
        if (rec.get("workload") != workload or expcast or v_format != "e4m3" or mma != "fp8"
                or p_format != "e4m3"):
            return None
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return int(rec["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def _cpu_baseline(w, q, k, v, rows_n, expcast, qk_hadamard=False, v_format="e4m3", rope=None,
                  p_format="e4m3"):
    """Time the oracle (plain NumPy, float64) on one head: quantization of
    that head's full Q/K/V plus the tiled FP8 recurrence for ``rows_n``
    evenly spaced query rows over the whole K/V context.  Throughput counted
    as 4 * rows * S * D flops.  ``cores`` is the number of threads the BLAS
    library ran with (the oracle's matrix products are its only parallel
    part); the host's logical CPU count and model are recorded next to it."""
    import workloads
    from oracle import pipeline
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    qh, kh, vh = workloads.head_slices(q, k, v, 0, 0)
    rows = pipeline.sample_rows(w.S, rows_n)
    t0 = time.perf_counter()
    pipeline.smoothed_attention_head(qh, kh, vh, rows=rows, kmeans_kt=w.kmeans,
                                     expcast=expcast, qk_hadamard=qk_hadamard,
                                     v_format=v_format, rope=rope, p_format=p_format)
    dt = time.perf_counter() - t0
    flops = 4.0 * len(rows) * w.S * w.D
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "host_cpu_count": os.cpu_count(), "host_cpu_model": _cpu_model(),
            "sample": f"head 0 of {w.name} (S={w.S}, D={w.D}): "
                      f"{'rotary embedding, ' if rope is not None else ''}full-head statistics and "
                      f"quantizers (V {v_format}{', QK Hadamard' if qk_hadamard else ''})"
                      f"{' and k-means' if w.kmeans else ''}, then the "
                      f"tiled recurrence for {len(rows)} query rows over all {w.S} keys; "
                      f"{dt:.1f} s wall; flops counted 4*rows*S*D"}


def _settle(run, dev, seconds=0.3):
    """Back-to-back launches for `seconds`, so that the clock reached under
    sustained load (power management reacts over tens of milliseconds) is
    what the timed launches see."""
    import time
    import torch
    t0 = time.time()
    while time.time() - t0 < seconds:
        for _ in range(4):
            run()
        torch.cuda.synchronize(dev)


def _mfma_loop_rates(dev, timed):
    """The matrix core on its own: libvsmooth_peak.so's loop of independent
    FP8 (32x32x64) or bf16 (32x32x16) products on register operands (random
    operand bytes, different for each of the eight accumulators), one wave
    per SIMD, timed after 0.3 s of sustained load.  Returns TFLOP/s, the
    shader clock (s_memtime ticks over event time) and the matrix core's
    cycles per product."""
    import ctypes
    import torch
    from bit_attention_video_smooth_amd.build import PEAK_LIB

    if not os.path.exists(PEAK_LIB):
        return {"mfma_loop": "libvsmooth_peak.so not built"}
    lib = ctypes.CDLL(PEAK_LIB)
    fn = lib.vs_peak_mfma_loop
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 3
    out = {}
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for kind, name, flops in ((0, "fp8", 2 * 32 * 32 * 64), (1, "bf16", 2 * 32 * 32 * 16)):
        # one workgroup of four waves per CU: one wave per SIMD, all resident
        for threads, blocks in ((256, 256),):
            iters = 40000 if kind == 0 else 80000
            waves = blocks * threads // 64
            ticks = torch.zeros(waves, dtype=torch.int64, device=dev)
            sink = torch.zeros(waves, dtype=torch.float32, device=dev)

            def run():
                rc = fn(kind, blocks, threads, iters, ctypes.c_void_p(ticks.data_ptr()),
                        ctypes.c_void_p(sink.data_ptr()), stream)
                if rc != 0:
                    raise RuntimeError(f"vs_peak_mfma_loop returned {rc}")
            _settle(run, dev)
            t = timed(run, n=5)
            tk = float(ticks.double().mean().item())      # each wave's loop, shader cycles
            per_simd = waves // 1024
            out[f"{name}_mfma_loop_{per_simd}w_tflops"] = round(waves * iters * 8 * flops / t / 1e12, 1)
            out[f"{name}_mfma_loop_{per_simd}w_clock_ghz"] = round(tk / t / 1e9, 3)
            out[f"{name}_mfma_loop_{per_simd}w_cycles_per_product"] = round(tk / (iters * 8 * per_simd), 1)
    return out


def _mix_loop_clocks(dev):
    """The clock each phase mix of the attention kernel holds under sustained
    load (libvsmooth_peak.so's vs_peak_mix_loop, eight waves per CU): FP8
    products with register operands, the same products with their A operand
    read from LDS (2 KB per product, as in the matrix-core phase), the vector
    phase's mix (max3 chain, exp2, E4M3 packs, row-sum adds), and products
    from LDS co-running with the vector mix on every SIMD; random operand
    bytes, the last launch after 0.3 s of sustained load.  Each wave's
    clock is its s_memtime ticks over its s_memrealtime (100 MHz) ticks."""
    import ctypes
    import torch
    from bit_attention_video_smooth_amd.build import PEAK_LIB

    if not os.path.exists(PEAK_LIB):
        return {"mix_loop": "libvsmooth_peak.so not built"}
    lib = ctypes.CDLL(PEAK_LIB)
    fn = lib.vs_peak_mix_loop
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    blocks = 256                        # one workgroup of eight waves per CU
    n = blocks * 8
    ticks = torch.zeros(n, dtype=torch.int64, device=dev)
    rticks = torch.zeros(n, dtype=torch.int64, device=dev)
    sink = torch.zeros(n, dtype=torch.float32, device=dev)
    out = {}
    for kind, name in ((3, "products_reg"), (0, "products_lds"), (1, "vector_mix"),
                       (2, "products_lds+vector_mix")):
        iters_p, iters_v = 20000, 8000

        def run():
            rc = fn(kind, blocks, iters_p, iters_v, ctypes.c_void_p(ticks.data_ptr()),
                    ctypes.c_void_p(rticks.data_ptr()), ctypes.c_void_p(sink.data_ptr()), stream)
            if rc != 0:
                raise RuntimeError(f"vs_peak_mix_loop returned {rc}")
        _settle(run, dev)
        torch.cuda.synchronize(dev)
        tk = ticks.double().cpu()
        rt = rticks.double().cpu()
        wave_in_wg = torch.arange(n) % 8
        if kind == 2:
            roles = (("_products", wave_in_wg < 4, iters_p), ("_vector", wave_in_wg >= 4, iters_v))
        else:
            roles = (("", wave_in_wg >= 0, iters_v if kind == 1 else iters_p),)
        for suffix, sel, it in roles:
            out[f"mix_{name}{suffix}_clock_ghz"] = round((tk[sel] / rt[sel] * 0.1).median().item(), 3)
            out[f"mix_{name}{suffix}_cycles_per_turn"] = round(tk[sel].median().item() / it, 1)
        if kind in (0, 3):
            # every wave's eight products per turn over the slowest wave's time
            secs = rt.max().item() / 1e8
            out[f"mix_{name}_tflops"] = round(n * iters_p * 8 * 2 * 32 * 32 * 64 / secs / 1e12, 1)
    return out


def _peaks(dev):
    """Practical ceilings on this machine next to the published peaks: the
    vendor library's dense FP8 (E4M3) and bf16 GEMMs (torch._scaled_mm /
    torch.matmul through hipBLASLt) and a large device-to-device copy, each
    timed with HIP events after warm-up."""
    import torch

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize(dev)
        return e0.elapsed_time(e1) / n * 1e-3

    out = {}
    for n in (8192, 16384):
        a = torch.randn(n, n, device=dev).to(torch.float8_e4m3fn)
        b = torch.randn(n, n, device=dev).to(torch.float8_e4m3fn).t()   # column-major B
        one = torch.ones((), device=dev)
        try:
            t = timed(lambda: torch._scaled_mm(a, b, scale_a=one, scale_b=one,
                                               out_dtype=torch.bfloat16))
            out[f"fp8_gemm_{n}_tflops"] = round(2.0 * n ** 3 / t / 1e12, 1)
        except Exception as exc:            # not every build exposes FP8 GEMMs
            out[f"fp8_gemm_{n}_tflops"] = f"unavailable: {type(exc).__name__}"
        x = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        y = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        t = timed(lambda: torch.matmul(x, y))
        out[f"bf16_gemm_{n}_tflops"] = round(2.0 * n ** 3 / t / 1e12, 1)
        del a, b, x, y
    out.update(_mfma_loop_rates(dev, timed))
    out.update(_mix_loop_clocks(dev))
    src = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    t = timed(lambda: dst.copy_(src), n=10)
    out["copy_4GiB_gbs"] = round(2.0 * src.numel() / t / 1e9, 1)   # read + write
    out["published"] = {"fp8_dense_tflops": FP8_PEAK_TFLOPS, "bf16_dense_tflops": 2500.0,
                        "hbm_gbs": HBM_PEAK_GBS}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="live")
    ap.add_argument("--expcast", type=int, default=None, help="override the workload's ExpCast flag")
    ap.add_argument("--gather", choices=["fused", "copy"], default="fused",
                    help="k-means workloads: quantizers read K/V through the permutation "
                         "(fused) or a gathered copy")
    ap.add_argument("--reuse-perm", action="store_true",
                    help="k-means workloads: timed steps keep the warm-up's permutation "
                         "(grouping amortized away)")
    ap.add_argument("--qk-hadamard", action="store_true",
                    help="rotate Q and the centred K by the Hadamard matrix in the quantizers")
    ap.add_argument("--v-format", choices=["e4m3", "mxfp4"], default="e4m3",
                    help="V residual format (mxfp4: E2M1 codes, E8M0 scale per 32 tokens)")
    ap.add_argument("--mma", choices=["fp8", "bf16"], default="fp8",
                    help="products on the FP8 matrix core (default) or the bf16 one "
                         "(float32-accurate sums of the same quantized operands)")
    ap.add_argument("--p-format", choices=["e4m3", "mxfp4"], default="e4m3",
                    help="probability tile: E4M3 (default) or 4-bit (E2M1 with an E8M0 "
                         "exponent per 32 keys)")
    ap.add_argument("--rope", choices=["fused", "pre"], default="fused",
                    help="video workloads: Q/K given before their 3D rotary embedding, which "
                         "the statistics pass and the quantizers apply (fused), or given "
                         "already rotated (pre)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the box's practical ceilings (library FP8/bf16 GEMMs, "
                         "device copy) and print them as one JSON line")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a known-size "
                         "kernel that scales FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards over (batch, head) with no exchange, so N GPUs run N "
              "independent shares - not measured here.", file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_attention_video_smooth_amd as vs
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.peaks:
        print(json.dumps({"peaks": _peaks(dev)}), flush=True)
        return
    w = workloads.WORKLOADS[args.workload]
    expcast = w.expcast if args.expcast is None else bool(args.expcast)
    print(f"[bench] generating {w.name} S={w.S} H={w.H} D={w.D} on the GPU", file=sys.stderr, flush=True)
    rope = None
    if "grid" in w.extra and args.rope == "fused":
        rope = workloads.rope_tables_3d(w.S, w.D, w.extra["grid"], device=dev)
    q, k, v = workloads.generate(w, device=dev, rotate=rope is None)
    plan = vs.Plan((w.B, w.S, w.H, w.D), dev, kmeans=w.kmeans, expcast=expcast,
                   fused_gather=args.gather == "fused", qk_hadamard=args.qk_hadamard,
                   v_format=args.v_format, mma=args.mma, rope=rope, p_format=args.p_format)
    regroup = not (args.reuse_perm and w.kmeans)
    torch.cuda.synchronize(dev)
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    for _ in range(args.warmup):
        plan.run(q, k, v)
    torch.cuda.synchronize(dev)
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # whole-path steps
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plan.run(q, k, v, regroup=regroup)
    torch.cuda.synchronize(dev)
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    # attention kernel alone: HIP events on the current stream, which is the
    # stream the binding launches on
    # (one event pair per launch: the mean is the roofline's launch duration,
    # the median the figure the pages quote, 20 runs after warm-up)
    stream = torch.cuda.current_stream(dev)
    n_attn = max(args.steps, 20)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_attn)]
    for e0, e1 in evs:
        e0.record(stream)
        plan.attn()
        e1.record(stream)
    torch.cuda.synchronize(dev)
    per = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    attn_ms = sum(per) / len(per)
    attn_med = per[len(per) // 2] if len(per) % 2 else 0.5 * (per[len(per) // 2 - 1] + per[len(per) // 2])
    attn_tflops = w.flops / (attn_ms * 1e-3) / 1e12
    print(f"[bench] attention kernel: {attn_ms:.3f} ms mean, {attn_med:.3f} ms median of {n_attn}, "
          f"{attn_tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)

    value = w.flops / (ms_step * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3" if args.v_format == "e4m3" else "fp8e4m3 (V: mxfp4)")
                 + ("" if args.p_format == "e4m3" else " (P: mxfp4)")
                 + ("" if args.mma == "fp8" else " operands, bf16 products"),
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} S={w.S} H={w.H} D={w.D}",
                   "kmeans": list(w.kmeans) if w.kmeans else None, "expcast": expcast,
                   "gather": args.gather if w.kmeans else None,
                   "grouping_per_step": bool(w.kmeans) and regroup,
                   "qk_hadamard": bool(args.qk_hadamard),
                   "rope": None if "grid" not in w.extra else
                           ("3D, fused into statistics and quantizers" if rope is not None
                            else "3D, applied to the inputs before the step"),
                   "v_format": args.v_format,
                   "p_format": args.p_format,
                   "products": "FP8 matrix core" if args.mma == "fp8" else "bf16 matrix core",
                   "smoothing": "K seq-mean centring + V block-mean restore",
                   "pct_fp8_peak_whole_step": round(100.0 * value / FP8_PEAK_TFLOPS, 2),
                   "attn_ms": round(attn_ms, 4),
                   "attn_ms_median": round(attn_med, 4), "attn_launches": n_attn,
                   "prep_ms": round(ms_step - attn_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": _traffic(w.name, expcast, args.v_format, args.mma,
                                         args.p_format)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        tables = None if rope is None else tuple(t.cpu().numpy() for t in rope)
        line["cpu_baseline"] = _cpu_baseline(w, q, k, v, args.cpu_rows, expcast,
                                             args.qk_hadamard, args.v_format, tables,
                                             args.p_format)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Build libvsmooth.so for gfx950 with hipcc (in-tree, next to this file).

    python -m bit_attention_video_smooth_amd.build

Each .hip source compiles to an object in parallel, then one shared library
is linked.  Packed-FP32 instruction forms are disabled for all device code.
The matrix-core rate microbenchmark (csrc/mfma_peak.hip, used by bench.py
--peaks only) links into its own libvsmooth_peak.so.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libvsmooth.so")
SOURCES = ["status.hip", "smooth_stats.hip", "quantize.hip", "attn_fwd.hip", "kmeans.hip",
           "grouping.hip"]
PEAK_SOURCE = "mfma_peak.hip"
PEAK_LIB = os.path.join(HERE, "libvsmooth_peak.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source extra flags: the microbenchmark's vector loop takes maxima of
# register values the compiler cannot prove quiet, and would quiet every
# input first; without NaN handling its loop is the attention kernel's mix.
EXTRA = {PEAK_SOURCE: ["-fno-honor-nans"]}


def _compile(src, obj):
    cmd = [HIPCC, *CFLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libvsmooth.so; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = SOURCES + [PEAK_SOURCE]
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(_compile, srcs, objs))
    peak_obj = objs.pop()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, peak_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, PEAK_LIB)
    shutil.rmtree(objdir, ignore_errors=True)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

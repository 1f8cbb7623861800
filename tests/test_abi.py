"""The C ABI without a GPU: the library loads, exports every entry point that
include/vsmooth.h declares, and rejects bad arguments on the host before
anything would be launched (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsmooth.h")


@pytest.fixture(scope="module")
def lib():
    from bit_attention_video_smooth_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        from bit_attention_video_smooth_amd import build
        build.build()
    return _abi.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vs_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls_and_helpers():
    names = _declared()
    for n in ["vs_smooth_stats", "vs_kmeans_permute", "vs_quantize_residual", "vs_fp8_attn_fwd"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from bit_attention_video_smooth_amd import _abi
    for n in _declared():
        assert hasattr(lib, n), n
        assert n in _abi.PROTOTYPES, n


def test_status_and_version(lib):
    assert lib.vs_version().decode().count(".") == 2
    for s in range(5):
        assert lib.vs_status_string(s).decode().startswith("VS_")
    assert b"unknown" in lib.vs_status_string(99)


def test_workspace_queries(lib):
    n = ctypes.c_size_t(0)
    assert lib.vs_smooth_stats_workspace_bytes(1, 32626, 56, 128, ctypes.byref(n)) == 0
    assert n.value == 2 * 56 * 255 * 128 * 8
    assert lib.vs_kmeans_workspace_bytes(1, 32760, 40, 128, 16, ctypes.byref(n)) == 0
    assert n.value >= 40 * 32760 * 128            # the int8 codes
    assert lib.vs_kmeans_workspace_bytes(1, 100, 1, 128, 257, ctypes.byref(n)) == 2
    assert lib.vs_kmeans_workspace_bytes(1, 100, 1, 96, 16, ctypes.byref(n)) == 2
    assert lib.vs_smooth_stats_workspace_bytes(1, 100, 1, 128, None) == 1


def test_attn_argument_errors(lib):
    f = lib.vs_fp8_attn_fwd
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: validation fails first
    args = lambda **kw: [kw.get("q8", fake), fake, fake, fake, fake, fake,  # noqa: E731
                         kw.get("vm", None), kw.get("mode", 0), None, kw.get("B", 1),
                         kw.get("S", 256), 1, kw.get("D", 128), kw.get("flags", 0), fake, fake,
                         None]
    assert f(*args(D=96)) == 2
    assert f(*args(q8=None)) == 1
    assert f(*args(B=-1)) == 1
    assert f(*args(mode=1)) == 1                      # block mean without a buffer
    assert f(*args(mode=7, vm=fake)) == 1
    assert f(*args(flags=32)) == 1
    assert f(*args(flags=16 | 1)) == 1                 # 4-bit P with ExpCast
    assert f(*args(flags=16 | 2)) == 1                 # 4-bit P with MXFP4 V
    assert f(*args(flags=16 | 8)) == 1                 # 4-bit P with bf16 products
    assert f(*args(flags=16, D=96)) == 2               # 4-bit P: a valid flag
    assert f(*args(flags=4, D=96)) == 2                # bf16 output: a valid flag
    assert f(*args(flags=8, D=96)) == 2                # bf16 QK operands: a valid flag
    assert f(*args(flags=3, D=96)) == 2                # ExpCast with MXFP4 V: a valid flag pair
    assert f(*args(q8=ctypes.c_void_p(0x1004))) == 2  # misaligned
    assert f(*args(S=0)) == 0                         # empty problem
    assert f(*args(S=0, D=96)) == 2


def test_noalloc_stats_limit_is_checked_before_any_launch(lib):
    """vs_smooth_stats_noalloc rejects a problem whose block sums exceed its
    32 MiB array with VS_ERR_WORKSPACE, and bad arguments as vs_smooth_stats
    does, all on the host (no GPU touched)."""
    from bit_attention_video_smooth_amd import _abi
    fake = ctypes.c_void_p(0x1000)
    f = lib.vs_smooth_stats_noalloc
    n = ctypes.c_size_t(0)
    assert lib.vs_smooth_stats_workspace_bytes(1, 115328, 56, 128, ctypes.byref(n)) == 0
    assert n.value > _abi.VS_NOALLOC_STATS_SCRATCH_BYTES
    assert f(fake, None, 1, 115328, 56, 128, 0, fake, None, None, None) == 3
    assert lib.vs_smooth_stats_workspace_bytes(1, 32626, 56, 128, ctypes.byref(n)) == 0
    assert n.value <= _abi.VS_NOALLOC_STATS_SCRATCH_BYTES          # the live shape fits
    assert f(fake, None, 1, 300, 2, 96, 0, fake, None, None, None) == 2
    assert f(fake, None, 1, 300, 2, 128, 0, fake, fake, None, None) == 1   # V mean without V
    assert f(fake, fake, 1, 300, 2, 128, 5, fake, None, None, None) == 1   # bad layout
    assert f(fake, fake, 1, 0, 2, 128, 0, fake, None, None, None) == 0     # empty problem


def test_pcodes_argument_errors(lib):
    """The diagnostic entry point: a code buffer and a positive stride are
    required, MXFP4 V is not supported; all rejected on the host."""
    f = lib.vs_fp8_attn_fwd_pcodes
    fake = ctypes.c_void_p(0x1000)
    args = lambda **kw: [fake, fake, fake, fake, fake, fake, None, 0, None, 1, 256, 1,  # noqa: E731
                         kw.get("D", 128), kw.get("flags", 0), fake, fake,
                         kw.get("codes", fake), kw.get("stride", 1), None]
    assert f(*args(codes=None)) == 1
    assert f(*args(stride=0)) == 1
    assert f(*args(flags=2)) == 2
    assert f(*args(flags=16)) == 2                       # no code buffer for 4-bit P
    assert f(*args(D=96)) == 2


def test_quant_stats_kmeans_argument_errors(lib):
    fake = ctypes.c_void_p(0x1000)
    q = lib.vs_quantize_residual
    base = [fake, fake, fake, 0, 1, 300, 2, 128, 0.1, None, None, 0,
            fake, fake, fake, fake, fake, fake, None, None]
    bad = list(base); bad[3] = 5
    assert q(*bad) == 1                                # bad layout
    bad = list(base); bad[9] = fake
    assert q(*bad) == 1                                # k_mean without q_mu
    bad = list(base); bad[11] = 1
    assert q(*bad) == 1                                # vmean block without buffer
    bad = list(base); bad[11] = 3
    assert q(*bad) == 1                                # block means out without buffer
    bad = list(base); bad[11] = 4; bad[10] = fake
    assert q(*bad) == 1                                # no such mode
    bad = list(base); bad[7] = 32
    assert q(*bad) == 2
    s = lib.vs_smooth_stats
    assert s(fake, fake, 1, 300, 2, 128, 0, None, None, None, fake, 1 << 30, None) == 1
    assert s(fake, None, 1, 300, 2, 128, 0, fake, fake, None, fake, 1 << 30, None) == 1  # V mean, no V
    assert s(fake, None, 1, 300, 2, 128, 0, fake, None, fake, fake, 1 << 30, None) == 1
    assert s(fake, fake, 1, 300, 2, 128, 0, fake, None, None, fake, 16, None) == 3
    assert s(fake, fake, 1, 300, 2, 128, 0, fake, None, None, None, 1 << 30, None) == 3
    qp = lib.vs_quantize_residual_perm
    assert qp(fake, fake, fake, None, 1, 300, 2, 128, 0.1, None, None, 0,
              fake, fake, fake, fake, fake, fake, None, None) == 1   # no permutation
    assert qp(fake, fake, fake, fake, 1, 300, 2, 32, 0.1, None, None, 0,
              fake, fake, fake, fake, fake, fake, None, None) == 2
    assert qp(fake, fake, fake, None, 1, 0, 2, 128, 0.1, None, None, 0,
              fake, fake, fake, fake, fake, fake, None, None) == 0   # empty problem
    qe = lib.vs_quantize_residual_ex
    ex = lambda **kw: [fake, fake, fake, kw.get("layout", 0), kw.get("perm", None),  # noqa: E731
                       kw.get("flags", 0), 1, 300, 2, kw.get("D", 128), 0.1,
                       kw.get("cos", None), kw.get("sin", None), None, None, 0,
                       fake, fake, fake, fake, fake, fake, None, None]
    assert qe(*ex(layout=1, perm=fake)) == 1            # a permutation needs BSHD input
    assert qe(*ex(flags=4)) == 1                        # no such flag
    assert qe(*ex(flags=32)) == 1
    assert qe(*ex(flags=16 | 2)) == 1                   # token-order V is E4M3 only
    assert qe(*ex(flags=16 | 8)) == 1
    assert qe(*ex(flags=16, D=96)) == 2                 # 4-bit P's V layout: a valid flag
    assert qe(*ex(flags=8, D=96)) == 2                  # bf16 Q/K: a valid flag
    assert qe(*ex(flags=1, D=96)) == 2
    assert qe(*ex(cos=fake)) == 1                       # rotary tables come in pairs
    assert qe(*ex(sin=fake)) == 1
    assert qe(*ex(cos=fake, sin=fake, D=96)) == 2
    assert qe(*ex(cos=ctypes.c_void_p(0x1004), sin=fake)) == 2         # tables must be 16-byte aligned
    se = lib.vs_smooth_stats_ex
    assert se(fake, fake, 1, 300, 2, 128, 0, fake, None, fake, None, None, fake, 1 << 30,
              None) == 1                                # rotary tables come in pairs
    assert se(fake, fake, 1, 300, 2, 128, 0, fake, ctypes.c_void_p(0x1008), fake, None, None, fake, 1 << 30,
              None) == 2
    assert se(fake, fake, 1, 300, 2, 128, 0, fake, fake, fake, None, None, fake, 16, None) == 3
    assert se(fake, fake, 1, 0, 2, 128, 0, fake, fake, fake, None, None, None, 0, None) == 0
    k = lib.vs_kmeans_permute
    assert k(fake, fake, 1, 300, 2, 128, 16, 2, fake, fake, fake, None, fake, 1 << 30, None) == 1
    assert k(fake, fake, 1, 300, 2, 128, 16, 0, fake, fake, fake, fake, fake, 1 << 30, None) == 1
    assert k(fake, fake, 1, 300, 2, 128, 300, 2, fake, fake, fake, fake, fake, 1 << 30, None) == 2
    assert k(fake, fake, 1, 300, 2, 128, 16, 2, fake, fake, fake, fake, fake, 64, None) == 3


def test_header_constants_match_the_binding():
    from bit_attention_video_smooth_amd import _abi
    text = open(HEADER).read()
    for name in ["VS_VMEAN_NONE", "VS_VMEAN_BLOCK", "VS_VMEAN_SEQ", "VS_VMEAN_BLOCK_OUT",
                 "VS_LAYOUT_BSHD", "VS_LAYOUT_BHSD", "VS_EXPCAST", "VS_QK_HADAMARD",
                 "VS_V_MXFP4", "VS_OUT_BF16", "VS_BF16_MMA", "VS_P_MXFP4"]:
        m = re.search(r"#define\s+" + name + r"\s+(\d+)", text)
        assert m and int(m.group(1)) == getattr(_abi, name), name
    m = re.search(r"#define\s+VS_NOALLOC_STATS_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _abi.VS_NOALLOC_STATS_SCRATCH_BYTES


@pytest.mark.parametrize("S,grid,cube", [(16, (2, 2, 4), (1, 2, 2)), (8, (1, 3, 3), (1, 2, 2)),
                                         (32626, (20, 48, 34), (2, 8, 8)),
                                         (115328, (71, 48, 34), (1, 8, 16)),
                                         (600, (5, 12, 10), (2, 4, 4)), (1, (1, 1, 1), (3, 3, 3))])
def test_cube_permutation_host_call_equals_the_oracle(lib, S, grid, cube):
    """vs_cube_permutation is a host function: checked here, without a GPU,
    against the oracle's sort-based definition."""
    import numpy as np
    from oracle import grouping
    buf = (ctypes.c_int32 * S)()
    assert lib.vs_cube_permutation(S, *grid, *cube, buf) == 0
    got = np.frombuffer(buf, dtype=np.int32).astype(np.int64)
    np.testing.assert_array_equal(got, grouping.cube_permutation(S, grid, cube))


def test_cube_permutation_argument_errors(lib):
    buf = (ctypes.c_int32 * 64)()
    assert lib.vs_cube_permutation(64, 2, 3, 4, 1, 1, 1, buf) == 1      # grid 24 < 64
    assert lib.vs_cube_permutation(8, 2, 2, 2, 0, 1, 1, buf) == 1
    assert lib.vs_cube_permutation(8, 2, 2, 2, 1, 1, 1, None) == 1
    assert lib.vs_cube_permutation(-1, 2, 2, 2, 1, 1, 1, buf) == 1
    assert lib.vs_cube_permutation(0, 2, 2, 2, 1, 1, 1, None) == 0


def test_size_limits_are_rejected_before_any_launch(lib):
    """Sizes past what the kernels address (32-bit per-head buffer ranges,
    65535 grid rows) return VS_ERR_UNSUPPORTED from the host checks."""
    fake = ctypes.c_void_p(0x1000)
    f = lib.vs_fp8_attn_fwd
    # S = 2^24 at D = 128: one head's codes span 2^31 bytes
    assert f(fake, fake, fake, fake, fake, fake, None, 0, None, 1, 1 << 24, 1, 128, 0,
             fake, fake, None) == 2
    assert f(fake, fake, fake, fake, fake, fake, None, 0, None, 1, (1 << 24) - 128, 1, 128, 4,
             None, fake, None) == 1            # just below: argument checks run (out NULL)
    q = lib.vs_quantize_residual
    assert q(fake, fake, fake, 0, 65536, 300, 2, 128, 0.1, None, None, 0,
             fake, fake, fake, fake, fake, fake, None, None) == 2
    assert q(fake, fake, fake, 0, 1, 300, 65536, 128, 0.1, None, None, 0,
             fake, fake, fake, fake, fake, fake, None, None) == 2

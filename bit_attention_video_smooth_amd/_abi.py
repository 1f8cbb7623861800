"""ctypes view of libvsmooth.so (include/vsmooth.h).  Loading only; no math."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libvsmooth.so")

VS_OK, VS_ERR_INVALID_ARG, VS_ERR_UNSUPPORTED, VS_ERR_WORKSPACE, VS_ERR_HIP = range(5)
VS_LAYOUT_BSHD, VS_LAYOUT_BHSD = 0, 1
VS_VMEAN_NONE, VS_VMEAN_BLOCK, VS_VMEAN_SEQ, VS_VMEAN_BLOCK_OUT = 0, 1, 2, 3
VS_EXPCAST = 1
VS_QK_HADAMARD = 1
VS_V_MXFP4 = 2
VS_OUT_BF16 = 4
VS_BF16_MMA = 8
VS_P_MXFP4 = 16
VS_NOALLOC_STATS_SCRATCH_BYTES = 32 << 20

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_U = ctypes.c_uint
_Z = ctypes.c_size_t
_PZ = ctypes.POINTER(ctypes.c_size_t)

#: every entry point of vsmooth.h with its argument types
PROTOTYPES = {
    "vs_status_string": (ctypes.c_char_p, [_I]),
    "vs_version": (ctypes.c_char_p, []),
    "vs_smooth_stats_workspace_bytes": (_I, [_I, _I, _I, _I, _PZ]),
    "vs_smooth_stats": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _Z, _P]),
    "vs_smooth_stats_ex": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "vs_smooth_stats_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "vs_quantize_residual": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _I,
                                  _P, _P, _P, _P, _P, _P, _P, _P]),
    "vs_quantize_residual_perm": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _I,
                                       _P, _P, _P, _P, _P, _P, _P, _P]),
    "vs_quantize_residual_ex": (_I, [_P, _P, _P, _I, _P, _U, _I, _I, _I, _I, _F, _P, _P, _P,
                                     _P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "vs_fp8_attn_fwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _U,
                             _P, _P, _P]),
    "vs_fp8_attn_fwd_pcodes": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _U,
                                    _P, _P, _P, _I, _P]),
    "vs_cube_permutation": (_I, [_I, _I, _I, _I, _I, _I, _I, _P]),
    "vs_kmeans_workspace_bytes": (_I, [_I, _I, _I, _I, _I, _PZ]),
    "vs_kmeans_permute": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
}

_lib = None


def load():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m bit_attention_video_smooth_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class VsError(RuntimeError):
    def __init__(self, status, where):
        msg = load().vs_status_string(status).decode()
        super().__init__(f"{where}: {msg}")
        self.status = status


def check(status, where):
    if status != VS_OK:
        raise VsError(status, where)

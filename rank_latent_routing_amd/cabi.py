"""ctypes declarations of the C ABI in include/flare.h, with no torch import.

``load(path)`` opens a build of the library and declares the argument and
result types of every entry point.  The Python binding uses it on the gfx950
library; the CPU tests use it on that library (to check that it loads and
exports every symbol) and on the host-only build with stand-in launchers
(to drive argument checks, planning and workspace carving without a GPU).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
BUILD_DIR = os.path.join(_HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libflare.so")
HOST_LIB_PATH = os.path.join(BUILD_DIR, "libflare_host.so")
HOST_SAN_LIB_PATH = os.path.join(BUILD_DIR, "libflare_host_san.so")

FLARE_OK = 0
FLARE_E_INVALID = -1
FLARE_E_UNSUPPORTED = -2
FLARE_E_WORKSPACE = -3
FLARE_E_HIP = -4
FLARE_E_SCRATCH = -5
FLARE_F32 = 0
FLARE_BF16 = 1
FLARE_FLAG_EXACT_SOFTMAX = 1
FLARE_MIX_FUSED_WO = 2

FLARE_ACCUMULATE_DQ = 1
FLARE_ACCUMULATE_DK = 2
FLARE_SUM_DQ_OVER_BATCH = 4

EXPORTS = ("flare_encode_workspace_size", "flare_encode", "flare_route_queries",
           "flare_decode", "flare_project_workspace_size", "flare_project",
           "flare_mix_workspace_size", "flare_mix",
           "flare_decode_backward_workspace_size", "flare_decode_backward",
           "flare_encode_backward_workspace_size", "flare_encode_backward",
           "flare_encdec_backward_workspace_size", "flare_encdec_backward",
           "flare_encode_static_scratch_bytes", "flare_encode_static",
           "flare_status_string", "flare_version")
# Entry points the host-only build leaves out (they need device memory).
DEVICE_ONLY = ("flare_encode_static_scratch_bytes", "flare_encode_static")


class FlareTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_l", ctypes.c_int64)]


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open a build of the library and declare its entry points."""
    if not os.path.exists(path):
        raise RuntimeError(
            f"library not built ({path} missing): run __graft_entry__.build() "
            "or python rank_latent_routing_amd/build.py")
    L = ctypes.CDLL(path)
    vp, i32, i64, f32, u32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_uint, ctypes.c_size_t)
    T = ctypes.POINTER(FlareTensor)
    L.flare_encode_workspace_size.argtypes = [i32, i32, i32, i64, i32]
    L.flare_encode_workspace_size.restype = sz
    L.flare_encode.argtypes = [T, T, T, T, vp, i32, i32, i32, i64, i32, f32, u32, vp, sz, vp]
    L.flare_route_queries.argtypes = [T, T, T, T, vp, i32, i32, i32, i64, i32, f32, u32, vp, sz, vp]
    L.flare_decode.argtypes = [T, T, T, T, vp, i32, i32, i32, i64, i32, f32, u32, vp]
    L.flare_decode_backward_workspace_size.argtypes = [i32, i32, i32, i64, i32]
    L.flare_decode_backward_workspace_size.restype = sz
    L.flare_decode_backward.argtypes = [T, T, T, T, vp, T, T, vp, vp, u32, i32, i32, i32, i64, i32,
                                        f32, vp, sz, vp]
    L.flare_encode_backward_workspace_size.argtypes = [i32, i32, i32, i64, i32]
    L.flare_encode_backward_workspace_size.restype = sz
    L.flare_encode_backward.argtypes = [T, T, T, T, vp, vp, vp, T, T, u32, i32, i32, i32, i64, i32,
                                        f32, vp, sz, vp]
    L.flare_encdec_backward_workspace_size.argtypes = [i32, i32, i32, i64, i32]
    L.flare_encdec_backward_workspace_size.restype = sz
    L.flare_encdec_backward.argtypes = [T, T, T, T, vp, T, vp, T, vp, T, T, u32, i32, i32, i32, i64, i32,
                                        f32, vp, sz, vp]
    L.flare_project_workspace_size.argtypes = [i32, i32, i32]
    L.flare_project_workspace_size.restype = sz
    L.flare_project.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i64, i32,
                                i32, i32, i32, i32, vp, sz, vp]
    L.flare_mix_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.flare_mix_workspace_size.restype = sz
    L.flare_mix.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32,
                            f32, u32, vp, sz, vp]
    for f in ("flare_encode", "flare_route_queries", "flare_decode",
              "flare_project", "flare_mix",
              "flare_decode_backward", "flare_encode_backward", "flare_encdec_backward"):
        getattr(L, f).restype = ctypes.c_int
    if hasattr(L, "flare_encode_static"):
        L.flare_encode_static.argtypes = [T, T, T, T, vp, i32, i32, i32, i64, i32, f32, u32, vp]
        L.flare_encode_static.restype = ctypes.c_int
        L.flare_encode_static_scratch_bytes.argtypes = []
        L.flare_encode_static_scratch_bytes.restype = sz
    L.flare_status_string.argtypes = [i32]
    L.flare_status_string.restype = ctypes.c_char_p
    L.flare_version.restype = ctypes.c_char_p
    return L

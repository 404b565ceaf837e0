"""ctypes loader for libdpnorm.so: argument marshalling only.

Every function of the C ABI declared in include/dpnorm.h is given its
argument and return types here. Nothing in this module computes anything of
the method; the Python API in ``__init__`` turns torch tensors into device
pointers and calls these functions.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdpnorm.so")

# DPNORM_STATIC_SCRATCH_BYTES: the static scratch of dpnorm_hutch_grouped_noalloc
STATIC_SCRATCH_BYTES = 64 << 20
# dpnorm_status
OK, ERR_NULL, ERR_SIZE, ERR_DTYPE, ERR_VALUE, ERR_WORKSPACE, ERR_ALIGN, ERR_HIP = range(8)
# dpnorm_dtype
F32, BF16 = 0, 1
# dpnorm_route
EXACT_AUTO, EXACT_EXPLICIT, EXACT_GRAM = 0, 1, 2
# dpnorm_kernel_kind
KERNEL_PREPARE, KERNEL_ROWPROJ, KERNEL_TCONTRACT, KERNEL_YSUM, KERNEL_FINISH = 1, 2, 3, 4, 5
KERNEL_NAMES = {1: "prepare", 2: "rowproj", 3: "tcontract", 4: "ysum", 5: "finish"}


class Layer(C.Structure):
    """struct dpnorm_layer: device pointers A [B][T][d], G [B][T][p], P [p][k]."""
    _fields_ = [("A", C.c_void_p), ("G", C.c_void_p), ("P", C.c_void_p), ("d", C.c_int64), ("p", C.c_int64)]


class Trace(C.Structure):
    """struct dpnorm_trace: host arrays of events and kernel kinds."""
    _fields_ = [("events", C.POINTER(C.c_void_p)), ("kinds", C.POINTER(C.c_int32)),
                ("capacity", C.c_int64), ("count", C.c_int64)]


_vp, _i64, _i32, _f32, _sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
_fp = C.POINTER(C.c_float)

SIGNATURES = {
    "dpnorm_version": ([], C.c_int),
    "dpnorm_status_string": ([C.c_int], C.c_char_p),
    "dpnorm_hutchpp_split": ([_i64, C.POINTER(_i64), C.POINTER(_i64)], C.c_int),
    "dpnorm_read_probe": ([_vp, _i64, _vp], C.c_int),
    "dpnorm_hutch_sign": ([_vp, _vp, _vp, C.c_int, _i64, _i64, _i64, _i64, _i64, _vp, C.c_int, _vp, _sz, _vp],
                          C.c_int),
    "dpnorm_hutch_sign_grouped": ([C.POINTER(Layer), _i64, C.c_int, _i64, _i64, _i64, _vp, C.c_int, _vp, _f32,
                                   _vp, _sz, _vp], C.c_int),
    "dpnorm_norms_routed_workspace": ([C.POINTER(Layer), _i64, C.c_int, _i64, _i64, _i64, C.POINTER(_sz)],
                                      C.c_int),
    "dpnorm_norms_routed": ([C.POINTER(Layer), _i64, C.c_int, _i64, _i64, _i64, _vp, C.c_int, _vp, _f32, _vp,
                             _vp, _sz, _vp], C.c_int),
    "dpnorm_hutch_workspace": ([C.c_int, _i64, _i64, _i64, _i64, _i64, C.POINTER(_sz)], C.c_int),
    "dpnorm_hutch_grouped_workspace": ([C.POINTER(Layer), _i64, C.c_int, _i64, _i64, _i64, C.POINTER(_sz)], C.c_int),
    "dpnorm_hutch": ([_vp, _vp, _vp, C.c_int, _i64, _i64, _i64, _i64, _i64, _vp, C.c_int, _vp, _sz, _vp], C.c_int),
    "dpnorm_hutch_grouped": ([C.POINTER(Layer), _i64, C.c_int, _i64, _i64, _i64, _vp, C.c_int, _vp, _f32, _vp, _sz,
                              _vp], C.c_int),
    "dpnorm_hutch_grouped_noalloc": ([C.POINTER(Layer), _i64, C.c_int, _i64, _i64, _i64, _vp, C.c_int, _vp, _f32,
                                      _vp], C.c_int),
    "dpnorm_hutch_grouped_traced": ([C.POINTER(Layer), _i64, C.c_int, _i64, _i64, _i64, _vp, C.c_int, _vp, _f32, _vp,
                                     _sz, _vp, C.POINTER(Trace)], C.c_int),
    "dpnorm_hutchpp_workspace": ([C.c_int, _i64, _i64, _i64, _i64, _i64, C.POINTER(_sz)], C.c_int),
    "dpnorm_hutchpp": ([_vp, _vp, _vp, _vp, C.c_int, _i64, _i64, _i64, _i64, _i64, _vp, C.c_int, _vp, _vp, _vp, _vp,
                        _vp, _sz, _vp], C.c_int),
    "dpnorm_exact_workspace": ([C.c_int, _i64, _i64, _i64, _i64, C.c_int, C.POINTER(_sz)], C.c_int),
    "dpnorm_exact": ([_vp, _vp, C.c_int, _i64, _i64, _i64, _i64, C.c_int, _vp, C.c_int, _vp, _sz, _vp], C.c_int),
    "dpnorm_clip_factors": ([_vp, _i64, _f32, _vp, _vp], C.c_int),
    "dpnorm_event_create": ([C.POINTER(_vp)], C.c_int),
    "dpnorm_event_destroy": ([_vp], C.c_int),
    "dpnorm_event_elapsed_ms": ([_vp, _vp, _fp], C.c_int),
    "dpnorm_event_record": ([_vp, _vp], C.c_int),
    "dpnorm_event_synchronize": ([_vp], C.c_int),
}

_LIB = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the built library and set every signature (raises if it is missing)."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"libdpnorm is not built ({path} missing): run __graft_entry__.build() "
            "or python sample_grad_norms_amd/build.py")
    lib = C.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path == LIB_PATH:
        _LIB = lib
    return lib

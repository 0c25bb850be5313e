"""ctypes loader for libfp8mot.so (argument marshalling only).

The library is built in-tree by ``mlp_fp8_quant_amd.build``.  There is no
fallback: if the shared library is missing, every call raises.
"""

import ctypes
import os

from .build import LIB_PATH

c_void_p = ctypes.c_void_p
c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_float = ctypes.c_float
c_size_t = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/fp8mot.h
SIGNATURES = {
    "fp8mot_init": (c_int, [c_int]),
    "fp8mot_status_string": (ctypes.c_char_p, [c_int]),
    "fp8mot_debug_quant_launches": (ctypes.c_uint64, []),
    "fp8mot_rw_ceiling": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_void_p]),
    "fp8mot_mfma_ceiling": (c_int, [c_void_p, c_i64, c_void_p, c_i64, c_i64, c_int, c_void_p,
                                   ctypes.POINTER(ctypes.c_double), c_void_p]),
    "fp8mot_convert_f32": (c_int, [c_void_p, c_void_p, c_i64, c_int, c_void_p]),
    "fp8_quant_static": (c_int, [c_void_p, c_void_p, c_i64, c_void_p, c_void_p]),
    "fp8_linear": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64,
                           c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p]),
    "fp8_quant_per_row": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_void_p]),
    "fp8_linear_rowwise": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64,
                                   c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "fp8_linear_ldc": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64, c_i64,
                               c_void_p, c_void_p, c_int, c_void_p, c_int, c_void_p]),
    "fp8_requantize_onto_max": (c_int, [c_void_p, c_void_p, c_i64, c_void_p, c_void_p,
                                        c_int, c_void_p]),
    "silu_mul_2in_fp8": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_void_p,
                                 c_void_p]),
    "silu_mul_2in_fp8_ab": (c_int, [c_void_p, c_void_p, c_void_p, c_i64, c_void_p,
                                    c_float, c_float, c_void_p]),
    "silu_mul_fp8": (c_int, [c_void_p, c_void_p, c_i64, c_i64, c_void_p,
                             c_float, c_float, c_void_p]),
    "gated_mlp_fp8_workspace": (c_size_t, [c_i64, c_i64, c_i64]),
    "gated_mlp_fp8": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                              c_int, c_void_p]),
    "gated_mlp_fp8_noalloc": (c_int, [c_void_p, c_i64, c_i64, c_i64, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_int, c_void_p]),
    "fp8_gate_up_swiglu": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_i64, c_i64, c_i64,
                                   c_int, c_void_p]),
    "qkv_fp8_workspace": (c_size_t, [c_i64, c_i64]),
    "qkv_fp8": (c_int, [c_void_p, c_i64, c_i64, c_void_p,
                        c_void_p, c_i64, c_void_p, c_void_p, c_i64, c_void_p,
                        c_void_p, c_i64, c_void_p, c_void_p, c_void_p, c_void_p,
                        c_void_p, c_size_t, c_int, c_void_p]),
    "fp8_observe": (c_int, [c_void_p, c_i64, c_void_p, c_int, c_float, c_void_p]),
    "fp8_observe_swiglu": (c_int, [c_void_p, c_void_p, c_i64, c_void_p, c_int,
                                   c_float, c_void_p]),
    "fp8_scale_from_state": (c_int, [c_void_p, c_void_p, c_void_p]),
    "fp8_check_shared_scale": (c_int, [ctypes.POINTER(c_float), c_int]),
}

STATUS = {
    0: "FP8MOT_OK", 1: "FP8MOT_ERR_INVALID_ARG", 2: "FP8MOT_ERR_MISALIGNED",
    3: "FP8MOT_ERR_SCALE_MISMATCH", 4: "FP8MOT_ERR_UNSUPPORTED",
    5: "FP8MOT_ERR_HIP", 6: "FP8MOT_ERR_WORKSPACE", 7: "FP8MOT_ERR_TOO_LARGE",
}

_lib = None
_funcs = {}


class Fp8motError(RuntimeError):
    """A libfp8mot call returned a non-OK status."""

    def __init__(self, func, status, message):
        super().__init__(f"{func}: {STATUS.get(status, status)}: {message}")
        self.func = func
        self.status = status


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mlp_fp8_quant_amd.build` (no CPU fallback exists)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def call(name, *args):
    """Call an int-returning entry point; raise Fp8motError on failure."""
    f = _funcs.get(name)
    if f is None:
        f = _funcs[name] = getattr(lib(), name)
    st = f(*args)
    if st != 0:
        raise Fp8motError(name, st, lib().fp8mot_status_string(st).decode())
    return st

"""ctypes loader of libdust.so (the C ABI in include/dust.h).

Only argument marshalling lives here: every step of the estimator runs in the
library's HIP kernels.  Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdust.so")

DUST_OK = 0
DUST_ERR_INVALID_ARG = 1
DUST_ERR_WORKSPACE = 2
DUST_ERR_HIP = 3
DUST_ERR_UNSUPPORTED = 4
DUST_ERR_TARGETS = 5

DUST_F32 = 0
DUST_BF16 = 1

DUST_SIGMA_MAX = 8.0
DUST_N_MAX = 65536
DUST_STAGE_EVENTS = 4
DUST_EMBEDDING_NOALLOC_BYTES = 16 << 20

_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_vp = ctypes.c_void_p
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/dust.h
SIGNATURES = {
    "dust_status_string": (ctypes.c_char_p, [_int]),
    "dust_version": (ctypes.c_char_p, []),
    "dust_head_estimate": (_int, [_vp, _int, _vp, _vp, _int, _i64, _i64, _i64, _i64, _f32, _i64,
                                  _f32, _u64, _u32, _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "dust_head_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _f32]),
    "dust_linear_estimate": (_int, [_vp, _int, _vp, _i64, _i64, _i64, _i64, _f32, _i64, _f32,
                                    _u64, _u32, _i64, _i64, _vp, _vp, _vp, _sz, _vp, _vp]),
    "dust_linear_workspace_size": (_sz, [_i64, _i64, _i64, _i64, _f32]),
    "dust_noise": (_int, [_u64, _u32, _i64, _i64, _i64, _i64, _vp, _vp]),
    "dust_philox4x32_10": (_int, [_u64, _vp, _vp, _i64, _vp]),
    "dust_head_losses": (_int, [_vp, _int, _vp, _i64, _i64, _f32, _i64, _u64, _u32, _vp, _vp]),
    "dust_centre": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "dust_reward_scan": (_int, [_vp, _i64, _i64, _i64, _f32, _vp, _vp]),
    "dust_error_estimate": (_int, [_vp, _i64, _i64, _i64, _f32, _u64, _u32, _i64, _i64, _vp,
                                   _vp]),
    "dust_outer_sum": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "dust_outer_sum_workspace_size": (_sz, [_i64, _i64, _i64]),
    "dust_perturbed_linear": (_int, [_vp, _vp, _int, _i64, _i64, _i64, _f32, _u64, _u32, _i64,
                                     _i64, _vp, _vp]),
    "dust_embedding_grad": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _sz, _vp]),
    "dust_embedding_workspace_size": (_sz, [_i64, _i64, _i64]),
    "dust_embedding_grad_noalloc": (_int, [_vp, _vp, _i64, _i64, _i64, _vp, _vp]),
    "dust_embedding_noalloc_bytes": (_sz, [_i64, _i64, _i64]),
    "dust_sgd_momentum": (_int, [_vp, _vp, _vp, _i64, _f32, _f32, _f32, _vp]),
    "dust_adam": (_int, [_vp, _vp, _vp, _vp, _i64, _f32, _f32, _f32, _f32, _f32, _i64, _vp]),
    "dust_ce_grad": (_int, [_vp, _int, _vp, _i64, _i64, _vp, _vp]),
    "dust_check_targets": (_int, [_vp, _i64, _i64, _vp, _vp]),
}

_lib = None


class DustError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {status_string(status)} ({status})")


def load() -> ctypes.CDLL:
    """Load libdust.so (built in place by build.py); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libdust.so not found at {LIB_PATH}: build it with "
            "`python -m activation_perturbation_estimator_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().dust_status_string(int(status)).decode()


def check(func: str, status: int) -> None:
    if status != DUST_OK:
        raise DustError(func, status)

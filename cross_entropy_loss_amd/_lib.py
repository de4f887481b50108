"""ctypes view of the C ABI in include/ce_mi355x.h (argument marshalling only).

Loading never falls back to anything: a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libce_mi355x.so")

CE_DTYPE_F32, CE_DTYPE_BF16, CE_DTYPE_F16 = 0, 1, 2
CE_OK, CE_ERR_INVALID_ARG, CE_ERR_DTYPE, CE_ERR_WORKSPACE, CE_ERR_UNSUPPORTED, CE_ERR_HIP, CE_ERR_SCRATCH = range(7)
CE_STATUS_LABEL_RANGE = 0x1
CE_STATUS_SYNC_TIMEOUT = 0x2
ABI_VERSION = 5

# every symbol the header declares, with its C signature
_i64, _int, _sz, _vp = ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "ce_abi_version": ([], _int),
    "ce_debug_sync_override": ([_int, _int], _int),
    "ce_error_string": ([_int], ctypes.c_char_p),
    "ce_workspace_bytes": ([_i64, _i64, _i64, _int], _sz),
    "ce_workspace_init": ([_vp, _sz, _vp], _int),
    "ce_forward": ([_vp, _i64, _vp, _i64, _i64, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                   _int),
    "ce_backward": ([_vp, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _int, _i64, _vp, _i64, _vp], _int),
    "ce_fwd_bwd_inplace": ([_vp, _i64, _vp, _i64, _i64, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                            _sz, _vp], _int),
    "ce_fwd_bwd_inplace_noalloc": ([_vp, _i64, _vp, _i64, _i64, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp], _int),
    "ce_linear_workspace_bytes": ([_i64, _i64, _i64, _i64, _int], _sz),
    "ce_rmsnorm_workspace_bytes": ([_i64, _i64, _int], _sz),
    "ce_rmsnorm_forward": ([_vp, _i64, _vp, _i64, _i64, _int, ctypes.c_float, _vp, _i64, _vp, _vp], _int),
    "ce_rmsnorm_backward": ([_vp, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _int, _vp, _i64, _vp, _vp, _sz, _vp], _int),
    "ce_linear_fwd_bwd": ([_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp,
                           _vp, _i64, _vp, _i64, _vp, _sz, _vp], _int),
    "ce_rope": ([_vp, _vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _i64, ctypes.c_double, _int,
                 _int, _vp], _int),
}

_lib = None


class CeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {error_string(code)} (code {code})")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises ImportError when it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m cross_entropy_loss_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if lib.ce_abi_version() != ABI_VERSION:
        raise ImportError(f"{path}: ABI version {lib.ce_abi_version()} != {ABI_VERSION}")
    if path == LIB_PATH:
        _lib = lib
    return lib


def error_string(code: int) -> str:
    return load().ce_error_string(code).decode()


def check(code: int, what: str) -> None:
    if code != CE_OK:
        raise CeError(code, what)

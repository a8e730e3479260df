"""ctypes declarations of the C ABI in ``include/fa.h`` (no logic here)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_DTYPE = -3
FA_ERR_HEADDIM = -4
FA_ERR_GQA = -5
FA_ERR_STRIDE = -6
FA_ERR_ALIGN = -7
FA_ERR_WORKSPACE = -8
FA_ERR_HIP = -9
FA_ERR_MASK = -10
FA_ERR_SCALE = -11
FA_ERR_DROPOUT = -12
STATUS_CODES = [FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_DTYPE, FA_ERR_HEADDIM, FA_ERR_GQA,
                FA_ERR_STRIDE, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_HIP, FA_ERR_MASK,
                FA_ERR_SCALE, FA_ERR_DROPOUT]

FA_BF16 = 0
FA_FP32 = 1
FA_FP8_E4M3 = 2
FA_MASK_BLOCK = 128
FA_NOALLOC_WORKSPACE_BYTES = 32 << 20


class Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("row", ctypes.c_int64)]


class Params(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("o_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("seqlens_k", ctypes.c_void_p),
        ("block_mask", ctypes.c_void_p),
        ("block_mask_ld", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("dropout_p", ctypes.c_float),
        ("dropout_offset", ctypes.c_uint32),
        ("dropout_seed", ctypes.c_uint64),
        ("descale_q", ctypes.c_float),
        ("descale_k", ctypes.c_float),
        ("descale_v", ctypes.c_float),
    ]


_P = ctypes.c_void_p
_S = Strides
#: name -> (restype, argtypes), in the order the header declares them.
SIGNATURES = {
    "fa_fwd": (ctypes.c_int, [ctypes.POINTER(Params), _P, _S, _P, _S, _P, _S, _P, _S, _P, _P, _P]),
    "fa_tile_log_words": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "fa_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "fa_bwd": (ctypes.c_int, [ctypes.POINTER(Params), _P, _S, _P, _S, _P, _S, _P, _S, _P, _S, _P,
                              _P, _S, _P, _S, _P, _S, _P, ctypes.c_size_t, _P, _P, _P]),
    "fa_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(Params), _P, _S, _P, _S, _P, _S, _P, _S, _P,
                                      _S, _P, _P, _S, _P, _S, _P, _S, _P, _P, _P]),
    "fa_decode_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Params)]),
    "fa_decode": (ctypes.c_int, [ctypes.POINTER(Params), _P, _S, _P, _S, _P, _S, _P, _S, _P, _P,
                                 ctypes.c_size_t, _P]),
    "fa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "fa_last_error_detail": (ctypes.c_char_p, []),
}

PARANOID_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                 "libfa_paranoid.so")
# The debug build with per-workgroup timeline stamps (include/fa_timeline.h).
TIMELINE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                 "libfa_timeline.so")

_lib = None


def load_variant(path: str) -> ctypes.CDLL:
    """A separately loaded build of the same ABI (the debug build with extra
    barriers); the caller keeps the handle."""
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is missing: build it first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once; raise RuntimeError (never fall back) if absent.
    The environment variable FA_LIBRARY names another build of the same
    library to load instead (the tests use it for the host-sanitizer build)."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("FA_LIBRARY", path)
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is missing: build it with `python -m exact_io_aware_29_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib

"""ctypes view of libattn.so (the C ABI declared in include/attn.h).

Loading fails loudly when the library has not been built: there is no
fallback path of any kind.
"""

from __future__ import annotations

import ctypes
import os

# ATTN_LIBRARY, when set, names another build of the same library to load
# instead (for example a host-sanitizer build of the C ABI)
LIB_PATH = os.environ.get("ATTN_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_F32, ATTN_BF16, ATTN_FP8_E4M3 = 0, 1, 2
ATTN_BIAS_NONE, ATTN_BIAS_ELEMENTWISE, ATTN_BIAS_ALIBI = 0, 1, 2
ATTN_V_ROW_MAJOR, ATTN_V_COL_MAJOR = 0, 1
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_EINVAL", 2: "ATTN_ENOTSUP", 3: "ATTN_EWORKSPACE", 4: "ATTN_ELAUNCH"}


class AttnParams(ctypes.Structure):
    _fields_ = [
        ("in_dtype", ctypes.c_int),
        ("out_dtype", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("window_left", ctypes.c_int),
        ("window_right", ctypes.c_int),
        ("q_descale", ctypes.c_float),
        ("k_descale", ctypes.c_float),
        ("v_descale", ctypes.c_float),
        ("kv_split_tokens", ctypes.c_int),
        ("sink_size", ctypes.c_int),
        ("sink_logits", ctypes.c_void_p),
        ("bias_type", ctypes.c_int),
        ("bias", ctypes.c_void_p),
        ("bias_stride", ctypes.c_int64 * 3),
        ("o_scale", ctypes.c_float),
        ("cache_batch_idx", ctypes.c_void_p),
        ("cache_batch_count", ctypes.c_int),
        ("min_seqlen_q", ctypes.c_int),
        ("head_dim_v", ctypes.c_int),
        ("v_layout", ctypes.c_int),
        ("v_pool_stride", ctypes.c_int64 * 3),
    ]


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64P = ctypes.POINTER(ctypes.c_int64)
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "attn_params_init": (None, [ctypes.POINTER(AttnParams), ctypes.c_float]),
    "attn_fwd": (_I, [ctypes.POINTER(AttnParams), _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                      _I64P, _I64P, _I64P, _I64P, _P, _P, _P, _SZ, _P]),
    "attn_fwd_varlen": (_I, [ctypes.POINTER(AttnParams), _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                             _I, _I, _I, _I64P, _I64P, _I64P, _I64P, _P, _SZ, _P]),
    "attn_fwd_paged": (_I, [ctypes.POINTER(AttnParams), _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I,
                            _I, _I, _I, _I, _I64P, _I64P, _I64P, _P, _SZ, _P]),
    "attn_fwd_varlen_paged": (_I, [ctypes.POINTER(AttnParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I,
                                   _I, _I, _I, _I, _I, _I, _I64P, _I64P, _I64P, _P]),
    "attn_fwd_paged_noalloc": (_I, [ctypes.POINTER(AttnParams), _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I,
                                    _I, _I, _I, _I, _I64P, _I64P, _I64P, _P]),
    "attn_workspace_bytes": (_SZ, [ctypes.POINTER(AttnParams), _I, _I, _I, _I, _I, _I]),
    "attn_num_splits": (_I, [ctypes.POINTER(AttnParams), _I, _I, _I, _I, _I]),
    "attn_last_error": (ctypes.c_char_p, []),
    "attn_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str) -> ctypes.CDLL:
    """Load a build of libattn at path with the C ABI's signatures."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_attn_amd.build`")
    handle = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def check(status: int):
    if status != 0:
        raise AttnError(status, lib().attn_last_error().decode(errors="replace"))


_I64_CACHE: dict = {}


def i64_array(vals):
    """A ctypes int64 array holding vals. The library only reads these arrays
    (const int64_t*), so equal stride tuples share one cached array."""
    key = tuple(vals)
    arr = _I64_CACHE.get(key)
    if arr is None:
        arr = (ctypes.c_int64 * len(key))(*map(int, key))
        if len(_I64_CACHE) >= 1024:
            _I64_CACHE.clear()
        _I64_CACHE[key] = arr
    return arr

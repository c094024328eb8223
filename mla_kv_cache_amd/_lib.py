"""ctypes loader for libattn_decode.so (the C ABI in include/attn_decode.h).

There is no fallback: if the shared library is missing or cannot be loaded,
``load()`` raises. Build it with ``python -m mla_kv_cache_amd.build``.
"""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn_decode.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = -1
ATTN_ERR_UNSUPPORTED = -2
ATTN_ERR_WORKSPACE = -3
ATTN_ERR_HIP = -4
ATTN_F32 = 0
ATTN_BF16 = 1

_c_int, _c_float, _c_size, _c_u64 = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64
_vp = ctypes.c_void_p
_ip = ctypes.POINTER(ctypes.c_int)
_sp = ctypes.POINTER(ctypes.c_size_t)

# name -> (restype, argtypes); every symbol include/attn_decode.h declares.
SIGNATURES = {
    "attn_status_str": (ctypes.c_char_p, [_c_int]),
    "attn_kv_cache_bytes": (_c_u64, [_c_u64] * 6),
    "attn_mla_cache_bytes": (_c_u64, [_c_u64] * 6),
    "attn_decode_gqa_plan": (_c_int, [_c_int] * 6 + [_ip, _ip, _sp]),
    "attn_decode_gqa_workspace_bytes": (_c_size, [_c_int] * 6),
    "attn_decode_gqa": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_float, _c_int, _vp, _vp, _c_size, _vp]),
    "attn_decode_gqa_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_float, _c_int, _vp, _vp]),
    "attn_decode_gqa_split": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_float, _c_int, _vp, _vp, _c_size, _vp]),
    "attn_decode_gqa_split_merge": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_float, _c_int, _vp, _vp, _c_size, _vp]),
    "attn_decode_gqa_partial": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_float, _c_int, _c_int, _vp, _vp, _vp]),
    "attn_decode_merge": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                   _vp, _vp]),
    "attn_decode_mla_plan": (_c_int, [_c_int] * 5 + [_ip, _ip, _sp]),
    "attn_decode_mla_workspace_bytes": (_c_size, [_c_int] * 5),
    "attn_decode_mla": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_float, _vp, _vp, _c_size, _vp]),
    "attn_decode_mla_partial": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_float, _c_int, _vp, _vp, _vp]),
    "attn_decode_gqa_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int,
                                      _c_int, _c_float, _c_int, _vp, _vp, _c_size, _vp]),
    "attn_kv_append": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "attn_decode_mla_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                      _c_float, _vp, _vp, _c_size, _vp]),
    "attn_latent_append": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp]),
    "attn_decode_gqa_window": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                        _c_int, _c_float, _c_int, _vp, _vp, _c_size, _vp]),
    "attn_decode_gqa_paged": (_c_int, [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 7 +
                              [_c_float, _c_int, _vp, _vp, _c_size, _vp]),
    "attn_kv_append_paged": (_c_int, [_vp] * 6 + [_c_int] * 7 + [_vp]),
    "attn_decode_mla_paged": (_c_int, [_vp] * 5 + [_c_int] * 7 + [_c_float, _vp, _vp, _c_size, _vp]),
    "attn_latent_append_paged": (_c_int, [_vp] * 4 + [_c_int] * 6 + [_vp]),
    "attn_mla_absorb_q": (_c_int, [_vp, _vp, _vp] + [_c_int] * 4 + [_vp]),
    "attn_mla_up_v": (_c_int, [_vp, _vp, _vp] + [_c_int] * 4 + [_vp]),
}

_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library once and attach the C signatures. Raises if it is absent."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"HIP library not built: {LIB_PATH} is missing "
                    "(run `python -m mla_kv_cache_amd.build`); there is no CPU fallback")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def status_str(st: int) -> str:
    return load().attn_status_str(int(st)).decode()

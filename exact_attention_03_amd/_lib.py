"""ctypes loader for libfa.so: symbol table and status handling.

The library is built in-tree by ``exact_attention_03_amd._build`` (or
``__graft_entry__.build()``).  Loading fails loudly if it is missing: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_DTYPE_F16, FA_DTYPE_BF16, FA_DTYPE_F32 = 0, 1, 2

_i64, _int, _f32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_i64p = ctypes.POINTER(ctypes.c_int64)
_intp = ctypes.POINTER(ctypes.c_int)


class KvSource(ctypes.Structure):
    """fa_kv_source of include/fa.h (field for field)."""
    _fields_ = [("k_cache", _vp), ("v_cache", _vp), ("block_tables", _vp), ("context_lens", _vp),
                ("block_size", _i64), ("num_blocks", _i64), ("max_blocks_per_seq", _i64),
                ("max_context_len", _i64), ("selected", _vp), ("n_selected", _vp), ("topk", _i64),
                ("row_lens", _vp)]


_srcp = ctypes.POINTER(KvSource)

# name -> (restype, argtypes); mirrors include/fa.h
SIGNATURES = {
    "fa_version": (_int, []),
    "fa_status_string": (ctypes.c_char_p, [_int]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_fwd": (_int, [_i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _f32, _int, _vp]),
    "fa_bwd_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "fa_bwd": (_int, [_i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                      _f32, _int, _vp, _sz, _vp]),
    "fa_bwd_noalloc": (_int, [_i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _f32, _int, _vp]),
    "fa_bwd_preprocess": (_int, [_i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp]),
    "fa_bwd_dkdv": (_int, [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _f32, _int, _int, _vp]),
    "fa_bwd_fused_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64]),
    "fa_bwd_fused": (_int, [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _int, _int,
                            _vp, _sz, _vp]),
    "fa_bwd_dq": (_int, [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _int, _vp]),
    "fa_bwd_dq_and_stats": (_int, [_i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _f32, _int, _vp]),
    "fa_fwd_gqa": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _f32, _int, _vp]),
    "fa_bwd_gqa": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _f32, _int, _vp, _sz, _vp]),
    "fa_bwd_dq_and_stats_gqa": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _f32, _int, _vp]),
    "fa_bwd_dkdv_gqa": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _int,
                               _int, _vp]),
    "fa_fwd_varlen": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _f32,
                             _int, _vp]),
    "fa_bwd_varlen": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _f32, _int, _vp, _sz, _vp]),
    "fa_bwd_dq_and_stats_varlen": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp, _f32, _int, _vp]),
    "fa_bwd_dkdv_varlen": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _f32, _int, _int, _vp]),
    "fa_reshape_and_cache": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp]),
    "fa_paged_decode_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64]),
    "fa_paged_decode": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _f32, _vp, _sz, _vp]),
    "fa_quest_page_minmax": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp]),
    "fa_quest_select": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp]),
    "fa_paged_decode_sparse": (_int, [_i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _f32, _vp, _sz, _vp]),
    "fa_paged_decode_sources_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _int, _srcp]),
    "fa_paged_decode_sources": (_int, [_i64, _i64, _i64, _i64, _int, _int, _vp, _int, _srcp, _vp, _vp, _f32, _vp,
                                       _sz, _vp]),
    "fa_paged_attention_sources_workspace_bytes": (_sz, [_i64, _i64, _i64, _i64, _i64, _int, _srcp]),
    "fa_paged_attention_sources": (_int, [_i64, _i64, _i64, _i64, _i64, _int, _int, _vp, _int, _srcp, _vp, _vp,
                                          _f32, _vp, _sz, _vp]),
    "fa_device_info": (_int, [_i64, _int, _intp, _intp]),
    "fa_dkdv_schedule": (_int, [_i64, _i64, _i64, _i64, _int, _int, _i64p, _i64p, _i64p]),
    "fa_fwd_tile_pairs": (_int, [_i64, _i64, _int, _i64p, _i64p]),
}

_lock = threading.Lock()
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        self.func = func
        self.detail = detail
        super().__init__(f"{func} failed with {status_name(status)}: {detail}")


def lib() -> ctypes.CDLL:
    """The loaded library (loaded once).  Raises if libfa.so has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m exact_attention_03_amd._build` "
                    "or __graft_entry__.build(); there is no fallback implementation")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def status_name(status: int) -> str:
    return lib().fa_status_string(status).decode()


def last_error() -> str:
    return lib().fa_last_error().decode()


def check(status: int, func: str) -> None:
    if status != FA_OK:
        raise FAError(status, func, last_error())

"""ctypes declarations of libmilo's C ABI (include/milo.h).

Argument marshalling only: every computation happens in the HIP library.  The
library must be built in-tree (block_wise_rank_amd/libmilo.so); loading fails
loudly when it is missing -- there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmilo.so")

MILO_OK, MILO_E_INVALID, MILO_E_UNSUPPORTED, MILO_E_WORKSPACE, MILO_E_HIP = range(5)
MILO_F32, MILO_BF16, MILO_I8, MILO_I4, MILO_I2 = 0, 1, 2, 3, 4
MILO_ALLOC_ENTROPY, MILO_ALLOC_UNIFORM, MILO_ALLOC_RANDOM = 0, 1, 2
MILO_NOALLOC_SCRATCH_BYTES = 32 << 20

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class milo_blocks(ctypes.Structure):
    _fields_ = [("x", _vp), ("dtype", ctypes.c_int), ("row0", _vp), ("row_stride", _i64),
                ("n_blocks", _i32), ("block_len", _i32), ("head_dim", _i32)]


class milo_factors(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("n_blocks", _i32), ("block_len", _i32),
                ("head_dim", _i32), ("rank", _vp), ("a_off", _vp), ("b_off", _vp),
                ("arena", _vp), ("arena_bytes", ctypes.c_size_t), ("a_scale", _vp),
                ("b_scale", _vp)]


class milo_alloc_options(ctypes.Structure):
    _fields_ = [("policy", ctypes.c_int), ("seed", ctypes.c_uint64)]


class milo_decode_args(ctypes.Structure):
    _fields_ = [("q", _vp), ("q_dtype", ctypes.c_int), ("q_pos", _vp), ("batch", _i32),
                ("n_q_heads", _i32), ("n_kv_heads", _i32), ("head_dim", _i32),
                ("k", ctypes.POINTER(milo_factors)), ("v", ctypes.POINTER(milo_factors)),
                ("blocks_per_seq", _i32), ("sel_ptr", _vp), ("sel_blk", _vp), ("sel_max", _i32),
                ("tail_k", _vp), ("tail_v", _vp), ("tail_dtype", ctypes.c_int),
                ("tail_cap", _i32), ("tail_len", _vp), ("tail_pos0", _vp),
                ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("out", _vp), ("out_dtype", ctypes.c_int), ("split_len", _i32),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("tail_seg_pos", _vp), ("tail_seg_valid", _vp), ("tail_seg_len", _i32)]


# Every symbol include/milo.h declares, with its ctypes signature.
SIGNATURES = {
    "milo_compress_blocks": (ctypes.c_int, [ctypes.POINTER(milo_blocks), _vp, _i32, _vp,
                                            ctypes.c_double, _vp, _vp, ctypes.POINTER(milo_factors),
                                            _vp, _vp, ctypes.POINTER(ctypes.c_size_t), _vp]),
    "milo_compress_blocks_ex": (ctypes.c_int, [ctypes.POINTER(milo_blocks), _vp, _i32, _vp,
                                               ctypes.c_double, _vp, _vp, ctypes.POINTER(milo_factors),
                                               _vp, ctypes.POINTER(milo_alloc_options), _vp,
                                               ctypes.POINTER(ctypes.c_size_t), _vp]),
    "milo_allocate_ranks": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _i32, _vp, ctypes.c_double,
                                           _vp, _vp, _vp, ctypes.POINTER(ctypes.c_size_t), _vp]),
    "milo_allocate_ranks_ex": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _i32, _vp, ctypes.c_double,
                                              _vp, _vp, ctypes.POINTER(milo_alloc_options), _vp,
                                              ctypes.POINTER(ctypes.c_size_t), _vp]),
    "milo_reconstruct": (ctypes.c_int, [ctypes.POINTER(milo_factors), _vp, _i32, _vp,
                                        ctypes.c_int, _vp]),
    "milo_reconstruct_ex": (ctypes.c_int, [ctypes.POINTER(milo_factors), _vp, _i32, _vp, _vp,
                                           ctypes.c_int, _vp]),
    "milo_fetch_blocks": (ctypes.c_int, [ctypes.POINTER(milo_factors), ctypes.POINTER(milo_factors), _vp,
                                         _i32, _vp]),
    "milo_decode_attention": (ctypes.c_int, [ctypes.POINTER(milo_decode_args),
                                             ctypes.POINTER(ctypes.c_size_t), _vp]),
    "milo_decode_attention_noalloc": (ctypes.c_int, [ctypes.POINTER(milo_decode_args), _vp]),
    "milo_arena_bytes": (ctypes.c_size_t, [ctypes.c_int, _i32, _i32, _vp, _i32, _vp]),
    "milo_compress_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32]),
    "milo_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "milo_profile_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_i32),
                                         ctypes.POINTER(ctypes.c_double), ctypes.c_int]),
    "milo_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "milo_last_error": (ctypes.c_char_p, []),
    "milo_abi_version": (ctypes.c_int, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load libmilo and declare every exported function; raises if it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"libmilo is not built ({path} missing); run `python -c 'import __graft_entry__ as g; "
            f"g.build()'` -- the HIP library is required, there is no fallback")
    L = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = L
    return L

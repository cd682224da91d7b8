"""ctypes view of libcpattn.so: the argument structs and function signatures of include/cpattn.h.

The library is loaded from this package directory only. If it is missing the import fails with an error that says how
to build it: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpattn.so")

CPATTN_OK, CPATTN_EINVAL, CPATTN_EUNSUPPORTED, CPATTN_ELAUNCH = 0, 1, 2, 3
CPATTN_F32, CPATTN_BF16, CPATTN_FP8_E4M3 = 0, 1, 2
CPATTN_KV_SAME, CPATTN_KV_FP8_E4M3 = 0, 1
CPATTN_GQA, CPATTN_MLA = 0, 1
MAX_PARTIALS = 17
CPATTN_FLAG_FIXED_SPLITS = 1
CPATTN_FLAG_PAD_LSE_ONLY = 2

_p = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64


class PagedArgs(C.Structure):
    _fields_ = [
        ("kind", _i32), ("dtype", _i32), ("num_rows", _i32), ("num_tokens", _i32), ("num_partners", _i32),
        ("stripe_begin", _i32), ("stripe_count", _i32), ("page_size", _i32), ("num_pages", _i32),
        ("num_q_heads", _i32), ("num_kv_heads", _i32), ("head_dim", _i32), ("head_dim_v", _i32),
        ("scale", C.c_float), ("max_ctx_len", _i32), ("max_row_tokens", _i32), ("max_pages", _i32),
        ("flags", _i32), ("interleave", _i32), ("kv_format", _i32), ("k_descale", C.c_float),
        ("v_descale", C.c_float),
        ("q_row_start", _p), ("ctx_len", _p), ("block_table", _p), ("bt_stride", _i64),
        ("q", _p), ("q_stride_token", _i64), ("q_stride_head", _i64),
        ("k_pool", _p), ("v_pool", _p),
        ("kv_stride_stripe", _i64), ("kv_stride_page", _i64), ("kv_stride_slot", _i64), ("kv_stride_head", _i64),
        ("out", _p), ("out_stride_stripe", _i64), ("out_stride_token", _i64), ("out_stride_head", _i64),
        ("lse", _p), ("lse_stride_stripe", _i64), ("lse_stride_token", _i64),
        ("workspace", _p), ("workspace_bytes", _i64),
    ]


class OwnArgs(C.Structure):
    _fields_ = [
        ("dtype", _i32), ("num_rows", _i32), ("bucket_tokens", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
        ("head_dim", _i32), ("scale", C.c_float), ("max_row_tokens", _i32), ("flags", _i32), ("reserved0", _i32),
        ("cu_seqlens", _p), ("q", _p), ("q_stride_token", _i64), ("q_stride_head", _i64),
        ("k", _p), ("v", _p), ("kv_stride_token", _i64), ("kv_stride_head", _i64),
        ("out", _p), ("out_stride_token", _i64), ("out_stride_head", _i64),
        ("lse", _p), ("lse_stride_token", _i64),
    ]


class MergeArgs(C.Structure):
    _fields_ = [
        ("num_partials", _i32), ("num_tokens", _i32), ("num_heads", _i32), ("head_dim_v", _i32),
        ("out_dtype", _i32), ("reserved0", _i32), ("token_count", _p),
        ("part_out", _p * MAX_PARTIALS), ("part_lse", _p * MAX_PARTIALS),
        ("part_out_stride_token", _i64 * MAX_PARTIALS), ("part_out_stride_head", _i64 * MAX_PARTIALS),
        ("part_lse_stride_token", _i64 * MAX_PARTIALS), ("part_lse_stride_head", _i64 * MAX_PARTIALS),
        ("out", _p), ("out_stride_token", _i64), ("out_stride_head", _i64),
        ("lse_out", _p), ("lse_out_stride_token", _i64),
    ]


class MergeOut(C.Structure):
    _fields_ = [
        ("out_dtype", _i32), ("reserved0", _i32), ("out", _p), ("out_stride_token", _i64), ("out_stride_head", _i64),
        ("lse", _p), ("lse_stride_token", _i64),
    ]


EXPORTS = {
    "cpattn_last_error": (C.c_char_p, []),
    "cpattn_version": (C.c_char_p, []),
    "cpattn_struct_size": (_i64, [_i32]),
    "cp_slot_map": (_i32, [_p, _i64, _i32, _i32, _i32, _p, _p, _p]),
    "cp_slot_map_rank": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _i64, _p, _p]),
    "cp_kv_write": (_i32, [_p, _i64, _p, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _p, _i64, _i64, _i64, _i64,
                           _i32, _i32, _i32, _i32, _i32, _i32, _i64, _p]),
    "cp_paged_attn_partial": (_i32, [C.POINTER(PagedArgs), _p]),
    "cp_paged_attn_workspace_size": (_i32, [C.POINTER(PagedArgs), C.POINTER(_i64)]),
    "cp_paged_attn_partial_noalloc": (_i32, [C.POINTER(PagedArgs), _p]),
    "cp_paged_attn_merged": (_i32, [C.POINTER(PagedArgs), C.POINTER(MergeOut), _p]),
    "cp_paged_attn_noalloc_scratch_bytes": (_i64, []),
    "cp_own_token_attn": (_i32, [C.POINTER(OwnArgs), _p]),
    "cp_lse_merge": (_i32, [C.POINTER(MergeArgs), _p]),
    "cp_stripe_length": (_i32, [_i32, _i32, _i32, _i32, _i32, C.POINTER(_i32)]),
    "cp_debug_gather_stripe": (_i32, [_p, _i32, _i64, _i64, _i64, _i64, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _p, _i64, C.POINTER(_i32), _p]),
    "cp_debug_stream_read": (_i32, [_p, _i64, _p, _i32, _p]),
}

_LIB = None


class CpattnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"cpattn status {code}: {msg}")
        self.code = code


def load():
    """Load libcpattn.so (once) and bind the exported functions; raise if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m cp_slot_map_amd.build` "
                          "(or __graft_entry__.build()) first. There is no non-HIP fallback.")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    sizes = [lib.cpattn_struct_size(i) for i in range(4)]
    mine = [C.sizeof(PagedArgs), C.sizeof(OwnArgs), C.sizeof(MergeArgs), C.sizeof(MergeOut)]
    if sizes != mine:
        raise ImportError(f"libcpattn struct sizes {sizes} do not match the binding's {mine}")
    _LIB = lib
    return lib


def check(status):
    if status != CPATTN_OK:
        raise CpattnError(status, _LIB.cpattn_last_error().decode())

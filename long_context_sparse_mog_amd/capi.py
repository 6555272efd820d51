"""ctypes mirror of ``include/mog.h``: the structs and the exported functions of
libmog, with the same names.  Argument marshalling only; every step of the
method runs in the library's HIP kernels.  Importing this module does not load
the library; the first call does, and fails loudly if it is not built.
"""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libmog.so")

MOG_MAX_SEQ = 256
MOG_MAX_LEN = 1 << 22
MOG_MAX_FOLD = 1 << 15
MOG_DECODE_NOALLOC_MAX_WS = 64 << 20

(MOG_OK, MOG_ERR_INVALID_ARG, MOG_ERR_UNSUPPORTED, MOG_ERR_WORKSPACE, MOG_ERR_HIP,
 MOG_ERR_CAPACITY) = range(6)
MOG_F32, MOG_BF16 = 0, 1
MOG_KV_CONTIGUOUS, MOG_KV_PAGED = 0, 1
MOG_OP_BUILD, MOG_OP_DECODE, MOG_OP_DENSE = 0, 1, 2

i32 = C.c_int32
i64 = C.c_int64
vp = C.c_void_p


class mog_kv(C.Structure):
    _fields_ = [("format", i32), ("dtype", i32), ("n_seq", i32), ("n_kv_heads", i32),
                ("head_dim", i32), ("max_len", i32), ("page_size", i32), ("n_pages", i32),
                ("max_blocks", i32), ("seq_lens", C.POINTER(i32)), ("k", vp), ("v", vp),
                ("block_table", vp)]


class mog_dims(C.Structure):
    _fields_ = [("n_seq", i32), ("n_kv_heads", i32), ("head_dim", i32), ("dtype", i32),
                ("n_sink", i32), ("n_recent", i32), ("fold_capacity", i32), ("fm_dim", i32),
                ("rows_external", i32), ("seq_lens", C.POINTER(i32))]


class mog_unit(C.Structure):
    _fields_ = [("seq", i32), ("kv_head", i32), ("N", i32), ("n_mid", i32), ("C", i32),
                ("S", i32), ("n_fold", i32), ("reserved1", i32), ("row_base", i64),
                ("cl_base", i64), ("sub_base", i64), ("off_base", i64)]


class mog_layout(C.Structure):
    _fields_ = [("n_seq", i32), ("n_kv_heads", i32), ("head_dim", i32), ("dtype", i32),
                ("n_sink", i32), ("n_recent", i32), ("n_units", i32), ("max_C", i32),
                ("max_S", i32), ("fold_capacity", i32), ("fm_dim", i32), ("fm_scale", C.c_float),
                ("seq_lens", i32 * MOG_MAX_SEQ),
                ("fold_count", i32 * MOG_MAX_SEQ), ("total_mid", i64),
                ("total_cl", i64), ("total_sub", i64), ("total_off", i64), ("units", vp),
                ("k_mid", vp), ("v_mid", vp), ("perm", vp), ("sub_off", vp), ("cl_ms", vp),
                ("cl_vbar", vp), ("sub_ms", vp), ("sub_vbar", vp), ("cl_ms16", vp), ("cl_vbar16", vp),
                ("sub_ms16", vp), ("sub_vbar16", vp), ("fold_sub", vp),
                ("fold_pos", vp), ("cl_fold", vp), ("sub_fold", vp),
                ("append_scratch", vp), ("fm_w", vp), ("cl_fz", vp), ("sub_fz", vp),
                ("rows_external", i32)]


class mog_build_params(C.Structure):
    _fields_ = [("kmeans_iters", i32), ("n_sink", i32), ("n_recent", i32), ("fold_capacity", i32),
                ("seed", C.c_uint64), ("fm_dim", i32), ("fm_scale", C.c_float), ("fm_w", vp),
                ("rows_k", vp), ("rows_v", vp)]


class mog_decode_params(C.Structure):
    _fields_ = [("n_q_heads", i32), ("top_c", i32), ("top_s", i32), ("residual", i32),
                ("scale", C.c_float), ("splits", i32), ("shared_selection", i32),
                ("top_c_per_seq", C.POINTER(i32)),
                ("top_s_per_seq", C.POINTER(i32)), ("exact_begin", vp), ("exact_end", vp),
                ("exact_repeat", i32)]


# name -> (restype, argtypes); every name is declared in include/mog.h
SIGNATURES = {
    "mog_layout_size": (i32, [C.POINTER(mog_dims), C.POINTER(C.c_size_t)]),
    "mog_layout_rows": (i32, [C.POINTER(mog_dims), C.POINTER(i64)]),
    "mog_layout_init": (i32, [C.POINTER(mog_dims), vp, C.c_size_t, C.POINTER(mog_layout), vp]),
    "mog_layout_unit": (i32, [C.POINTER(mog_layout), i32, C.POINTER(mog_unit)]),
    "mog_layout_sync_stats": (i32, [C.POINTER(mog_layout), vp]),
    "mog_workspace_size": (i32, [i32, C.POINTER(mog_kv), C.POINTER(mog_layout),
                                 C.POINTER(mog_build_params), C.POINTER(mog_decode_params),
                                 C.POINTER(C.c_size_t)]),
    "mog_build": (i32, [C.POINTER(mog_kv), C.POINTER(mog_build_params), vp, C.c_size_t, vp,
                        C.c_size_t, C.POINTER(mog_layout), vp]),
    "mog_decode": (i32, [C.POINTER(mog_layout), C.POINTER(mog_kv), vp,
                         C.POINTER(mog_decode_params), vp, vp, vp, vp, vp, C.c_size_t, vp]),
    "mog_decode_noalloc": (i32, [C.POINTER(mog_layout), C.POINTER(mog_kv), vp,
                                 C.POINTER(mog_decode_params), vp, vp, vp, vp, vp]),
    "mog_append": (i32, [C.POINTER(mog_kv), C.POINTER(mog_layout), vp]),
    "mog_dense_decode": (i32, [C.POINTER(mog_kv), vp, C.POINTER(mog_decode_params), vp, vp, vp,
                               C.c_size_t, vp]),
    "mog_status_string": (C.c_char_p, [i32]),
    "mog_last_error": (C.c_char_p, []),
}

_lib = None


class MogError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


def lib() -> C.CDLL:
    """The loaded libmog; raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libmog is not built ({LIB_PATH} missing); run "
                "`python -m long_context_sparse_mog_amd.build_lib` (there is no fallback path)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int, where: str) -> None:
    if status != MOG_OK:
        detail = lib().mog_last_error().decode()
        raise MogError(status, where, detail or lib().mog_status_string(status).decode())


def int_array(values) -> C.Array:
    arr = (i32 * max(1, len(values)))()
    for i, v in enumerate(values):
        arr[i] = int(v)
    return arr

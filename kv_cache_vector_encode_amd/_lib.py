"""ctypes declarations of libtq's C ABI (include/tq.h). Loading fails loudly if the
library has not been built: there is no fallback path."""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
STATUS = {0: "TQ_OK", -1: "TQ_ERR_INVALID_ARG", -2: "TQ_ERR_NULL", -3: "TQ_ERR_ALIGN",
          -4: "TQ_ERR_NOT_ORTHOGONAL", -5: "TQ_ERR_WORKSPACE", -6: "TQ_ERR_HIP", -7: "TQ_ERR_NO_DEVICE"}

# every function include/tq.h declares
EXPORTS = (
    "tq_version", "tq_last_error", "tq_codebook_init", "tq_codebook_get", "tq_codebook_dims",
    "tq_codebook_free", "tq_rotation_from_gaussian", "tq_rotation_from_matrix", "tq_rotation_compute",
    "tq_rotation_get", "tq_rotation_dims", "tq_rotation_free", "tq_rotation_hadamard", "tq_encode",
    "tq_encode_norm_corrected", "tq_decode",
    "tq_attn_workspace_size", "tq_scores_compressed", "tq_attn_decode", "tq_attn_decode_noalloc",
    "tq_window_append_workspace_size",
    "tq_window_append", "tq_gq_encode", "tq_gq_decode", "tq_qjl_create", "tq_qjl_free", "tq_qjl_encode",
)


class AttnParams(C.Structure):
    _fields_ = [
        ("cb_k", C.c_void_p), ("cb_v", C.c_void_p), ("rot_k", C.c_void_p), ("rot_v", C.c_void_p),
        ("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
        ("q", C.c_void_p), ("q_dtype", C.c_int32),
        ("k_packed", C.c_void_p), ("k_norms", C.c_void_p), ("v_packed", C.c_void_p), ("v_norms", C.c_void_p),
        ("seq_lens", C.c_void_p), ("max_seq_len", C.c_int32),
        ("block_table", C.c_void_p), ("block_size", C.c_int32), ("max_blocks_per_seq", C.c_int32),
        ("batch_per_rot", C.c_int32), ("scale", C.c_float),
        ("out", C.c_void_p), ("out_dtype", C.c_int32), ("lse", C.c_void_p),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t), ("num_splits", C.c_int32),
        ("k_window", C.c_void_p), ("v_window", C.c_void_p), ("window", C.c_int32), ("window_dtype", C.c_int32),
        ("qjl_k", C.c_void_p), ("k_signs", C.c_void_p), ("k_rnorms", C.c_void_p),
    ]


class WindowAppendParams(C.Structure):
    _fields_ = [
        ("cb_k", C.c_void_p), ("cb_v", C.c_void_p), ("rot_k", C.c_void_p), ("rot_v", C.c_void_p),
        ("batch", C.c_int32), ("num_kv_heads", C.c_int32), ("n_new", C.c_int32),
        ("k_new", C.c_void_p), ("v_new", C.c_void_p), ("k_window", C.c_void_p), ("v_window", C.c_void_p),
        ("window", C.c_int32), ("window_dtype", C.c_int32), ("seq_lens", C.c_void_p),
        ("k_packed", C.c_void_p), ("k_norms", C.c_void_p), ("v_packed", C.c_void_p), ("v_norms", C.c_void_p),
        ("max_seq_len", C.c_int32), ("block_table", C.c_void_p), ("block_size", C.c_int32),
        ("max_blocks_per_seq", C.c_int32), ("batch_per_rot", C.c_int32),
        ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
    ]


_LIB = None


def lib():
    """The loaded libtq.so (raises if it is missing)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError("libtq.so is not built (expected at %s); run "
                          "`python -m kv_cache_vector_encode_amd.build_lib`" % LIB_PATH)
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, f32 = C.c_void_p, C.c_int, C.c_int64, C.c_float
    sig = {
        "tq_version": ([], i32),
        "tq_last_error": ([], C.c_char_p),
        "tq_codebook_init": ([i32, i32], vp),
        "tq_codebook_get": ([vp, vp, vp, vp], i32),
        "tq_codebook_dims": ([vp, vp, vp], i32),
        "tq_codebook_free": ([vp], None),
        "tq_rotation_from_gaussian": ([i32, i32, vp], vp),
        "tq_rotation_from_matrix": ([i32, i32, vp], vp),
        "tq_rotation_hadamard": ([i32, i32, vp], vp),
        "tq_rotation_compute": ([i32, vp, vp], i32),
        "tq_rotation_get": ([vp, vp], i32),
        "tq_rotation_dims": ([vp, vp, vp], i32),
        "tq_rotation_free": ([vp], None),
        "tq_encode": ([vp, vp, i64, vp, i32, i64, i64, vp, vp, vp, vp], i32),
        "tq_encode_norm_corrected": ([vp, vp, i64, vp, i32, i64, i64, vp, vp, vp, vp], i32),
        "tq_decode": ([vp, vp, i64, vp, vp, vp, i64, vp, i32, vp], i32),
        "tq_attn_workspace_size": ([C.POINTER(AttnParams)], C.c_size_t),
        "tq_scores_compressed": ([C.POINTER(AttnParams), vp, vp], i32),
        "tq_attn_decode": ([C.POINTER(AttnParams), vp], i32),
        "tq_attn_decode_noalloc": ([C.POINTER(AttnParams), vp], i32),
        "tq_window_append_workspace_size": ([C.POINTER(WindowAppendParams)], C.c_size_t),
        "tq_window_append": ([C.POINTER(WindowAppendParams), vp], i32),
        "tq_gq_encode": ([i32, i32, vp, i32, i64, i64, vp, vp, vp, vp], i32),
        "tq_gq_decode": ([i32, i32, vp, vp, vp, i64, vp, i32, vp], i32),
        "tq_qjl_create": ([vp, vp], vp),
        "tq_qjl_free": ([vp], None),
        "tq_qjl_encode": ([vp, vp, i64, vp, i32, i64, i64, vp, vp, vp, vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _LIB = L
    return L


class TQError(RuntimeError):
    def __init__(self, status, msg: str):
        # status is None for a failed handle creation (the C call returns NULL)
        head = "handle creation failed" if status is None else "%s (%d)" % (STATUS.get(status, "?"), status)
        super().__init__("%s: %s" % (head, msg))
        self.status = status


def check(status: int):
    if status != 0:
        raise TQError(status, lib().tq_last_error().decode())
    return status


def last_error() -> str:
    return lib().tq_last_error().decode()

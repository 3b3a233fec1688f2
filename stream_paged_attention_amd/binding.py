"""ctypes binding of libtfattn.so, the C ABI in include/tf_attn.h.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Pointers are passed as Python ints (device addresses from
``torch.Tensor.data_ptr()``), streams as the ``hipStream_t`` handle
(``torch.cuda.current_stream().cuda_stream``).  There is no fallback: if the
library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtfattn.so")

TF_KV_CONTIG, TF_KV_PAGED, TF_KV_RING = 0, 1, 2
KIND_CODE = {"contig": TF_KV_CONTIG, "paged": TF_KV_PAGED, "ring": TF_KV_RING}

TF_MASK_CAUSAL, TF_MASK_FULL, TF_MASK_TREE = 0, 1, 2
MASK_CODE = {"causal": TF_MASK_CAUSAL, "full": TF_MASK_FULL, "tree": TF_MASK_TREE}

TF_OK = 0
TF_E_INVALID = -1
TF_E_UNSUPPORTED = -2
TF_E_PAST_PAGES = -3
TF_E_WORKSPACE = -4
TF_E_LAUNCH = -5

TF_ERR_PAST_PAGES = 1
TF_ERR_BAD_PAGE = 2
TF_ERR_BAD_ROWS = 4
TF_ERR_BAD_RING = 8
TF_ERR_PARTIALS = 16
TF_ERR_BAD_LAYER = 32
TF_ERR_HINTS = 64
TF_ERR_STORAGE = 128

TF_STATIC_PARTIALS_BYTES = 16 << 20

EXPORTS = ("tf_attn_rows", "tf_attn_merge", "tf_attn_static", "tf_argmax", "tf_argmax_workspace_bytes",
           "tf_kv_put", "tf_state_save", "tf_state_restore", "tf_plan_partials",
           "tf_check_segments", "tf_strerror")


class tf_segment(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pages", ctypes.c_void_p),
                ("capacity", ctypes.c_int32), ("first", ctypes.c_int32),
                ("row_offset", ctypes.c_int32), ("n_rows", ctypes.c_int32),
                ("key_count", ctypes.c_int32), ("partial_offset", ctypes.c_int32)]


class tf_attn_args(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("total_rows", ctypes.c_int32), ("max_rows", ctypes.c_int32),
                ("max_keys", ctypes.c_int32), ("min_rows", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("pool_pages", ctypes.c_int32),
                ("split_keys", ctypes.c_int32), ("scale", ctypes.c_float),
                ("mask", ctypes.c_int32),
                ("segs", ctypes.c_void_p), ("tree", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("partials", ctypes.c_void_p), ("partials_bytes", ctypes.c_size_t),
                ("err", ctypes.c_void_p)]


class tf_put_args(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("n_segments", ctypes.c_int32),
                ("total_rows", ctypes.c_int32), ("max_rows", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("pool_pages", ctypes.c_int32),
                ("segs", ctypes.c_void_p), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("err", ctypes.c_void_p)]


class tf_state_layer(ctypes.Structure):
    _fields_ = [("pool_k", ctypes.c_void_p), ("pool_v", ctypes.c_void_p),
                ("state_k", ctypes.c_void_p), ("state_v", ctypes.c_void_p)]


class tf_state_args(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("pool_pages", ctypes.c_int32), ("at", ctypes.c_int32),
                ("n_pages", ctypes.c_int32), ("pages", ctypes.c_void_p),
                ("layers", ctypes.c_void_p), ("err", ctypes.c_void_p)]


assert ctypes.sizeof(tf_segment) == 48

_lib = None


def load(path: str = LIB_PATH):
    """Open the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run __graft_entry__.build() or stream_paged_attention_amd/build.py)")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.tf_attn_rows.restype = ctypes.c_int
    lib.tf_attn_rows.argtypes = [ctypes.POINTER(tf_attn_args), vp]
    lib.tf_attn_merge.restype = ctypes.c_int
    lib.tf_attn_merge.argtypes = [ctypes.POINTER(tf_attn_args), vp]
    lib.tf_attn_static.restype = ctypes.c_int
    lib.tf_attn_static.argtypes = [ctypes.POINTER(tf_attn_args), vp]
    lib.tf_argmax.restype = ctypes.c_int
    lib.tf_argmax.argtypes = [vp, i32, i32, ctypes.c_int64, vp, vp, vp, sz, vp]
    lib.tf_argmax_workspace_bytes.restype = sz
    lib.tf_argmax_workspace_bytes.argtypes = [i32, i32]
    lib.tf_kv_put.restype = ctypes.c_int
    lib.tf_kv_put.argtypes = [ctypes.POINTER(tf_put_args), vp]
    for name in ("tf_state_save", "tf_state_restore"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [ctypes.POINTER(tf_state_args), vp]
    lib.tf_plan_partials.restype = ctypes.c_int
    lib.tf_plan_partials.argtypes = [ctypes.POINTER(tf_segment), i32, i32, i32, i32,
                                     ctypes.POINTER(sz)]
    lib.tf_check_segments.restype = ctypes.c_int
    lib.tf_check_segments.argtypes = [ctypes.POINTER(tf_attn_args), ctypes.POINTER(tf_segment)]
    lib.tf_strerror.restype = ctypes.c_char_p
    lib.tf_strerror.argtypes = [ctypes.c_int]
    if path == LIB_PATH:
        _lib = lib
    return lib


def tf_attn_rows(args: tf_attn_args, stream: int, lib=None) -> int:
    return (lib or load()).tf_attn_rows(ctypes.byref(args), ctypes.c_void_p(stream))


def tf_attn_merge(args: tf_attn_args, stream: int, lib=None) -> int:
    return (lib or load()).tf_attn_merge(ctypes.byref(args), ctypes.c_void_p(stream))


def tf_attn_static(args: tf_attn_args, stream: int, lib=None) -> int:
    return (lib or load()).tf_attn_static(ctypes.byref(args), ctypes.c_void_p(stream))


def tf_argmax(logits: int, n_rows: int, vocab: int, row_stride: int, ids: int, flags: int,
              workspace: int, workspace_bytes: int, stream: int, lib=None) -> int:
    return (lib or load()).tf_argmax(logits, n_rows, vocab, row_stride, ids, flags, workspace,
                                     workspace_bytes, ctypes.c_void_p(stream))


def tf_argmax_workspace_bytes(n_rows: int, vocab: int, lib=None) -> int:
    return int((lib or load()).tf_argmax_workspace_bytes(n_rows, vocab))


def tf_kv_put(args: tf_put_args, stream: int, lib=None) -> int:
    return (lib or load()).tf_kv_put(ctypes.byref(args), ctypes.c_void_p(stream))


def tf_state_save(args: tf_state_args, stream: int, lib=None) -> int:
    return (lib or load()).tf_state_save(ctypes.byref(args), ctypes.c_void_p(stream))


def tf_state_restore(args: tf_state_args, stream: int, lib=None) -> int:
    return (lib or load()).tf_state_restore(ctypes.byref(args), ctypes.c_void_p(stream))


def tf_plan_partials(segs, n_q_heads: int, head_dim: int, split_keys: int, lib=None):
    """Fill partial_offset of a ctypes tf_segment array; returns (rc, partials_bytes)."""
    out = ctypes.c_size_t(0)
    rc = (lib or load()).tf_plan_partials(segs, len(segs), n_q_heads, head_dim, split_keys,
                                          ctypes.byref(out))
    return rc, int(out.value)


def tf_check_segments(args: tf_attn_args, segs, lib=None) -> int:
    return (lib or load()).tf_check_segments(ctypes.byref(args), segs)


def tf_strerror(code: int, lib=None) -> str:
    return (lib or load()).tf_strerror(code).decode()

"""ctypes front end of the float64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()`` and
by the CPU-baseline leg of bench.py.  The HIP library never imports it.

Inputs are plain numpy arrays: bf16 bit patterns as uint16, each stream's
*logical* K/V rows ``[key][kv_head][dim]``.  Nothing here knows about pages,
rings or the HIP path's partial layout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open an oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    _declare(lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = load_library(_LIB)
    return _lib


def _declare(lib) -> None:
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_attn.restype = ctypes.c_int
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.oracle_attn.argtypes = [ctypes.c_int, i32p, i32p, i32p, i64p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, ctypes.c_double, u16p, u16p,
                                u16p, ctypes.c_int, u64p, f64p, ctypes.c_int]
    lib.oracle_attn_partials.restype = ctypes.c_int
    lib.oracle_attn_partials.argtypes = [ctypes.c_int, i32p, i32p, i32p, i64p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_double, u16p, u16p, u16p, ctypes.c_int,
                                         u64p, ctypes.c_int, ctypes.c_int, f64p, f64p, f64p,
                                         ctypes.c_int]
    lib.oracle_merge.restype = None
    lib.oracle_merge.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, f64p, f64p,
                                 f64p, f64p]
    lib.oracle_argmax.restype = None
    lib.oracle_argmax.argtypes = [u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                  i32p, ctypes.POINTER(ctypes.c_uint8)]


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


MASKS = {"causal": 0, "full": 1, "tree": 2}


def _mask_args(mask: str, tree, n_total_rows: int):
    """(mask code, uint64 ancestor masks per packed row, kept alive by the caller)."""
    code = MASKS[mask]
    if code == MASKS["tree"]:
        t = np.ascontiguousarray(tree, dtype=np.uint64)
        assert t.shape == (n_total_rows,)
    else:
        t = np.zeros(1, dtype=np.uint64)
    return code, t


def _concat(arrs):
    return np.ascontiguousarray(np.concatenate([np.asarray(a, np.uint16) for a in arrs]))


def _layout(n_rows: Sequence[int], key_counts: Sequence[int], k_logical, v_logical):
    n_rows = np.ascontiguousarray(n_rows, dtype=np.int32)
    kcs = np.ascontiguousarray(key_counts, dtype=np.int32)
    offs = np.zeros(len(n_rows), dtype=np.int32)
    if len(n_rows) > 1:
        offs[1:] = np.cumsum(n_rows)[:-1]
    base = np.zeros(len(kcs), dtype=np.int64)
    if len(kcs) > 1:
        base[1:] = np.cumsum(kcs.astype(np.int64))[:-1]
    for k, kc in zip(k_logical, kcs):
        assert k.shape[0] == kc
    return n_rows, kcs, offs, base, _concat(k_logical), _concat(v_logical)


def attn_raw(n_rows, key_counts, row_offsets, key_base, q, k_all, v_all, *, n_q_heads,
             n_kv_heads, head_dim, scale, mask: str = "causal", tree=None, threads: int = 0,
             lib=None):
    """Unsplit attention over explicit per-segment offsets.

    Segment s reads query rows ``row_offsets[s] ..`` of ``q`` and keys
    ``key_base[s] ..`` of the concatenated logical ``k_all``/``v_all``.
    ``mask`` is "causal", "full" or "tree" (then ``tree`` holds one uint64
    ancestor mask per row of ``q``).  Returns ``(out, threads_used)``.
    """
    lib = lib or _load()
    assert n_q_heads % n_kv_heads == 0
    nr = np.ascontiguousarray(n_rows, dtype=np.int32)
    kcs = np.ascontiguousarray(key_counts, dtype=np.int32)
    offs = np.ascontiguousarray(row_offsets, dtype=np.int32)
    base = np.ascontiguousarray(key_base, dtype=np.int64)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k_all = np.ascontiguousarray(k_all, dtype=np.uint16)
    v_all = np.ascontiguousarray(v_all, dtype=np.uint16)
    assert q.shape[1:] == (n_q_heads, head_dim)
    assert np.all(nr >= 1) and np.all(nr <= kcs)
    assert int((offs + nr).max()) <= q.shape[0]
    assert int((base + kcs).max()) <= k_all.shape[0] and k_all.shape == v_all.shape
    assert k_all.shape[1:] == (n_kv_heads, head_dim)
    if mask == "tree":
        assert int(nr.max()) <= 64
    code, tr = _mask_args(mask, tree, q.shape[0])
    out = np.full((q.shape[0], n_q_heads, head_dim), np.nan, dtype=np.float64)
    used = lib.oracle_attn(len(nr), _p(nr, ctypes.c_int32), _p(kcs, ctypes.c_int32),
                           _p(offs, ctypes.c_int32), _p(base, ctypes.c_int64), n_q_heads,
                           n_kv_heads, head_dim, float(scale), _p(q, ctypes.c_uint16),
                           _p(k_all, ctypes.c_uint16), _p(v_all, ctypes.c_uint16), code,
                           _p(tr, ctypes.c_uint64), _p(out, ctypes.c_double), int(threads))
    return out, used


def attn(n_rows, key_counts, q, k_logical, v_logical, *, n_q_heads, n_kv_heads, head_dim,
         scale, mask: str = "causal", tree=None, threads: int = 0,
         return_threads: bool = False, lib=None):
    """Unsplit softmax attention in float64 -> ``[total_rows][Hq][D]``."""
    nr, kcs, offs, base, k_all, v_all = _layout(n_rows, key_counts, k_logical, v_logical)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    assert q.shape[0] == int(nr.sum())
    out, used = attn_raw(nr, kcs, offs, base, q, k_all, v_all, n_q_heads=n_q_heads,
                         n_kv_heads=n_kv_heads, head_dim=head_dim, scale=scale, mask=mask,
                         tree=tree, threads=threads, lib=lib)
    return (out, used) if return_threads else out


def attn_partials(n_rows, key_counts, q, k_logical, v_logical, *, n_q_heads, n_kv_heads,
                  head_dim, scale, split, mask: str = "causal", tree=None, threads: int = 0,
                  lib=None):
    """Split-K partials in float64.

    Returns ``(m, l, o)`` with shapes ``[rows][Hq][n_split]`` and
    ``[rows][Hq][n_split][D]``; ``n_split = ceil(max key_count / split)``.
    """
    lib = lib or _load()
    nr, kcs, offs, base, k_all, v_all = _layout(n_rows, key_counts, k_logical, v_logical)
    q = np.ascontiguousarray(q, dtype=np.uint16)
    total = int(nr.sum())
    n_split = int(-(-int(kcs.max()) // split))
    m = np.empty((total, n_q_heads, n_split), dtype=np.float64)
    l = np.empty_like(m)
    o = np.empty((total, n_q_heads, n_split, head_dim), dtype=np.float64)
    code, tr = _mask_args(mask, tree, total)
    lib.oracle_attn_partials(len(nr), _p(nr, ctypes.c_int32), _p(kcs, ctypes.c_int32),
                             _p(offs, ctypes.c_int32), _p(base, ctypes.c_int64), n_q_heads,
                             n_kv_heads, head_dim, float(scale), _p(q, ctypes.c_uint16),
                             _p(k_all, ctypes.c_uint16), _p(v_all, ctypes.c_uint16), code,
                             _p(tr, ctypes.c_uint64), int(split), n_split, _p(m, ctypes.c_double),
                             _p(l, ctypes.c_double), _p(o, ctypes.c_double), int(threads))
    return m, l, o


def merge(m: np.ndarray, l: np.ndarray, o: np.ndarray, lib=None) -> np.ndarray:
    """Merge partials ``(m, l, o)`` over their split axis (axis -1 of m)."""
    lib = lib or _load()
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.ascontiguousarray(o, dtype=np.float64)
    n_split = m.shape[-1]
    d = o.shape[-1]
    n = int(np.prod(m.shape[:-1]))
    out = np.empty(m.shape[:-1] + (d,), dtype=np.float64)
    lib.oracle_merge(n, n_split, d, _p(m, ctypes.c_double), _p(l, ctypes.c_double),
                     _p(o, ctypes.c_double), _p(out, ctypes.c_double))
    return out


def argmax(logits: np.ndarray, vocab: int | None = None, lib=None):
    """First largest id and nonfinite flag per row of bf16 logits ``[rows][>=vocab]``."""
    lib = lib or _load()
    logits = np.ascontiguousarray(logits, dtype=np.uint16)
    rows, stride = logits.shape
    vocab = stride if vocab is None else vocab
    ids = np.empty(rows, dtype=np.int32)
    flags = np.empty(rows, dtype=np.uint8)
    lib.oracle_argmax(_p(logits, ctypes.c_uint16), rows, vocab, stride,
                      _p(ids, ctypes.c_int32), _p(flags, ctypes.c_uint8))
    return ids, flags


def attn_workload(w, rows=None, threads: int = 0, return_threads: bool = False):
    """Oracle output for a synthetic workload (all rows, or a sample of packed rows).

    The workload's ``mask`` ("causal", "full" or "tree", with ``tree`` the
    ancestor masks) picks the keys each row sees.  A sampled row r of an
    n-row segment is evaluated as a one-row segment over the keys it sees when
    those are a prefix of its stream: the first ``kc - n + r + 1`` (causal) or
    all ``kc`` (full).  Under a tree mask the sampled rows' whole segments are
    evaluated.  With ``rows`` given, the result has one entry per sampled row.
    """
    mask = getattr(w, "mask", "causal")
    kw = dict(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
              scale=w.scale, threads=threads)
    kcs_all = [s.key_count for s in w.segments]
    base_all = np.zeros(len(kcs_all), dtype=np.int64)
    if len(kcs_all) > 1:
        base_all[1:] = np.cumsum(np.asarray(kcs_all, dtype=np.int64))[:-1]
    k_all = _concat(w.k_logical)
    v_all = _concat(w.v_logical)
    if rows is None or mask == "tree":
        out, used = attn_raw([s.n_rows for s in w.segments], kcs_all,
                             [s.row_offset for s in w.segments], base_all, w.q, k_all, v_all,
                             mask=mask, tree=getattr(w, "tree", None), **kw)
        if rows is not None:
            out = out[[int(r) for r in rows]]
        return (out, used) if return_threads else out
    seg_of = []
    for si, s in enumerate(w.segments):
        seg_of.extend((si, r) for r in range(s.n_rows))
    rows = [int(r) for r in rows]
    n_rows, kcs, offs, base = [], [], [], []
    for i, row in enumerate(rows):
        si, r = seg_of[row]
        s = w.segments[si]
        n_rows.append(1)
        kcs.append(s.key_count if mask == "full" else s.key_count - s.n_rows + r + 1)
        offs.append(i)
        base.append(base_all[si])
    out, used = attn_raw(n_rows, kcs, offs, base, w.q[rows], k_all, v_all, **kw)
    return (out, used) if return_threads else out

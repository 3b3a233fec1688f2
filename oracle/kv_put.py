"""Reference KV append: where each new key and value row of a round goes.

TEST INFRASTRUCTURE ONLY: imported by tests/ (and nothing else); the HIP
library never imports it and shares no code with it.

What it computes (TensorFold PR #1653, "spark25 CUDA: the full layers' caches
in pages of the core pool ...", the commit that writes a chunk's K/V rows into
the pool's pages, page by page; TensorFold PR #1562, the MTP drafter's shared
round, whose ring rows are written at the ring's head and step the slot with a
wrap):

  * A segment's new keys are its last n_rows logical keys,
    j = key_count - n_rows + r for row r (the round's rows are in the cache
    before the round attends; a row sees itself).
  * Row r's K (and V) vector for every kv head comes from packed row
    row_offset + r of k_new / v_new ([rows][kv_head][dim]).
  * Logical key j of a paged stream lives in page pages[j // P] at offset
    j % P; of a ring in slot (first + j) mod slots; of a contiguous buffer in
    row j.  Nothing else is written.

Storage layouts match the library's: pool [page][kv_head][P][dim], rings and
buffers [kv_head][slots][dim], all bf16 bit patterns (uint16).  Plain loops,
one key at a time; error cases (a key past the storage) raise.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def put_paged(pool_k: np.ndarray, pool_v: np.ndarray, segments: Sequence, k_new: np.ndarray,
              v_new: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Copies of the K and V pools with every segment's new rows written.

    ``segments``: objects with n_rows, key_count, row_offset and pages (the
    stream's page list)."""
    k, v = pool_k.copy(), pool_v.copy()
    page_size = k.shape[2]
    for s in segments:
        for r in range(s.n_rows):
            j = s.key_count - s.n_rows + r
            page = int(s.pages[j // page_size])
            off = j % page_size
            for h in range(k.shape[1]):
                k[page, h, off, :] = k_new[s.row_offset + r, h, :]
                v[page, h, off, :] = v_new[s.row_offset + r, h, :]
    return k, v


def put_ring(ring_k: np.ndarray, ring_v: np.ndarray, seg, k_new: np.ndarray,
             v_new: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Copies of one stream's ring [kv_head][slots][dim] with its new rows written
    (``seg``: n_rows, key_count, row_offset, first)."""
    k, v = ring_k.copy(), ring_v.copy()
    slots = k.shape[1]
    for r in range(seg.n_rows):
        j = seg.key_count - seg.n_rows + r
        slot = (seg.first + j) % slots
        for h in range(k.shape[0]):
            k[h, slot, :] = k_new[seg.row_offset + r, h, :]
            v[h, slot, :] = v_new[seg.row_offset + r, h, :]
    return k, v


def put_contig(buf_k: np.ndarray, buf_v: np.ndarray, seg, k_new: np.ndarray,
               v_new: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Copies of one stream's buffer [kv_head][capacity][dim] with its new rows written."""
    k, v = buf_k.copy(), buf_v.copy()
    if seg.key_count > k.shape[1]:
        raise ValueError("key past the buffer")
    for r in range(seg.n_rows):
        j = seg.key_count - seg.n_rows + r
        for h in range(k.shape[0]):
            k[h, j, :] = k_new[seg.row_offset + r, h, :]
            v[h, j, :] = v_new[seg.row_offset + r, h, :]
    return k, v


def new_rows(k_logical: Sequence[np.ndarray], segments: Sequence) -> np.ndarray:
    """The packed source a round hands over: each segment's last n_rows logical
    rows, in packed row order ([rows][kv_head][dim])."""
    rows = [k_logical[i][s.key_count - s.n_rows:s.key_count] for i, s in enumerate(segments)]
    return np.ascontiguousarray(np.concatenate(rows, axis=0))

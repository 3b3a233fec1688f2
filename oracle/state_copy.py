"""Reference kept-state copy: the K and V rows of a stream's positions [0, at).

TEST INFRASTRUCTURE ONLY: imported by tests/ (and nothing else);
the HIP library never imports it and shares no code with it.

What it computes (TensorFold PR #1503, the prompt-cache commit of the
lfm2_moe pool: a kept state is every attention layer's K/V rows [0, at),
taken from the stream's pool pages and later restored into the pages the
resuming stream leases):

  * Position j of a stream lives in pool page pages[j // P] at offset j % P
    (pool layout [page][kv_head][P][dim]).
  * save: for every layer and every j < at, the state's row (j // P, :, j % P)
    takes the pool's row (pages[j // P], :, j % P); a state buffer is the
    stream's logical pages in order, [ceil(at / P)][kv_head][P][dim].
  * restore: the same rows copied back, into another page list.
  * Nothing else is written: state rows at or past `at` (save) and every pool
    row not named by a position below `at` (restore) keep their contents.

Plain loops, one position at a time, on bf16 bit patterns (uint16).
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np


def save(pools: Sequence[Tuple[np.ndarray, np.ndarray]], pages: Sequence[int], at: int,
         states: Sequence[Tuple[np.ndarray, np.ndarray]]) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Copies of the layers' (K, V) state buffers after saving positions [0, at)."""
    out = []
    for (pk, pv), (sk, sv) in zip(pools, states):
        page_size = pk.shape[2]
        nk, nv = sk.copy(), sv.copy()
        for j in range(at):
            lp, off = j // page_size, j % page_size
            pid = int(pages[lp])
            nk[lp, :, off, :] = pk[pid, :, off, :]
            nv[lp, :, off, :] = pv[pid, :, off, :]
        out.append((nk, nv))
    return out


def restore(states: Sequence[Tuple[np.ndarray, np.ndarray]], pages: Sequence[int], at: int,
            pools: Sequence[Tuple[np.ndarray, np.ndarray]]) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Copies of the layers' (K, V) pools after restoring positions [0, at) into `pages`."""
    out = []
    for (sk, sv), (pk, pv) in zip(states, pools):
        page_size = pk.shape[2]
        nk, nv = pk.copy(), pv.copy()
        for j in range(at):
            lp, off = j // page_size, j % page_size
            pid = int(pages[lp])
            nk[pid, :, off, :] = sk[lp, :, off, :]
            nv[pid, :, off, :] = sv[lp, :, off, :]
        out.append((nk, nv))
    return out

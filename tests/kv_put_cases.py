"""Workloads for the KV-append tests: the storage before a round (committed
keys only, poison elsewhere) and the round's packed new rows."""
import dataclasses

import numpy as np

from oracle import kv_put as okv
from stream_paged_attention_amd import synth


def round_inputs(w):
    """(w_before, k_new, v_new): w with only its committed keys placed (same
    pages, ring heads and buffers), and the packed new rows of the round."""
    committed_k = [kl[: s.key_count - s.n_rows] for kl, s in zip(w.k_logical, w.segments)]
    committed_v = [vl[: s.key_count - s.n_rows] for vl, s in zip(w.v_logical, w.segments)]
    if w.kind == "paged":
        lists = [s.pages for s in w.segments]
        before = dataclasses.replace(
            w, pool_k=synth.place_paged(committed_k, w.page_size, w.pool_pages, lists),
            pool_v=synth.place_paged(committed_v, w.page_size, w.pool_pages, lists))
    elif w.kind == "ring":
        before = dataclasses.replace(
            w, store_k=[synth.place_ring(c, s.capacity, s.first) for c, s in zip(committed_k, w.segments)],
            store_v=[synth.place_ring(c, s.capacity, s.first) for c, s in zip(committed_v, w.segments)])
    else:
        before = dataclasses.replace(
            w, store_k=[synth.place_contig(c, s.capacity) for c, s in zip(committed_k, w.segments)],
            store_v=[synth.place_contig(c, s.capacity) for c, s in zip(committed_v, w.segments)])
    return before, okv.new_rows(w.k_logical, w.segments), okv.new_rows(w.v_logical, w.segments)


def oracle_after(before, k_new, v_new):
    """The storage after the round, by the reference."""
    if before.kind == "paged":
        return okv.put_paged(before.pool_k, before.pool_v, before.segments, k_new, v_new)
    put = okv.put_ring if before.kind == "ring" else okv.put_contig
    ks, vs = [], []
    for i, s in enumerate(before.segments):
        k, v = put(before.store_k[i], before.store_v[i], s, k_new, v_new)
        ks.append(k)
        vs.append(v)
    return ks, vs


def workloads():
    """Paged (permuted pool, rows across page boundaries), ring (wrapping),
    contiguous."""
    return [
        synth.make_workload("put-paged", synth.KIND_PAGED, 8, 2, 128, [1, 5, 40], [33, 300, 1000], seed=61,
                            page_size=32, pool_pages=60),
        synth.make_workload("put-ring", synth.KIND_RING, 8, 2, 64, [3, 16], [40, 100], seed=62,
                            ring_slots=[41, 100], ring_heads=[5, 99]),
        synth.make_workload("put-contig", synth.KIND_CONTIG, 16, 4, 256, [2, 7], [20, 500], seed=63,
                            contig_capacity=[30, 512]),
    ]

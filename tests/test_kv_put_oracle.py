"""Pins of the reference KV append (oracle/kv_put.py), CPU only."""
import dataclasses

import numpy as np
import pytest

from oracle import kv_put as okv
from stream_paged_attention_amd import synth
from tests.kv_put_cases import oracle_after, round_inputs, workloads


@pytest.mark.parametrize("w", workloads(), ids=lambda w: w.name)
def test_put_completes_the_generators_placement(w):
    # the generator places every key itself (independent code); appending the
    # new rows to a storage holding only the committed keys must give the same
    before, k_new, v_new = round_inputs(w)
    k, v = oracle_after(before, k_new, v_new)
    if w.kind == "paged":
        assert np.array_equal(k, w.pool_k) and np.array_equal(v, w.pool_v)
    else:
        for i in range(len(w.segments)):
            assert np.array_equal(k[i], w.store_k[i]) and np.array_equal(v[i], w.store_v[i])


def test_page_boundary_by_hand():
    # 33 keys, 2 new: keys 31 and 32 go to the last row of the first page and
    # the first row of the second
    seg = synth.Segment(n_rows=2, key_count=33, row_offset=0, pages=np.array([7, 3], dtype=np.int32))
    pool = np.zeros((10, 2, 32, 64), dtype=np.uint16)
    k_new = np.arange(2 * 2 * 64, dtype=np.uint16).reshape(2, 2, 64) + 1
    k, v = okv.put_paged(pool, pool, [seg], k_new, k_new + 1000)
    expect = pool.copy()
    expect[7, :, 31, :] = k_new[0]
    expect[3, :, 0, :] = k_new[1]
    assert np.array_equal(k, expect)
    assert np.array_equal(v[3, :, 0, :], k_new[1] + 1000)
    assert np.count_nonzero(k) == np.count_nonzero(expect)


def test_ring_wrap_by_hand():
    # 5 slots, logical key 0 in slot 3, 4 keys of which the last 3 are new:
    # keys 1, 2, 3 land in slots 4, 0, 1
    seg = synth.Segment(n_rows=3, key_count=4, row_offset=1, first=3, capacity=5)
    ring = np.zeros((1, 5, 64), dtype=np.uint16)
    k_new = (np.arange(4, dtype=np.uint16)[:, None, None] + 1) * np.ones((4, 1, 64), dtype=np.uint16)
    k, _ = okv.put_ring(ring, ring, seg, k_new, k_new)
    assert [int(k[0, s, 0]) for s in range(5)] == [3, 4, 0, 0, 2]


def test_contig_refuses_keys_past_the_buffer():
    seg = synth.Segment(n_rows=1, key_count=9, row_offset=0, capacity=8)
    buf = np.zeros((1, 8, 64), dtype=np.uint16)
    with pytest.raises(ValueError):
        okv.put_contig(buf, buf, seg, np.zeros((1, 1, 64), dtype=np.uint16), np.zeros((1, 1, 64), dtype=np.uint16))


def test_new_rows_are_the_last_keys_in_row_order():
    w = workloads()[0]
    k_new = okv.new_rows(w.k_logical, w.segments)
    assert k_new.shape[0] == w.total_rows
    s = w.segments[2]
    assert np.array_equal(k_new[s.row_offset:s.row_offset + s.n_rows], w.k_logical[2][s.key_count - s.n_rows:])

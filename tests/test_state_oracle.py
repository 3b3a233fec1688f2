"""Pins of the kept-state reference (oracle/state_copy.py) to what the seeded
generator placed, independent of the reference's own loops (CPU only)."""
import numpy as np
import pytest

from oracle import state_copy
from stream_paged_attention_amd import synth
from tests.state_cases import layers_case


@pytest.mark.parametrize("page_size,at", [(32, 100), (32, 128), (64, 1), (512, 700)])
def test_saved_state_holds_the_logical_rows(page_size, at):
    case = layers_case(seed=page_size + at, n_layers=2, hkv=2, d=8, page_size=page_size, at=at)
    states = state_copy.save(case.pools, case.pages, at, case.states)
    for (sk, sv), (lk, lv) in zip(states, case.logical):
        n_pages = -(-at // page_size)
        # the state is the stream's pages in order: read it back as logical rows
        rows_k = synth.gather_paged(sk, np.arange(n_pages), at)
        rows_v = synth.gather_paged(sv, np.arange(n_pages), at)
        np.testing.assert_array_equal(rows_k, lk[:at])
        np.testing.assert_array_equal(rows_v, lv[:at])


def test_state_rows_past_at_keep_their_contents():
    case = layers_case(seed=3, n_layers=1, hkv=2, d=8, page_size=32, at=70)
    states = state_copy.save(case.pools, case.pages, 70, case.states)
    sk, _ = states[0]
    before, _ = case.states[0]
    np.testing.assert_array_equal(sk[2, :, 6:, :], before[2, :, 6:, :])   # rows 70.. of page 2
    assert not np.array_equal(sk[2, :, :6, :], before[2, :, :6, :])


def test_restore_into_new_pages_gives_the_rows_back_and_nothing_else():
    case = layers_case(seed=4, n_layers=2, hkv=2, d=8, page_size=32, at=90)
    states = state_copy.save(case.pools, case.pages, 90, case.states)
    rng = np.random.Generator(np.random.PCG64(4))
    free = np.setdiff1d(np.arange(case.pool_pages), case.pages[:3])
    new_pages = rng.choice(free, size=3, replace=False).astype(np.int32)
    pools2 = state_copy.restore(states, new_pages, 90, case.pools)
    for (pk2, pv2), (pk, pv), (lk, lv) in zip(pools2, case.pools, case.logical):
        np.testing.assert_array_equal(synth.gather_paged(pk2, new_pages, 90), lk[:90])
        np.testing.assert_array_equal(synth.gather_paged(pv2, new_pages, 90), lv[:90])
        # every other pool row is untouched: the three new pages' rows below 90
        # are the only change
        mask = np.ones(pk.shape[0] * pk.shape[2], dtype=bool)
        for j in range(90):
            mask[int(new_pages[j // 32]) * 32 + j % 32] = False
        flat = lambda a: a.transpose(0, 2, 1, 3).reshape(-1, a.shape[1], a.shape[3])
        np.testing.assert_array_equal(flat(pk2)[mask], flat(pk)[mask])
        np.testing.assert_array_equal(flat(pv2)[mask], flat(pv)[mask])


def test_round_trip_to_the_same_pages_changes_nothing():
    case = layers_case(seed=5, n_layers=1, hkv=4, d=8, page_size=64, at=200)
    states = state_copy.save(case.pools, case.pages, 200, case.states)
    pools2 = state_copy.restore(states, case.pages, 200, case.pools)
    for (a, b), (c, d) in zip(pools2, case.pools):
        np.testing.assert_array_equal(a, c)
        np.testing.assert_array_equal(b, d)


def test_empty_state_copies_nothing():
    case = layers_case(seed=6, n_layers=1, hkv=2, d=8, page_size=32, at=40)
    states = state_copy.save(case.pools, case.pages, 0, case.states)
    np.testing.assert_array_equal(states[0][0], case.states[0][0])
    pools2 = state_copy.restore(case.states, case.pages, 0, case.pools)
    np.testing.assert_array_equal(pools2[0][0], case.pools[0][0])

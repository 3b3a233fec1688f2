"""The input generator: bf16 rounding and the placement of logical K/V (CPU only)."""
import numpy as np
import pytest
import torch

from stream_paged_attention_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.standard_normal(100000, dtype=np.float32) * np.float32(3.0)
    # exact ties to even: a value halfway between two bf16 numbers
    x[:4] = np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38], dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(ref),
                                  torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def _check_paged(w):
    used = np.zeros(w.pool_pages, bool)
    for i, s in enumerate(w.segments):
        np.testing.assert_array_equal(synth.gather_paged(w.pool_k, s.pages, s.key_count), w.k_logical[i])
        np.testing.assert_array_equal(synth.gather_paged(w.pool_v, s.pages, s.key_count), w.v_logical[i])
        assert not used[s.pages].any(), "streams share a page"
        used[s.pages] = True
        tail = s.key_count % w.page_size
        if tail:
            assert (w.pool_k[s.pages[-1], :, tail:, :] == synth.BF16_NAN).all()
    assert (w.pool_k[~used] == synth.BF16_NAN).all()
    assert (w.pool_v[~used] == synth.BF16_NAN).all()


def test_paged_placement_round_trips():
    w = synth.make_workload("t", synth.KIND_PAGED, 4, 2, 8, [1, 3, 2], [40, 33, 5], seed=3,
                            page_size=32, pool_pages=12)
    _check_paged(w)
    w2 = synth.restore(w, synth.KIND_PAGED, seed=99, pool_pages=20)
    _check_paged(w2)
    assert any(not np.array_equal(a.pages, b.pages) for a, b in zip(w.segments, w2.segments))


def test_ring_placement_round_trips_and_poisons_the_rest():
    w = synth.make_workload("t", synth.KIND_RING, 4, 2, 8, [2, 1], [30, 50], seed=4,
                            ring_slots=[40, 50], ring_heads=[35, 7])
    for i, s in enumerate(w.segments):
        assert s.first == (([35, 7][i]) - s.key_count) % s.capacity
        np.testing.assert_array_equal(synth.gather_ring(w.store_k[i], s.first, s.key_count), w.k_logical[i])
        valid = (s.first + np.arange(s.key_count)) % s.capacity
        rest = np.setdiff1d(np.arange(s.capacity), valid)
        assert (w.store_v[i][:, rest, :] == synth.BF16_NAN).all()
    # the second ring wraps: key 0 at slot 7, the newest key at slot 6
    assert w.segments[1].first == 7


def test_contig_placement():
    w = synth.make_workload("t", synth.KIND_CONTIG, 2, 1, 4, [1], [9], seed=5,
                            contig_capacity=[16])
    np.testing.assert_array_equal(w.store_k[0][:, :9, :].transpose(1, 0, 2), w.k_logical[0])
    assert (w.store_k[0][:, 9:, :] == synth.BF16_NAN).all()


@pytest.mark.parametrize("name", ["single64", "decode16", "ring17"])
def test_workload_structure(name):
    w = synth.make_synthetic(name)
    if name == "single64":
        assert w.kind == synth.KIND_CONTIG and w.segments[0].key_count == 256
        assert w.logits.shape == (1, 1024)
    if name == "decode16":
        kcs = np.array([s.key_count for s in w.segments])
        assert len(kcs) == 16 and kcs.min() >= 512 and kcs.max() <= 4096
        assert w.pool_k.shape == (4096, 8, 32, 128)
        _check_paged(w)
    if name == "ring17":
        assert len(w.segments) == 17 and all(s.capacity == 4200 == s.key_count for s in w.segments)
        assert w.logits.shape == (32, 128000)
        assert w.total_rows == sum(s.n_rows for s in w.segments)
        for i, s in enumerate(w.segments):
            np.testing.assert_array_equal(synth.gather_ring(w.store_k[i], s.first, s.key_count), w.k_logical[i])


def test_workloads_are_deterministic():
    a, b = synth.make_synthetic("single64"), synth.make_synthetic("single64")
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.logits, b.logits)

"""Seeded random shapes against the float64 oracle.

Each case draws a storage kind, head dim, head counts, page size, split size,
mask and a ragged set of segments (1 to 20 rows, so the decode and the
matrix-core kernels and both head-dim-256 shapes all occur, often in one
launch), then checks the whole output against the oracle (the small-case
bound of test_gpu_parity: 2e-3 + 2^-8 |ref| + the bf16-weight term) and a
batched launch against one launch per segment, byte for byte.  The cases are
drawn from a fixed seed, so a failure names a reproducible case.
"""
import dataclasses

import numpy as np
import pytest

from oracle import oracle
from stream_paged_attention_amd import binding, launch, synth
from tests.test_gpu_parity import REL_SMALL, assert_close, weight_allowance

pytestmark = pytest.mark.gpu

N_CASES = 60
HEADS = [(8, 2), (16, 4), (16, 2), (4, 4), (32, 8), (8, 1)]


def _case(i):
    rng = np.random.Generator(np.random.PCG64(1000 + i))
    kind = ["paged", "ring", "contig"][int(rng.integers(0, 3))]
    d = [64, 128, 256][int(rng.integers(0, 3))]
    hq, hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    n_seg = int(rng.integers(1, 6))
    rows = [int(rng.integers(1, 21)) for _ in range(n_seg)]
    # keep the oracle's work per case small: keys shrink with heads and dims
    cap = max(64, 3_000_000 // (hq * d))
    keys = [int(rng.integers(r, max(r, cap) + 1)) for r in rows]
    split = [0, 32, 64, 256, 512][int(rng.integers(0, 5))]
    mask = ["causal", "causal", "full", "tree"][int(rng.integers(0, 4))]
    page = [32, 64, 256][int(rng.integers(0, 3))]
    return kind, d, hq, hkv, rows, keys, split, mask, page, int(rng.integers(0, 1 << 30))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(gpu, i):
    kind, d, hq, hkv, rows, keys, split, mask, page, seed = _case(i)
    print(f"random {i}: {kind} D{d} {hq}/{hkv} rows {rows} keys {keys} split {split} {mask} P{page}",
          flush=True)
    kw = {}
    if kind == "paged":
        kw = dict(page_size=page, pool_pages=sum(-(-k // page) for k in keys) + 3)
    elif kind == "ring":
        kw = dict(ring_slots=[k + 7 for k in keys], ring_heads=[(k * 3) % (k + 7) for k in keys])
    else:
        kw = dict(contig_capacity=[k + 1 for k in keys])
    w = synth.make_workload("random", kind, hq, hkv, d, rows, keys, seed=seed, split_keys=split, **kw)
    if mask == "tree":
        w = synth.with_trees(w, seed)
    elif mask == "full":
        w = dataclasses.replace(w, mask="full")
    dw = launch.DeviceWorkload(w, gpu)
    assert dw.check_table() == binding.TF_OK
    dw.run()
    got = dw.output()
    ref = oracle.attn_workload(w)
    assert_close(got, ref, rel=REL_SMALL, what=f"random {i}", extra=weight_allowance(w, ref))
    assert dw.error_word() == 0
    assert np.array_equal(got, dw.run_per_segment()), f"random {i}: batched differs from per-segment"


def test_many_streams_in_one_launch(gpu):
    # 256 decode streams of 1 to 2048 keys in one launch (grid size, partial
    # record offsets, the page list of every stream), against the oracle
    rng = np.random.Generator(np.random.PCG64(77))
    keys = [int(k) for k in rng.integers(1, 2049, size=256)]
    w = synth.make_workload("many", synth.KIND_PAGED, 16, 4, 128, [1] * 256, keys, seed=78,
                            page_size=32, pool_pages=sum(-(-k // 32) for k in keys) + 9, split_keys=256)
    dw = launch.DeviceWorkload(w, gpu)
    assert dw.check_table() == binding.TF_OK
    dw.run()
    ref = oracle.attn_workload(w)
    assert_close(dw.output(), ref, rel=REL_SMALL, what="many streams", extra=weight_allowance(w, ref))
    assert dw.error_word() == 0


def test_long_prompt_chunk(gpu):
    # one 1024-row prompt chunk at head dim 128 (32 query tiles per kv head,
    # causal over 1500 committed keys), against the oracle
    w = synth.make_workload("long", synth.KIND_PAGED, 16, 4, 128, [1024], [2524], seed=79,
                            page_size=64, pool_pages=45, split_keys=512)
    dw = launch.DeviceWorkload(w, gpu)
    assert dw.check_table() == binding.TF_OK
    dw.run()
    ref = oracle.attn_workload(w)
    assert_close(dw.output(), ref, rel=REL_SMALL, what="long prompt", extra=weight_allowance(w, ref))
    assert dw.error_word() == 0

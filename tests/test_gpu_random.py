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


ARGMAX_CASES = 40


def _argmax_case(i):
    """Rows, vocabulary, row stride, base shift and plants of one seeded case."""
    rng = np.random.Generator(np.random.PCG64(5000 + i))
    rows = int(rng.integers(1, 41))
    vocab = int(np.exp(rng.uniform(0.0, np.log(200_000))))
    vocab = max(1, vocab)
    pad = int(rng.integers(0, 9))          # row stride = vocab + pad
    shift = int(rng.integers(0, 2))        # 1: the buffer starts one element past 16-byte alignment
    return rows, vocab, pad, shift, int(rng.integers(0, 1 << 30))


def _argmax_rows(rows, vocab, seed):
    """Random bf16 logits with plants: ties across the kernel's chunk
    boundaries and at both ends, NaN and +-Inf, all-equal rows."""
    from tests.test_gpu_parity import ARGMAX_CHUNK
    rng = np.random.Generator(np.random.PCG64(seed))
    x = synth.normal_logits(rng, rows, vocab)
    for r in range(rows):
        kind = int(rng.integers(0, 8))
        if kind == 0 and vocab > 1:
            bounds = [b for b in range(ARGMAX_CHUNK, vocab, ARGMAX_CHUNK)]
            ids = sorted({int(rng.integers(0, vocab)), (bounds[-1] if bounds else vocab - 1)})
            synth.plant_tie(x, r, ids)
        elif kind == 1:
            synth.plant_tie(x, r, sorted({0, vocab - 1}))
        elif kind == 2:
            x[r, int(rng.integers(0, vocab))] = synth.BF16_NAN
        elif kind == 3:
            x[r, int(rng.integers(0, vocab))] = synth.BF16_POS_INF
            x[r, int(rng.integers(0, vocab))] = synth.BF16_NAN
        elif kind == 4:
            x[r, :] = synth.BF16_NEG_INF
        elif kind == 5:
            x[r, :] = synth.f32_to_bf16_bits(np.float32(rng.normal()))
    return x


@pytest.mark.parametrize("i", range(ARGMAX_CASES))
def test_random_argmax(gpu, i):
    # one launch over rows of a random vocabulary and stride, aligned or not:
    # ids and flags bit-exact against the oracle, the workspace left zero
    import torch
    rows, vocab, pad, shift, seed = _argmax_case(i)
    print(f"random argmax {i}: rows {rows} vocab {vocab} stride +{pad} shift {shift}", flush=True)
    x = _argmax_rows(rows, vocab, seed)
    rids, rflags = oracle.argmax(x)
    stride = vocab + pad
    buf = np.zeros((rows * stride + shift,), dtype=np.uint16)
    for r in range(rows):
        buf[shift + r * stride: shift + r * stride + vocab] = x[r]
    xd = launch._dev(buf, gpu)
    ids = torch.full((rows,), -7, dtype=torch.int32, device=gpu)
    flags = torch.full((rows,), 9, dtype=torch.uint8, device=gpu)
    nbytes = binding.tf_argmax_workspace_bytes(rows, vocab)
    ws = torch.zeros(max(nbytes, 8) // 8, dtype=torch.int64, device=gpu)
    st = torch.cuda.current_stream(gpu).cuda_stream
    assert binding.tf_argmax(xd.data_ptr() + 2 * shift, rows, vocab, stride, ids.data_ptr(),
                             flags.data_ptr(), ws.data_ptr(), nbytes, st) == binding.TF_OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy(), rids)
    np.testing.assert_array_equal(flags.cpu().numpy(), rflags)
    assert not ws.cpu().numpy().any(), f"random argmax {i}: workspace left dirty"


PUT_CASES = 24


def _put_workload(i):
    """A seeded round for tf_kv_put: storage kind, head dim, heads, page size,
    ring heads (wrapping or not), ragged segments of 1-20 new rows."""
    rng = np.random.Generator(np.random.PCG64(7000 + i))
    kind = ["paged", "ring", "contig"][int(rng.integers(0, 3))]
    d = [64, 128, 256][int(rng.integers(0, 3))]
    hq, hkv = HEADS[int(rng.integers(0, len(HEADS)))]
    n_seg = int(rng.integers(1, 6))
    rows = [int(rng.integers(1, 21)) for _ in range(n_seg)]
    cap = max(64, 1_500_000 // (hq * d))
    keys = [int(rng.integers(r, max(r, cap) + 1)) for r in rows]
    page = [32, 64, 128, 256, 512, 1024][int(rng.integers(0, 6))]
    seed = int(rng.integers(0, 1 << 30))
    if kind == "paged":
        kw = dict(page_size=page, pool_pages=sum(-(-k // page) for k in keys) + int(rng.integers(1, 6)))
    elif kind == "ring":
        slots = [k + int(rng.integers(0, 40)) for k in keys]
        kw = dict(ring_slots=slots, ring_heads=[int(rng.integers(0, s)) for s in slots])
    else:
        kw = dict(contig_capacity=[k + int(rng.integers(0, 40)) for k in keys])
    w = synth.make_workload(f"put{i}", kind, hq, hkv, d, rows, keys, seed=seed, split_keys=64, **kw)
    return w, page


@pytest.mark.parametrize("i", range(PUT_CASES))
def test_random_put(gpu, i):
    # the round's new rows appended by tf_kv_put: storage bit-exact against the
    # reference append, no error bit, and attention after the put byte-equal
    # to attention over the same keys placed beforehand
    from tests.kv_put_cases import oracle_after, round_inputs
    w, page = _put_workload(i)
    print(f"random put {i}: {w.kind} D{w.head_dim} {w.n_q_heads}/{w.n_kv_heads} "
          f"rows {[s.n_rows for s in w.segments]} keys {[s.key_count for s in w.segments]} P{page}", flush=True)
    before, k_new, v_new = round_inputs(w)
    dw = launch.DeviceWorkload(before, gpu)
    dw.kv_put(k_new, v_new)
    assert dw.error_word() == 0
    ek, ev = oracle_after(before, k_new, v_new)
    k, v = dw.storage()
    if w.kind == "paged":
        assert np.array_equal(k, ek) and np.array_equal(v, ev)
    else:
        assert all(np.array_equal(a, b) for a, b in zip(k, ek))
        assert all(np.array_equal(a, b) for a, b in zip(v, ev))
    dw.run()
    ref = launch.DeviceWorkload(w, gpu)
    ref.run()
    assert np.array_equal(dw.output(), ref.output()), f"random put {i}: attention after the put differs"


STATE_CASES = 16


@pytest.mark.parametrize("i", range(STATE_CASES))
def test_random_state_copy(gpu, i):
    # tf_state_save then tf_state_restore into fresh pages of the same pool:
    # every byte as the reference gives it (the pool untouched by the save,
    # the rows past `at` and the other pages untouched by the restore)
    from oracle import state_copy
    from tests.state_cases import layers_case
    rng = np.random.Generator(np.random.PCG64(9000 + i))
    layers = int(rng.integers(1, 5))
    hkv = [1, 2, 4, 8][int(rng.integers(0, 4))]
    d = [64, 128, 256][int(rng.integers(0, 3))]
    page = [32, 64, 128, 256, 512, 1024][int(rng.integers(0, 6))]
    at = int(rng.integers(1, max(2, 400_000 // (hkv * d)) + 1))
    print(f"random state {i}: {layers} layers, Hkv {hkv}, D{d}, P{page}, at {at}", flush=True)
    case = layers_case(seed=int(rng.integers(0, 1 << 30)), n_layers=layers, hkv=hkv, d=d, page_size=page, at=at)
    ds = launch.DeviceState(case.pools, case.states, case.pages, at, gpu)
    ds.save()
    pools, states = ds.host()
    ref_states = state_copy.save(case.pools, case.pages, at, case.states)
    for (gk, gv), (rk, rv) in zip(states, ref_states):
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    for (gk, gv), (rk, rv) in zip(pools, case.pools):
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    free = np.setdiff1d(np.arange(case.pool_pages), case.pages)
    new_pages = rng.choice(free, size=len(case.pages), replace=False).astype(np.int32)
    ds.set_pages(new_pages)
    ds.restore()
    pools2, _ = ds.host()
    ref_pools = state_copy.restore(ref_states, new_pages, at, case.pools)
    for (gk, gv), (rk, rv) in zip(pools2, ref_pools):
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    assert ds.error_word() == 0

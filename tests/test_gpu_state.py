"""GPU kept-state copy (tf_state_save / tf_state_restore) against the reference
in oracle/state_copy.py: bit-exact (byte work), plus the error bits and a
restore-then-attend check."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import state_copy
from stream_paged_attention_amd import binding, launch, synth
from tests.state_cases import layers_case

pytestmark = pytest.mark.gpu

CASES = [
    # layers, Hkv, D, page size, at
    (2, 2, 64, 32, 100),
    (3, 8, 128, 32, 128),        # whole pages only
    (1, 4, 256, 64, 1),          # one row
    (10, 8, 64, 512, 6243),      # ten layers, 512-position pages, a 6,243-position history
    (2, 8, 128, 1024, 1500),
]


def _fresh_pages(case, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    n = len(case.pages)
    free = np.setdiff1d(np.arange(case.pool_pages), case.pages)
    return rng.choice(free, size=n, replace=False).astype(np.int32)


@pytest.mark.parametrize("layers,hkv,d,page_size,at", CASES)
def test_save_and_restore_match_reference(gpu, layers, hkv, d, page_size, at):
    print(f"state: {layers} layers, Hkv {hkv}, D{d}, P{page_size}, at {at}", flush=True)
    case = layers_case(seed=at + d, n_layers=layers, hkv=hkv, d=d, page_size=page_size, at=at)
    ds = launch.DeviceState(case.pools, case.states, case.pages, at, gpu)
    ds.save()
    pools, states = ds.host()
    ref_states = state_copy.save(case.pools, case.pages, at, case.states)
    for (gk, gv), (rk, rv) in zip(states, ref_states):
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    for (gk, gv), (rk, rv) in zip(pools, case.pools):
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)      # save reads only
    new_pages = _fresh_pages(case, seed=at)
    ds.set_pages(new_pages)
    ds.restore()
    pools2, _ = ds.host()
    ref_pools = state_copy.restore(ref_states, new_pages, at, case.pools)
    for (gk, gv), (rk, rv) in zip(pools2, ref_pools):
        assert np.array_equal(gk, rk) and np.array_equal(gv, rv)
    assert ds.error_word() == 0


def test_bad_page_id_skips_that_page(gpu):
    case = layers_case(seed=7, n_layers=2, hkv=2, d=64, page_size=32, at=100)
    pages = case.pages.copy()
    pages[1] = 10 ** 6
    ds = launch.DeviceState(case.pools, case.states, pages, 100, gpu)
    ds.save()
    _, states = ds.host()
    assert ds.error_word() & binding.TF_ERR_BAD_PAGE
    ref = state_copy.save(case.pools, case.pages, 100, case.states)
    for (gk, _), (rk, _), (sk, _) in zip(states, ref, case.states):
        assert np.array_equal(gk[1], sk[1])                      # skipped page untouched
        assert np.array_equal(gk[[0, 2, 3]], rk[[0, 2, 3]])


def test_null_layer_pointer_skips_that_layer(gpu):
    case = layers_case(seed=8, n_layers=2, hkv=2, d=64, page_size=32, at=64)
    ds = launch.DeviceState(case.pools, case.states, case.pages, 64, gpu)
    table = ds.host_layers
    table[1].state_k = None
    raw = bytes(ctypes.string_at(ctypes.addressof(table), ctypes.sizeof(table)))
    ds.layers = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(ds.device)
    ds.save()
    _, states = ds.host()
    assert ds.error_word() & binding.TF_ERR_BAD_LAYER
    ref = state_copy.save(case.pools, case.pages, 64, case.states)
    assert np.array_equal(states[0][0], ref[0][0]) and np.array_equal(states[0][1], ref[0][1])
    assert np.array_equal(states[1][1], case.states[1][1])      # layer 1 skipped (V too)


def test_restored_stream_attends_like_the_original(gpu):
    # a stream's history saved from its pages and restored into another
    # stream's pages of an emptied pool: the next decode row reads the same keys
    at = 1000
    w1 = synth.make_workload("orig", synth.KIND_PAGED, 8, 2, 128, [1], [at], seed=31, page_size=32,
                             pool_pages=80, split_keys=256)
    w2 = synth.restore(w1, synth.KIND_PAGED, seed=77, pool_pages=80)
    d1 = launch.DeviceWorkload(w1, gpu)
    d1.run()
    out1 = d1.output()
    d2 = launch.DeviceWorkload(w2, gpu)
    d2.k_store[0][0].fill_(int(np.int16(synth.BF16_NAN.view(np.int16))))
    d2.v_store[0][0].fill_(int(np.int16(synth.BF16_NAN.view(np.int16))))
    n_state = -(-at // 32)
    sk = torch.empty((n_state, 2, 32, 128), dtype=torch.int16, device=d1.device)
    sv = torch.empty_like(sk)
    st = torch.cuda.current_stream(d1.device).cuda_stream

    def call(fn, pool_k, pool_v, pages):
        table = (binding.tf_state_layer * 1)()
        table[0].pool_k, table[0].pool_v = pool_k.data_ptr(), pool_v.data_ptr()
        table[0].state_k, table[0].state_v = sk.data_ptr(), sv.data_ptr()
        raw = bytes(ctypes.string_at(ctypes.addressof(table), ctypes.sizeof(table)))
        dev_table = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(d1.device)
        pg = torch.from_numpy(np.ascontiguousarray(pages, dtype=np.int32)).to(d1.device)
        a = binding.tf_state_args()
        a.n_layers, a.n_kv_heads, a.head_dim, a.page_size, a.pool_pages = 1, 2, 128, 32, 80
        a.at, a.n_pages, a.pages, a.layers, a.err = at, len(pages), pg.data_ptr(), dev_table.data_ptr(), d1.err.data_ptr()
        assert fn(a, st) == binding.TF_OK
        torch.cuda.synchronize(d1.device)

    call(binding.tf_state_save, d1.k_store[0][0], d1.v_store[0][0], w1.segments[0].pages)
    call(binding.tf_state_restore, d2.k_store[0][0], d2.v_store[0][0], w2.segments[0].pages)
    d2.run()
    assert np.array_equal(d2.output(), out1)
    assert d1.error_word() == 0 and d2.error_word() == 0

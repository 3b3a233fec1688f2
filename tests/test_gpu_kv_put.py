"""tf_kv_put on the GPU against the reference append (bit-exact storage)."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle
from stream_paged_attention_amd import binding, launch, synth
from tests.kv_put_cases import oracle_after, round_inputs, workloads

pytestmark = pytest.mark.gpu


def _storage_equal(dw, expect_k, expect_v):
    k, v = dw.storage()
    if dw.w.kind == "paged":
        return np.array_equal(k, expect_k) and np.array_equal(v, expect_v)
    return all(np.array_equal(a, b) for a, b in zip(k, expect_k)) and \
        all(np.array_equal(a, b) for a, b in zip(v, expect_v))


@pytest.mark.parametrize("w", workloads(), ids=lambda w: w.name)
def test_put_matches_reference(gpu, w):
    print(f"kv_put {w.name}", flush=True)
    before, k_new, v_new = round_inputs(w)
    dw = launch.DeviceWorkload(before, gpu)
    dw.kv_put(k_new, v_new)
    assert dw.error_word() == 0
    ek, ev = oracle_after(before, k_new, v_new)
    assert _storage_equal(dw, ek, ev)


@pytest.mark.parametrize("w", workloads(), ids=lambda w: w.name)
def test_put_then_attend_equals_preplaced(gpu, w):
    before, k_new, v_new = round_inputs(w)
    w2 = dataclasses.replace(w, split_keys=64)
    b2 = dataclasses.replace(before, split_keys=64)
    a = launch.DeviceWorkload(b2, gpu)
    a.kv_put(k_new, v_new)
    a.run()
    ref = launch.DeviceWorkload(w2, gpu)
    ref.run()
    assert np.array_equal(a.output(), ref.output())


def test_put_synthetic_workloads(gpu):
    # the round's rows of the decode, verify and ring drafter workloads
    for name in ("decode16", "verify8", "ring17"):
        w = synth.make_synthetic(name)
        before, k_new, v_new = round_inputs(w)
        dw = launch.DeviceWorkload(before, gpu)
        dw.kv_put(k_new, v_new)
        assert dw.error_word() == 0
        ek, ev = oracle_after(before, k_new, v_new)
        assert _storage_equal(dw, ek, ev), name


def test_put_error_bits_and_no_write(gpu):
    w = workloads()[0]
    before, k_new, v_new = round_inputs(w)
    dw = launch.DeviceWorkload(before, gpu)
    k0, v0 = dw.storage()
    hs = dw._host_segments(0)
    hs[1].capacity = 2                   # 300 keys in 2 pages of 32: past the pages
    pages = dw.pages.cpu().numpy()
    pages[int(dw.page_off[2]) + 31] = 10 ** 6   # segment 2: the page of keys 992..1023
    dw.pages.copy_(torch.from_numpy(pages).to(dw.pages.device))
    hs2 = dw._host_segments(0)
    hs2[1].capacity = 2
    dw.tables[0] = dw._upload(hs2)
    dw.kv_put(k_new, v_new)
    err = dw.error_word()
    assert err & binding.TF_ERR_PAST_PAGES and err & binding.TF_ERR_BAD_PAGE
    k1, _ = dw.storage()
    ek, _ = oracle_after(before, k_new, v_new)
    # segment 1 wrote nothing; segment 2 wrote every row but the bad page's
    s1, s2 = w.segments[1], w.segments[2]
    for j in range(s1.key_count - s1.n_rows, s1.key_count):
        page, off = s1.pages[j // 32], j % 32
        assert np.array_equal(k1[page, :, off], k0[page, :, off])
    for j in range(s2.key_count - s2.n_rows, s2.key_count):
        page, off = s2.pages[j // 32], j % 32
        if j // 32 == 31:
            continue
        assert np.array_equal(k1[page, :, off], ek[page, :, off])

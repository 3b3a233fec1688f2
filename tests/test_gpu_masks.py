"""GPU parity of the full (non-causal) and tree masks against the float64 oracle.

Same bar as the causal path: |bf16 output - float64 oracle| <= 2e-3 + 2^-8
|oracle| on these small hand-shaped cases, NaN positions identical, a batched
launch bit-equal to one launch per segment.  Shapes cover both rows kernels
(at most 4 query vectors per kv head: the VALU kernel; more: the MFMA
kernel), blocks that straddle a 32-key tile and a split boundary, blocks with
no context (key count == rows), the 64-row tree limit, and every storage kind.
"""
import dataclasses

import numpy as np
import pytest

from oracle import oracle
from stream_paged_attention_amd import binding, launch, synth
from tests.test_gpu_parity import REL_SMALL, assert_close, f32, weight_allowance

pytestmark = pytest.mark.gpu

MASK_SHAPES = [
    # kind, D, Hq, Hkv, rows, keys, split
    ("paged", 128, 4, 4, [3, 1, 4], [70, 40, 4], 64),     # VALU; block [61, 70) across split 64
    ("paged", 64, 8, 4, [2, 1], [33, 500], 32),          # VALU, G 2
    ("ring", 256, 4, 4, [4], [130], 0),                  # VALU, one split
    ("paged", 128, 16, 2, [9, 16, 5], [100, 16, 2000], 64),   # MFMA
    ("paged", 256, 16, 4, [12], [75], 32),               # MFMA D256 4-wave blocks, block across tiles and splits
    ("paged", 256, 16, 4, [24, 3], [400, 90], 64),       # MFMA D256 8-wave blocks (96 vectors)
    ("contig", 64, 8, 1, [7, 3], [300, 45], 96),         # MFMA D64
    ("ring", 128, 16, 2, [64], [4200], 512),             # the 64-row tree limit, wrapped ring
    ("paged", 128, 8, 2, [64, 1], [64, 900], 0),         # 64 rows, no context
]


def _workload(kind, d, hq, hkv, rows, keys, split, seed):
    kw = {}
    if kind == "paged":
        kw = dict(page_size=32, pool_pages=sum(-(-k // 32) for k in keys) + 5)
    elif kind == "ring":
        kw = dict(ring_slots=[k + 3 for k in keys], ring_heads=[(k * 5) % (k + 3) for k in keys])
    elif kind == "contig":
        kw = dict(contig_capacity=[k + 2 for k in keys])
    return synth.make_workload("mask", kind, hq, hkv, d, rows, keys, seed=seed, split_keys=split, **kw)


def _masked(w, mask, seed):
    if mask == "tree":
        return synth.with_trees(w, seed)
    return dataclasses.replace(w, mask=mask)


@pytest.mark.parametrize("mask", ["full", "tree"])
@pytest.mark.parametrize("kind,d,hq,hkv,rows,keys,split", MASK_SHAPES)
def test_mask_matches_oracle_and_per_segment(gpu, mask, kind, d, hq, hkv, rows, keys, split):
    print(f"{mask}: {kind} D{d} {hq}/{hkv} rows {rows} keys {keys} split {split}", flush=True)
    seed = sum(keys) + d + len(rows)
    w = _masked(_workload(kind, d, hq, hkv, rows, keys, split, seed), mask, seed)
    dw = launch.DeviceWorkload(w, gpu)
    assert dw.check_table() == binding.TF_OK
    dw.run()
    batched = dw.output()
    ref = oracle.attn_workload(w)
    assert_close(batched, ref, rel=REL_SMALL, what=f"{mask} mask", extra=weight_allowance(w, ref))
    assert dw.error_word() == 0
    assert np.array_equal(batched, dw.run_per_segment()), "batched launch differs from per-segment"


@pytest.mark.parametrize("kind,d,hq,hkv,rows,keys,split", [MASK_SHAPES[0], MASK_SHAPES[3], MASK_SHAPES[6]])
def test_chain_tree_equals_causal_bitwise(gpu, kind, d, hq, hkv, rows, keys, split):
    # a tree whose rows form one chain sees exactly the causal keys, folded
    # in the same order: the same bits
    w = _workload(kind, d, hq, hkv, rows, keys, split, seed=77)
    a = launch.DeviceWorkload(w, gpu)
    a.run()
    b = launch.DeviceWorkload(synth.with_trees(w, 0, chain=True), gpu)
    b.run()
    assert np.array_equal(a.output(), b.output())


def test_full_equals_causal_for_one_row_segments(gpu):
    w = synth.make_workload("decode", synth.KIND_PAGED, 32, 8, 128, [1] * 6,
                            [512, 700, 33, 4096, 1, 2000], seed=5, page_size=32, pool_pages=260,
                            split_keys=512)
    a = launch.DeviceWorkload(w, gpu)
    a.run()
    b = launch.DeviceWorkload(dataclasses.replace(w, mask="full"), gpu)
    b.run()
    assert np.array_equal(a.output(), b.output())


def test_full_mask_reads_the_newest_key_from_every_row(gpu):
    w = _workload("paged", 128, 16, 2, [6], [200], 64, seed=9)
    w.k_logical[0][199, 1, 7] = synth.BF16_NAN
    w = dataclasses.replace(synth.restore(w, synth.KIND_PAGED, seed=4), mask="full")
    dw = launch.DeviceWorkload(w, gpu)
    dw.run()
    got = f32(dw.output())
    ref = oracle.attn_workload(w)
    assert_close(dw.output(), ref, rel=REL_SMALL, what="full NaN", extra=weight_allowance(w, ref))
    assert np.isnan(got[:, 8:16]).all() and np.isfinite(got[:, 0:8]).all()


@pytest.mark.parametrize("hq", [4, 16])          # VALU kernel, MFMA kernel
def test_tree_never_reads_a_sibling_key(gpu, hq):
    n, kc = 4, 90
    w = _workload("paged", 128, hq, 4, [n], [kc], 32, seed=10)
    w.k_logical[0][kc - n + 2, :, 0] = synth.BF16_NAN     # row 2's key and value
    w.v_logical[0][kc - n + 2, :, :] = synth.BF16_NAN
    w = synth.restore(w, synth.KIND_PAGED, seed=4)
    w = dataclasses.replace(w, mask="tree", tree=synth.ancestor_masks([-1, 0, 0, 1]))
    dw = launch.DeviceWorkload(w, gpu)
    dw.run()
    got = f32(dw.output())
    ref = oracle.attn_workload(w)
    assert_close(dw.output(), ref, rel=REL_SMALL, what="tree NaN", extra=weight_allowance(w, ref))
    assert np.isnan(got[2]).all() and np.isfinite(got[[0, 1, 3]]).all()


def test_tree_segment_past_64_rows_sets_error(gpu):
    # the host refuses max_rows > 64 under a tree mask; a segment that still
    # holds more rows is refused by the kernels and nothing is written for it
    w = _workload("paged", 128, 8, 2, [65, 3], [200, 50], 64, seed=11)
    w = dataclasses.replace(w, mask="tree", tree=np.zeros(68, dtype=np.uint64))
    dw = launch.DeviceWorkload(w, gpu)
    a = dw.args(0)
    assert binding.tf_attn_rows(a, 0) == binding.TF_E_INVALID
    dw.out.fill_(0x1234)
    a.max_rows = 64
    st = __import__("torch").cuda.current_stream(dw.device).cuda_stream
    assert binding.tf_attn_rows(a, st) == binding.TF_OK
    assert binding.tf_attn_merge(a, st) == binding.TF_OK
    got = dw.output()
    assert dw.error_word() & binding.TF_ERR_BAD_ROWS
    assert (got[:65] == 0x1234).all()
    ref = oracle.attn([3], [50], w.q[65:], [w.k_logical[1]],
                      [w.v_logical[1]], n_q_heads=8, n_kv_heads=2, head_dim=128, scale=w.scale,
                      mask="tree", tree=np.zeros(3, dtype=np.uint64))
    v1 = np.abs(synth.bf16_bits_to_f32(w.v_logical[1]).astype(np.float64)).max(axis=0)   # [Hkv][D]
    extra = 2.0 ** -9 * (np.repeat(v1, 4, axis=0)[None] + np.abs(ref))
    assert_close(got[65:], ref, rel=REL_SMALL, what="tree segment after a refused one", extra=extra)

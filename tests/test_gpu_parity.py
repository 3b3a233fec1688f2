"""GPU parity of the HIP path against the float64 oracle, and its equalities.

Tolerance: |bf16 output - float64 oracle| <= 2e-3 for the
five synthetic workloads, NaN positions identical; argmax ids and flags
bit-exact.  Small hand-shaped cases can produce outputs of magnitude >= 0.5,
where bf16's own rounding exceeds 2e-3: half an ulp of x is between 2^-9 |x|
(top of a binade) and 2^-8 |x| (bottom of a binade).  There the bound is
2e-3 + 2^-8 |oracle| (the rounding of the stored result plus the fp32 path).
"""
import math

import numpy as np
import pytest

from oracle import oracle
from stream_paged_attention_amd import binding, launch, synth

pytestmark = pytest.mark.gpu


def f32(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def assert_close(got_bits, ref, tol=2e-3, rel=0.0, what="", extra=None):
    got = f32(got_bits)
    assert got.shape == ref.shape
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions differ ({nan_g.sum()} vs {nan_r.sum()})"
    fin = ~nan_r
    err = np.abs(got[fin] - ref[fin])
    bound = tol + rel * np.abs(ref[fin])
    if extra is not None:
        bound = bound + extra[fin]
    worst = float(np.max(err - bound)) if err.size else -1.0
    assert worst <= 0.0, f"{what}: max |err| {float(err.max()):.3e} exceeds the bound"
    return float(err.max()) if err.size else 0.0


REL_SMALL = 2.0 ** -8


def weight_allowance(w, ref):
    """Per output element, what rounding the attention weights to bf16 may
    move it: the weights enter the value products (and l) with a relative
    error of at most 2^-9 each and are normalised by the same rounded sum, so
    the output is a convex combination of the visible values with perturbed
    weights, |delta| <= 2^-9 * max_j |v_j - out| <= 2^-9 * (max_j |v_j| +
    |out|).  max_j runs over all of the segment's keys (a superset of those a
    row sees) and over finite values (nonfinite ones are handled by the NaN
    rule and compared apart).  It matters only where a row sees few keys; the
    five synthetic workloads are held to 2e-3 without it."""
    extra = np.zeros(ref.shape)
    group = w.n_q_heads // w.n_kv_heads
    for si, s in enumerate(w.segments):
        v = np.abs(synth.bf16_bits_to_f32(w.v_logical[si]).astype(np.float64))
        v = np.where(np.isfinite(v), v, 0.0)
        vmax = np.repeat(v.max(axis=0), group, axis=0)          # [Hq][D]
        rows = slice(s.row_offset, s.row_offset + s.n_rows)
        extra[rows] = 2.0 ** -9 * (vmax[None] + np.nan_to_num(np.abs(ref[rows]), posinf=0.0))
    return extra


@pytest.fixture(scope="module")
def workloads(gpu):
    cache = {}

    def get(name):
        if name not in cache:
            w = synth.make_synthetic(name)
            cache[name] = (w, launch.DeviceWorkload(w, gpu))
        return cache[name]
    return get


# --------------------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["single64", "decode16", "verify8", "prompt512", "ring17"])
def test_workload_matches_oracle(workloads, name):
    # every output element of the workload against the float64 oracle (the
    # prompt chunk's 512 x 16 x 256 outputs take the oracle ~10 s on 16 cores)
    w, dw = workloads(name)
    print(f"{name}: {synth.WORKLOAD_TITLES[name]}", flush=True)
    assert dw.check_table() == binding.TF_OK
    dw.out.fill_(0x7FA5)          # a NaN pattern no kernel writes: every element must be overwritten
    dw.run()
    got = dw.output()
    assert not np.any(got == 0x7FA5), f"{name}: output elements left unwritten"
    ref = oracle.attn_workload(w)
    assert ref.shape == got.shape
    err = assert_close(got, ref, what=name)
    assert dw.error_word() == 0
    print(f"{name}: {got.size} outputs, max |err| = {err:.3e}")


@pytest.mark.parametrize("name", ["single64", "verify8", "ring17"])
def test_workload_argmax_bit_exact(workloads, name):
    w, _ = workloads(name)
    ids, flags = launch.argmax(w.logits)
    rids, rflags = oracle.argmax(w.logits)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(flags, rflags)
    if name == "ring17":
        assert flags[4] == 1 and flags[5] == 1 and flags[:4].sum() == 0
        assert ids[0] == 0


@pytest.mark.parametrize("name", ["decode16", "verify8", "ring17"])
def test_batched_equals_per_segment(workloads, name):
    w, dw = workloads(name)
    dw.run()
    batched = dw.output()
    single = dw.run_per_segment()
    assert np.array_equal(batched, single), f"{name}: batched launch differs from per-segment"


def test_rotated_grid_batched_equals_per_segment(gpu):
    # 2 kv heads x 4 segments: the batched matrix-core launch rotates segments
    # by split, each single-segment launch does not; the bytes must agree
    keys = [5000, 300, 2100, 64]
    w = synth.make_workload("rot", synth.KIND_PAGED, 16, 2, 128, [40, 3, 17, 1], keys, seed=44,
                            page_size=32, pool_pages=sum(-(-k // 32) for k in keys) + 5, split_keys=512)
    dw = launch.DeviceWorkload(w, gpu)
    dw.run()
    batched = dw.output()
    assert np.array_equal(batched, dw.run_per_segment()), "rotated grid: batched differs from per-segment"
    assert dw.error_word() == 0


def test_prompt_and_small_d256_shapes_agree_bitwise(gpu):
    # head dim 256: a launch holding a segment of more than 64 query vectors
    # per kv head runs every segment on the prompt shape (eight waves, 128
    # vectors a workgroup); alone, the short segments take the small shape
    # (four waves).  The bytes of every segment must agree (and the long one
    # spans two query tiles).
    keys = [3000, 260, 1400, 97]
    w = synth.make_workload("wide", synth.KIND_PAGED, 16, 4, 256, [40, 3, 16, 1], keys, seed=61,
                            page_size=32, pool_pages=sum(-(-k // 32) for k in keys) + 5, split_keys=512)
    dw = launch.DeviceWorkload(w, gpu)
    dw.run()
    batched = dw.output()
    assert np.array_equal(batched, dw.run_per_segment()), "D256: prompt and small shapes differ"
    assert dw.error_word() == 0
    ref = oracle.attn_workload(w)
    assert_close(batched, ref, rel=REL_SMALL, what="D256 shapes", extra=weight_allowance(w, ref))


@pytest.mark.parametrize("name", ["decode16", "verify8", "prompt512", "ring17"])
def test_repeats_are_byte_identical(workloads, name):
    # five runs give the same bytes: the decode kernel (decode16) and the
    # matrix-core kernel with its hand-counted DMA waits (verify8, prompt512,
    # ring17); the first run's bytes are compared with each later one at once
    w, dw = workloads(name)
    first = None
    for i in range(5):
        dw.out.fill_(0x7FA5)
        dw.run()
        o = dw.output().copy()
        if first is None:
            first = o
        else:
            assert np.array_equal(o, first), f"{name}: run {i} differs from run 0"


# --------------------------------------------------------------------------- storage equalities

def _small_paged(seed=3, d=128, hq=8, hkv=2, rows=(1, 4, 2, 16), keys=(900, 97, 33, 1500),
                 split=64):
    return synth.make_workload("small", synth.KIND_PAGED, hq, hkv, d, list(rows), list(keys),
                               seed=seed, page_size=32, pool_pages=200, split_keys=split)


def test_page_permutations_are_byte_equal(gpu):
    w = _small_paged()
    a = launch.DeviceWorkload(w, gpu)
    a.run()
    b = launch.DeviceWorkload(synth.restore(w, synth.KIND_PAGED, seed=1234, pool_pages=300), gpu)
    b.run()
    assert np.array_equal(a.output(), b.output())


def test_paged_contig_ring_are_byte_equal(gpu):
    w = _small_paged(seed=5)
    outs = []
    for kind, kw in ((synth.KIND_PAGED, {}), (synth.KIND_CONTIG, dict(capacity=[1000, 200, 40, 1600])),
                     (synth.KIND_RING, dict(ring_slots=None, ring_first=[899, 50, 0, 1234]))):
        ww = synth.restore(w, kind, seed=9, **kw)
        dw = launch.DeviceWorkload(ww, gpu)
        assert dw.check_table() == binding.TF_OK
        dw.run()
        outs.append(dw.output())
    assert np.array_equal(outs[0], outs[1]), "paged != contiguous"
    assert np.array_equal(outs[0], outs[2]), "wrapped ring != contiguous"


def test_poison_outside_ranges_changes_nothing(gpu):
    w = _small_paged(seed=6)
    outs = []
    for kind, kw in ((synth.KIND_PAGED, dict(pool_pages=180)), (synth.KIND_RING, dict(ring_slots=1700)),
                     (synth.KIND_CONTIG, dict(capacity=[1024, 128, 64, 1600]))):
        pair = []
        for fill in (synth.BF16_NAN, np.uint16(0)):
            dw = launch.DeviceWorkload(synth.restore(w, kind, seed=2, fill=fill, **kw), gpu)
            dw.run()
            pair.append(dw.output())
        assert np.array_equal(pair[0], pair[1]), f"{kind}: NaN poison outside the range leaked"
        outs.append(pair[0])
    ref = oracle.attn_workload(w)
    assert_close(outs[0], ref, rel=REL_SMALL, what="poisoned paged", extra=weight_allowance(w, ref))


# --------------------------------------------------------------------------- shapes, splits, edges

SHAPES = [
    # kind, D, Hq, Hkv, rows, keys, split
    ("paged", 64, 8, 2, [1], [256], 0),
    ("paged", 64, 4, 4, [3, 1], [70, 33], 32),
    ("paged", 128, 32, 8, [1, 1, 1], [512, 513, 4096], 512),
    ("paged", 128, 16, 2, [16, 2], [4200, 17], 512),
    ("paged", 128, 8, 1, [5], [5], 32),            # every key is a new row
    ("paged", 128, 8, 8, [1], [1], 0),             # a single key
    ("paged", 256, 16, 4, [1, 7, 16], [2049, 300, 2064], 512),
    ("paged", 256, 16, 4, [9], [1000], 0),
    ("contig", 128, 16, 2, [3, 1], [777, 64], 96),
    ("ring", 128, 16, 2, [16, 1, 4], [4200, 333, 80], 512),
    ("ring", 256, 8, 2, [2], [129], 64),
    # more than 8 query vectors per kv head: the matrix-core kernel
    ("paged", 64, 8, 2, [12], [500], 128),         # D64
    ("paged", 128, 16, 2, [40, 3], [1100, 90], 256),   # 320 vectors: two query tiles (256 a tile)
    ("paged", 256, 16, 4, [40], [700], 512),       # 160 vectors: two query tiles (128 a tile)
    ("paged", 128, 16, 4, [6], [5000], 0),         # one split of 157 tiles: page ids reloaded
    ("contig", 64, 8, 2, [20], [333], 0),
    ("ring", 256, 16, 4, [5, 16], [4100, 700], 1024),
    # more than 64 splits a row: the merge reads the splits past 64 in a loop
    ("paged", 128, 32, 8, [1, 1], [131072, 3000], 512),   # a long decode context, 256 splits
    ("paged", 128, 8, 2, [1, 3], [20000, 20000], 32),    # 625 splits, both rows kernels
    ("contig", 64, 64, 1, [1], [2100], 32),              # 64 query heads on one kv head (MFMA)
    # hkv * n_segments a multiple of 8: the matrix-core grid rotates segments by split
    ("paged", 128, 16, 2, [40, 3, 17, 1], [5000, 300, 2100, 64], 512),   # 1 to 5 query tiles
    ("ring", 256, 16, 4, [33, 2], [3000, 1500], 256),
    # D256 contiguous buffers in both matrix-core shapes (at most 64 query
    # vectors per kv head: 4-wave blocks; more: 8-wave blocks)
    ("contig", 256, 16, 4, [3, 12], [900, 260], 128),
    ("contig", 256, 16, 4, [20, 1], [500, 77], 256),
]


@pytest.mark.parametrize("kind,d,hq,hkv,rows,keys,split", SHAPES)
def test_shapes_match_oracle(gpu, kind, d, hq, hkv, rows, keys, split):
    print(f"shape {kind} D{d} {hq}/{hkv} rows {rows} keys {keys} split {split}", flush=True)
    kw = {}
    if kind == "paged":
        kw = dict(page_size=32, pool_pages=sum(-(-k // 32) for k in keys) + 7)
    elif kind == "ring":
        kw = dict(ring_slots=[k + 5 for k in keys], ring_heads=[(k * 7) % (k + 5) for k in keys])
    elif kind == "contig":
        kw = dict(contig_capacity=[k + 3 for k in keys])
    w = synth.make_workload("shape", kind, hq, hkv, d, rows, keys, seed=sum(keys) + d,
                            split_keys=split, **kw)
    dw = launch.DeviceWorkload(w, gpu)
    assert dw.check_table() == binding.TF_OK
    dw.run()
    ref = oracle.attn_workload(w)
    assert_close(dw.output(), ref, rel=REL_SMALL, what="shape", extra=weight_allowance(w, ref))
    assert dw.error_word() == 0


PAGE_SHAPES = [
    # Hq, Hkv, D, rows, keys, split: decode (VALU) and prompt chunks (MFMA)
    (8, 2, 128, [1, 3], [1000, 257], 256),
    (8, 2, 128, [1, 1], [2100, 513], 512),
    (8, 2, 64, [64], [1500], 512),          # D64 prompt chunk
    (16, 2, 128, [128, 2], [3000, 700], 1024),   # D128 prompt chunk and a short verify
    (16, 4, 256, [1, 24], [1200, 2500], 512),
    (16, 4, 256, [3, 16], [900, 2100], 512),     # D256 verify (4-wave blocks)
]


@pytest.mark.parametrize("page_size", [64, 256, 512, 1024])
@pytest.mark.parametrize("hq,hkv,d,rows,keys,split", PAGE_SHAPES)
def test_other_page_sizes(gpu, page_size, hq, hkv, d, rows, keys, split):
    print(f"P{page_size} D{d} {hq}/{hkv} rows {rows} keys {keys} split {split}", flush=True)
    pool = sum(-(-k // page_size) for k in keys) + 3
    w = synth.make_workload("pages", synth.KIND_PAGED, hq, hkv, d, rows, keys, seed=8 + d,
                            page_size=page_size, pool_pages=pool, split_keys=split)
    dw = launch.DeviceWorkload(w, gpu)
    assert dw.check_table() == binding.TF_OK
    dw.run()
    ref = oracle.attn_workload(w)
    assert_close(dw.output(), ref, rel=REL_SMALL, what=f"P{page_size}", extra=weight_allowance(w, ref))
    assert dw.error_word() == 0


def test_different_split_sizes_agree_within_tolerance(gpu):
    w = _small_paged(seed=12)
    ref = oracle.attn_workload(w)
    for split in (0, 32, 128, 512):
        dw = launch.DeviceWorkload(w, gpu, split_keys=split)
        dw.run()
        assert_close(dw.output(), ref, rel=REL_SMALL, what=f"split {split}", extra=weight_allowance(w, ref))


def test_partial_records_match_oracle_partials(gpu):
    # m is a reference and l, o are relative to it: the log-sum-exp and o / l
    # are what a record fixes.  The value products take the weights rounded
    # to bf16 (relative error <= 2^-9 each, sums in fp32), so o / l may differ
    # from the float64 result by at most 2^-9 * max |v| over the split's keys
    # (a weighted mean of per-key errors 2^-9 p_j |v_jd| / l); the test allows
    # that plus 1e-5.  Where l sums the rounded weights, the log-sum-exp moves
    # by at most -log(1 - 2^-9).
    split = 64
    w = synth.make_workload("parts", synth.KIND_PAGED, 8, 2, 128, [3, 1], [200, 130], seed=14,
                            page_size=32, pool_pages=20, split_keys=split)
    dw = launch.DeviceWorkload(w, gpu)
    dw.run()
    recs = dw.partial_records()
    m, l, o = oracle.attn_partials([s.n_rows for s in w.segments], [s.key_count for s in w.segments],
                                   w.q, w.k_logical, w.v_logical, n_q_heads=8, n_kv_heads=2,
                                   head_dim=128, scale=w.scale, split=split)
    row = 0
    for seg in w.segments:
        ns = -(-seg.key_count // split)
        for r in range(seg.n_rows):
            for h in range(8):
                for t in range(ns):
                    rec = recs[dw.host_segs[w.segments.index(seg)].partial_offset + (r * 8 + h) * ns + t]
                    mr, lr, orr = m[row, h, t], l[row, h, t], o[row, h, t]
                    if mr == -np.inf:
                        assert rec[0] == -np.inf and rec[1] == 0 and not np.any(rec[4:])
                        continue
                    # m is a reference: one of the split's scaled scores, at most
                    # 8 ln 2 below their max; the log-sum-exp and o / l are fixed
                    assert mr - 8 * np.log(2) - 1e-5 <= rec[0] <= mr + 1e-5 * max(1.0, abs(mr))
                    lse_g, lse_r = rec[0] + np.log(rec[1]), mr + np.log(lr)
                    # l may be the sum of the bf16-rounded weights (the matrix-core
                    # kernel): |log l - log sum p| <= -log(1 - 2^-9)
                    assert abs(lse_g - lse_r) <= 1e-5 * max(1.0, abs(lse_r)) - np.log1p(-2.0 ** -9)
                    si = w.segments.index(seg)
                    vk = synth.bf16_bits_to_f32(w.v_logical[si][t * split:(t + 1) * split, h // 4]).astype(np.float64)
                    bound = 1e-5 + 2.0 ** -9 * np.max(np.abs(vk), axis=0)
                    assert np.all(np.abs(rec[4:] / rec[1] - orr / lr) <= bound)
            row += 1


# --------------------------------------------------------------------------- NaN rule

def _nan_case(gpu, plant):
    w = synth.make_workload("nan", synth.KIND_PAGED, 8, 2, 128, [4, 1], [300, 70], seed=21,
                            page_size=32, pool_pages=20, split_keys=64)
    plant(w)
    w2 = synth.restore(w, synth.KIND_PAGED, seed=3)
    dw = launch.DeviceWorkload(w2, gpu)
    dw.run()
    got, ref = dw.output(), oracle.attn_workload(w2)
    assert_close(got, ref, rel=REL_SMALL, what="nan rule", extra=weight_allowance(w2, ref))
    return f32(got)


def test_nan_key_poisons_its_group(gpu):
    def plant(w):
        w.k_logical[0][100, 1, 5] = synth.BF16_NAN
    got = _nan_case(gpu, plant)
    assert np.isnan(got[0:4, 4:8]).all() and np.isfinite(got[0:4, 0:4]).all()


def test_nan_value_poisons_one_lane(gpu):
    def plant(w):
        w.v_logical[0][10, 0, 77] = synth.BF16_POS_INF
    got = _nan_case(gpu, plant)
    assert np.isnan(got[0:4, 0:4, 77]).all()
    assert np.isfinite(got[0:4, 0:4, :77]).all()


@pytest.mark.parametrize("d,hq,hkv,rows,dim,other", [
    # D256 launches of at most 64 query vectors per kv head: 4-wave blocks
    (256, 16, 4, 2, 200, 0),    # 8 query vectors: four waves split the 16 dim blocks (four each)
    (256, 16, 4, 7, 37, 0),     # 28 vectors: two waves a block
    # beside an 80-vector segment the launch takes 8-wave blocks
    (256, 16, 4, 2, 200, 20),   # eight waves split the dims (two each)
    (256, 16, 4, 7, 37, 20),    # four waves a block
    (64, 8, 2, 5, 61, 0),       # D64, 20 vectors: two waves a block
])
def test_nan_value_reaches_its_lane_when_waves_split_dims(gpu, d, hq, hkv, rows, dim, other):
    # a nonfinite value at a visible key poisons exactly its output lane,
    # whichever wave of the block owns that dim (matrix-core kernel)
    keys = 300
    seg_rows = [rows] + ([other] if other else [])
    w = synth.make_workload("nansplit", synth.KIND_PAGED, hq, hkv, d, seg_rows, [keys] * len(seg_rows),
                            seed=23 + d + other, page_size=32, pool_pages=40, split_keys=64)
    w.v_logical[0][keys - rows - 5, 0, dim] = synth.BF16_POS_INF       # seen by every row
    w.v_logical[0][keys - 1, 1 % hkv, dim - 1] = synth.BF16_NAN        # seen by the last row only
    w2 = synth.restore(w, synth.KIND_PAGED, seed=4)
    dw = launch.DeviceWorkload(w2, gpu)
    dw.run()
    got, ref = dw.output(), oracle.attn_workload(w2)
    assert_close(got, ref, rel=REL_SMALL, what="nan split dims", extra=weight_allowance(w2, ref))
    g = f32(got)[:rows]       # the first segment's rows
    group = hq // hkv
    assert np.isnan(g[:, 0:group, dim]).all()
    assert np.isfinite(np.delete(g[:, 0:group, :], dim, axis=2)).all()
    kv1 = (1 % hkv) * group
    assert np.isnan(g[rows - 1, kv1:kv1 + group, dim - 1]).all()
    if rows > 1 and kv1 != 0:
        assert np.isfinite(g[:rows - 1, kv1:kv1 + group, dim - 1]).all()
    if other:
        assert np.isfinite(f32(got)[rows:]).all()


def test_nan_in_newest_key_reaches_only_last_row(gpu):
    def plant(w):
        w.k_logical[0][299, :, 3] = synth.BF16_NAN
        w.v_logical[0][299, :, :] = synth.BF16_NAN
    got = _nan_case(gpu, plant)
    assert np.isnan(got[3]).all() and np.isfinite(got[0:3]).all() and np.isfinite(got[4]).all()


# --------------------------------------------------------------------------- device error word

def test_bad_page_id_sets_error_and_nan(gpu):
    w = _small_paged(seed=30)
    dw = launch.DeviceWorkload(w, gpu)
    pages = dw.pages.cpu().numpy()
    pages[int(dw.page_off[1]) + 1] = 10 ** 6          # segment 1, second page
    dw.pages.copy_(__import__("torch").from_numpy(pages).to(dw.pages.device))
    dw.run()
    got = f32(dw.output())
    assert dw.error_word() & binding.TF_ERR_BAD_PAGE
    s1 = w.segments[1]
    assert np.isnan(got[s1.row_offset:s1.row_offset + s1.n_rows]).all()
    s0 = w.segments[0]
    assert np.isfinite(got[s0.row_offset:s0.row_offset + s0.n_rows]).all()


def test_key_count_past_pages_sets_error(gpu):
    import ctypes
    import torch
    w = _small_paged(seed=31)
    dw = launch.DeviceWorkload(w, gpu)
    hs = dw._host_segments(0)
    for i in range(len(hs)):
        hs[i].partial_offset = dw.host_segs[i].partial_offset
    hs[2].capacity = 1                                   # 33 keys in one page of 32
    dw.tables[0] = dw._upload(hs)
    assert binding.tf_check_segments(dw.args(0), hs) == binding.TF_E_PAST_PAGES
    dw.run()
    got = f32(dw.output())
    assert dw.error_word() & binding.TF_ERR_PAST_PAGES
    s2 = w.segments[2]
    assert np.isnan(got[s2.row_offset:s2.row_offset + s2.n_rows]).all()
    assert np.isfinite(got[:s2.row_offset]).all()


def test_segment_past_the_hints_sets_error_and_nan(gpu):
    # key_count above max_keys (decode segments) and n_rows above max_rows
    # (a matrix-core segment): the grid does not cover them; the rows it
    # covers are NaN, rows past max_rows are not written, the others are fine
    w = synth.make_workload("hints", synth.KIND_PAGED, 8, 2, 128, [1, 20, 1], [700, 900, 1500], seed=33,
                            page_size=32, pool_pages=120, split_keys=256)
    ref = oracle.attn_workload(w)
    dw = launch.DeviceWorkload(w, gpu)
    a = dw.args(0)
    a.max_keys = 1400        # segment 2 holds 1500 keys
    a.max_rows = 12          # segment 1 has 20 rows
    a.min_rows = 0
    dw.out.fill_(0x7FA5)
    st = __import__("torch").cuda.current_stream(gpu).cuda_stream
    assert binding.tf_attn_rows(a, st) == binding.TF_OK
    assert binding.tf_attn_merge(a, st) == binding.TF_OK
    got = dw.output()
    assert dw.error_word() == binding.TF_ERR_HINTS
    s0, s1, s2 = w.segments
    assert_close(got[s0.row_offset:s0.row_offset + 1], ref[s0.row_offset:s0.row_offset + 1], what="in-bounds segment")
    assert np.isnan(f32(got[s2.row_offset])).all()
    assert np.isnan(f32(got[s1.row_offset:s1.row_offset + 12])).all()
    assert np.all(got[s1.row_offset + 12:s1.row_offset + 20] == 0x7FA5), "rows past max_rows were written"


@pytest.mark.parametrize("kind", ["contig", "ring"])
def test_buffer_past_32bit_offsets_sets_error(gpu, kind):
    # one kv head's run of 2^23 keys x D 256 x 2 bytes = 4 GiB: the kernels'
    # 32-bit offsets cannot address it, so the segment is refused on the
    # device (no key is read) and its rows are NaN.  The buffers are really
    # that large, so no access could leave them either way.
    import torch
    cap = 1 << 23
    w = synth.make_workload("big", synth.KIND_CONTIG, 4, 1, 256, [1], [64], seed=34, split_keys=0,
                            contig_capacity=[80])
    k = torch.zeros(cap * 256, dtype=torch.int16, device=gpu)
    v = torch.zeros(cap * 256, dtype=torch.int16, device=gpu)
    q = launch._dev(w.q, gpu)
    out = torch.full((1, 4, 256), 0x7FA5, dtype=torch.int16, device=gpu)
    err = torch.zeros(1, dtype=torch.int32, device=gpu)
    seg = (binding.tf_segment * 1)()
    seg[0].k, seg[0].v, seg[0].pages = k.data_ptr(), v.data_ptr(), None
    seg[0].capacity, seg[0].first, seg[0].row_offset, seg[0].n_rows, seg[0].key_count = cap, 0, 0, 1, 64
    seg[0].partial_offset = 0
    table = torch.frombuffer(bytearray(bytes(__import__("ctypes").string_at(
        __import__("ctypes").addressof(seg), __import__("ctypes").sizeof(seg)))), dtype=torch.uint8).to(gpu)
    a = binding.tf_attn_args()
    a.kind = binding.KIND_CODE[kind]
    a.n_segments, a.total_rows, a.max_rows, a.max_keys, a.min_rows = 1, 1, 1, 64, 1
    a.n_q_heads, a.n_kv_heads, a.head_dim, a.page_size, a.pool_pages = 4, 1, 256, 0, 0
    a.split_keys, a.scale, a.mask = 0, w.scale, binding.TF_MASK_CAUSAL
    a.segs, a.tree, a.q, a.out = table.data_ptr(), None, q.data_ptr(), out.data_ptr()
    a.partials, a.partials_bytes, a.err = None, 0, err.data_ptr()
    assert binding.tf_check_segments(a, seg) == binding.TF_E_UNSUPPORTED
    assert binding.tf_attn_rows(a, torch.cuda.current_stream(gpu).cuda_stream) == binding.TF_OK
    torch.cuda.synchronize()
    assert int(err.item()) & binding.TF_ERR_STORAGE
    assert np.isnan(f32(launch.to_host_u16(out))).all()


def test_argmax_small_cases(gpu):
    from tests import pins
    x = pins.argmax_rows(seed=40, rows=12, vocab=9000)
    ids, flags = launch.argmax(x)
    rids, rflags = oracle.argmax(x)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(flags, rflags)
    # a row stride wider than the vocabulary, with a larger value past the end
    wide = np.full((12, 9008), synth.f32_to_bf16_bits(np.float32(50.0)), dtype=np.uint16)
    wide[:, :9001] = np.concatenate([x, x[:, :1]], axis=1)
    ids2, flags2 = launch.argmax(wide, vocab=9001)
    rids2, rflags2 = oracle.argmax(wide, vocab=9001)
    np.testing.assert_array_equal(ids2, rids2)
    np.testing.assert_array_equal(flags2, rflags2)


def test_argmax_scalar_loads(gpu):
    # rows whose base is not 16-byte aligned (an odd row stride, or the whole
    # buffer shifted by one element) take the element-by-element loads;
    # several chunks a row, ties across the chunk boundary, nonfinite rows
    import torch
    vocab = 2 * 16384 + 77
    x = _vocab_edge_rows(vocab, seed=71)
    rids, rflags = oracle.argmax(x)
    st = torch.cuda.current_stream(gpu).cuda_stream
    rows = x.shape[0]
    for stride, shift in ((vocab + 3, 0), (vocab, 1)):
        buf = np.zeros((rows * stride + shift,), dtype=np.uint16)
        for r in range(rows):
            buf[shift + r * stride: shift + r * stride + vocab] = x[r]
        xd = launch._dev(buf, gpu)
        ids = torch.full((rows,), -1, dtype=torch.int32, device=gpu)
        flags = torch.full((rows,), 7, dtype=torch.uint8, device=gpu)
        nbytes = binding.tf_argmax_workspace_bytes(rows, vocab)
        ws = torch.zeros(nbytes // 8, dtype=torch.int64, device=gpu)
        assert binding.tf_argmax(xd.data_ptr() + 2 * shift, rows, vocab, stride, ids.data_ptr(),
                                 flags.data_ptr(), ws.data_ptr(), nbytes, st) == binding.TF_OK
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids.cpu().numpy(), rids)
        np.testing.assert_array_equal(flags.cpu().numpy(), rflags)


ARGMAX_CHUNK = 16384   # logits a workgroup of the argmax kernel reduces


def _vocab_edge_rows(vocab, seed):
    """Rows for one vocabulary size: random, ties at both ends, across the
    kernel's chunk boundary and at the last chunk's first id, all equal,
    all NaN, and a +inf after a NaN."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = synth.normal_logits(rng, 8, vocab)
    synth.plant_tie(x, 1, sorted({0, vocab - 1}))
    if vocab > ARGMAX_CHUNK:
        synth.plant_tie(x, 2, [ARGMAX_CHUNK - 1, ARGMAX_CHUNK])
        last = (vocab - 1) // ARGMAX_CHUNK * ARGMAX_CHUNK
        synth.plant_tie(x, 3, sorted({5, last}))
    else:
        synth.plant_tie(x, 2, sorted({vocab // 2, vocab - 1}))
    x[4, :] = synth.f32_to_bf16_bits(np.float32(-3.0))
    x[5, :] = synth.BF16_NAN
    x[6, 0] = synth.BF16_NAN
    x[6, vocab - 1] = synth.BF16_POS_INF
    x[7, :] = synth.BF16_NEG_INF
    return x


def test_argmax_reuses_its_workspace(gpu):
    # one zeroed workspace serves call after call: each leaves it zero, and
    # the ids and flags stay bit-exact across rows of different lengths,
    # nonfinite rows and ties across the argmax chunks
    import torch
    rows, vocab = 40, 128000
    x = _vocab_edge_rows(vocab, seed=61)
    rng = np.random.Generator(np.random.PCG64(62))
    x = np.concatenate([x, synth.normal_logits(rng, rows - x.shape[0], vocab)])
    rids, rflags = oracle.argmax(x)
    dev = gpu
    xd = launch._dev(x, dev)
    nbytes = binding.tf_argmax_workspace_bytes(rows, vocab)
    ws = torch.zeros(nbytes // 8, dtype=torch.int64, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    for it in range(4):
        ids = torch.full((rows,), -1, dtype=torch.int32, device=dev)
        flags = torch.full((rows,), 7, dtype=torch.uint8, device=dev)
        n = rows if it % 2 == 0 else rows // 2          # fewer rows on odd calls
        assert binding.tf_argmax(xd.data_ptr(), n, vocab, vocab, ids.data_ptr(), flags.data_ptr(),
                                 ws.data_ptr(), nbytes, st) == binding.TF_OK
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids.cpu().numpy()[:n], rids[:n])
        np.testing.assert_array_equal(flags.cpu().numpy()[:n], rflags[:n])
        assert not ws.cpu().numpy().any(), f"call {it} left the workspace dirty"


@pytest.mark.parametrize("vocab", [1, 2, 7, 64, 255, 256, 257, 8191, 8192, 8193, 16383, 16384, 16385,
                                   24577, 40961])
def test_argmax_vocab_edges(gpu, vocab):
    print(f"argmax vocab {vocab}", flush=True)
    x = _vocab_edge_rows(vocab, seed=vocab)
    ids, flags = launch.argmax(x)
    rids, rflags = oracle.argmax(x)
    np.testing.assert_array_equal(ids, rids)
    np.testing.assert_array_equal(flags, rflags)

"""Pins of the float64 oracle to references other than itself (CPU only)."""
import math

import numpy as np
import pytest

from oracle import oracle
from stream_paged_attention_amd import synth
from tests import pins


def test_matches_torch_sdpa_float64():
    # GQA head mapping, scale, causal count, max subtraction, P.V: all of it
    # against torch's own float64 attention.
    assert pins.check_attention(oracle.attn) <= 1e-12


@pytest.mark.parametrize("seed,h,d,n,kc", [(21, 3, 4, 1, 9), (22, 2, 16, 4, 30), (23, 1, 3, 3, 3)])
def test_matches_textbook_mha(seed, h, d, n, kc):
    n_rows, kcs, q, kl, vl = pins.random_case(seed, h, h, d, [(n, kc)])
    got = oracle.attn(n_rows, kcs, q, kl, vl, n_q_heads=h, n_kv_heads=h, head_dim=d,
                      scale=1 / math.sqrt(d))
    ref = pins.textbook_mha(n, kc, q, kl[0], vl[0], d)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def _one(q, k, v, hq=2, hkv=1, d=4, n=1):
    kc = k.shape[0]
    return oracle.attn([n], [kc], q, [k], [v], n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                       scale=1 / math.sqrt(d))


def test_closed_form_single_key_returns_v():
    _, _, q, kl, vl = pins.random_case(31, 2, 1, 4, [(1, 1)])
    out = _one(q, kl[0], vl[0])
    np.testing.assert_array_equal(out[0, 0], pins.f64(vl[0][0, 0]))
    np.testing.assert_array_equal(out[0, 1], pins.f64(vl[0][0, 0]))


def test_closed_form_identical_keys_give_mean_v():
    _, _, q, kl, vl = pins.random_case(32, 2, 1, 4, [(1, 37)])
    k = np.repeat(kl[0][:1], 37, axis=0)
    out = _one(q, k, vl[0])
    np.testing.assert_allclose(out[0, 0], pins.f64(vl[0][:, 0]).mean(axis=0), rtol=0, atol=1e-14)


def test_closed_form_constant_v():
    _, _, q, kl, _ = pins.random_case(33, 2, 1, 4, [(1, 50)])
    v = np.full((50, 1, 4), synth.f32_to_bf16_bits(np.float32(0.375)), dtype=np.uint16)
    out = _one(q, kl[0], v)
    np.testing.assert_allclose(out, 0.375, rtol=1e-15, atol=0)


def test_closed_form_zero_query_is_uniform_over_visible_keys():
    n, kc = 3, 10
    _, _, q, kl, vl = pins.random_case(34, 2, 1, 4, [(n, kc)])
    q[:] = 0
    out = _one(q, kl[0], vl[0], n=n)
    vv = pins.f64(vl[0][:, 0])
    for r in range(n):
        vis = kc - n + r + 1
        np.testing.assert_allclose(out[r, 0], vv[:vis].mean(axis=0), rtol=0, atol=1e-14)


def test_gqa_equals_mha_with_duplicated_kv_heads():
    hq, hkv, d = 8, 2, 8
    n_rows, kcs, q, kl, vl = pins.random_case(35, hq, hkv, d, [(2, 19), (1, 4)])
    g = hq // hkv
    kd = [np.repeat(k, g, axis=1) for k in kl]
    vd = [np.repeat(v, g, axis=1) for v in vl]
    a = oracle.attn(n_rows, kcs, q, kl, vl, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                    scale=1 / math.sqrt(d))
    b = oracle.attn(n_rows, kcs, q, kd, vd, n_q_heads=hq, n_kv_heads=hq, head_dim=d,
                    scale=1 / math.sqrt(d))
    np.testing.assert_array_equal(a, b)


def test_causal_rows_equal_one_row_segments():
    hq, hkv, d, n, kc = 4, 2, 8, 5, 23
    n_rows, kcs, q, kl, vl = pins.random_case(36, hq, hkv, d, [(n, kc)])
    a = oracle.attn(n_rows, kcs, q, kl, vl, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                    scale=1 / math.sqrt(d))
    vis = [kc - n + r + 1 for r in range(n)]
    b = oracle.attn([1] * n, vis, q, [kl[0][:v] for v in vis], [vl[0][:v] for v in vis],
                    n_q_heads=hq, n_kv_heads=hkv, head_dim=d, scale=1 / math.sqrt(d))
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("split", [1, 7, 32, 512])
def test_split_and_merge_equal_unsplit(split):
    hq, hkv, d = 4, 2, 8
    segs = [(1, 700), (3, 65), (2, 2), (4, 513)]
    n_rows, kcs, q, kl, vl = pins.random_case(37, hq, hkv, d, segs)
    kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, scale=1 / math.sqrt(d))
    full = oracle.attn(n_rows, kcs, q, kl, vl, **kw)
    m, l, o = oracle.attn_partials(n_rows, kcs, q, kl, vl, split=split, **kw)
    np.testing.assert_allclose(oracle.merge(m, l, o), full, rtol=0, atol=1e-12)
    # split t of a row is empty exactly when it starts at or past the row's causal limit
    row = 0
    for n, kc in segs:
        for r in range(n):
            vis = kc - n + r + 1
            for t in range(m.shape[2]):
                assert (m[row, :, t] == -np.inf).all() == (t * split >= vis)
            row += 1


def test_partials_hold_the_split_max_and_sums():
    hq, hkv, d, split = 2, 1, 4, 16
    n_rows, kcs, q, kl, vl = pins.random_case(38, hq, hkv, d, [(1, 40)])
    m, l, o = oracle.attn_partials(n_rows, kcs, q, kl, vl, n_q_heads=hq, n_kv_heads=hkv,
                                   head_dim=d, scale=0.5, split=split)
    qq, kk, vv = pins.f64(q[0, 0]), pins.f64(kl[0][:, 0]), pins.f64(vl[0][:, 0])
    s = kk @ qq * 0.5
    for t in range(3):
        st = s[t * split:(t + 1) * split]
        assert m[0, 0, t] == pytest.approx(st.max(), abs=1e-13)
        p = np.exp(st - st.max())
        assert l[0, 0, t] == pytest.approx(p.sum(), abs=1e-12)
        np.testing.assert_allclose(o[0, 0, t], p @ vv[t * split:(t + 1) * split], atol=1e-12)


# --------------------------------------------------------------------------- full and tree masks

def test_full_mask_matches_torch_sdpa_float64():
    # FULL: every row of a block sees every key of its stream.
    assert pins.check_attention(oracle.attn, pins.SDPA_CASES + pins.MASK_CASES, mask="full") <= 1e-12


def test_tree_mask_matches_torch_sdpa_float64():
    # tree: context, the row's own key and its ancestors' keys.
    assert pins.check_attention(oracle.attn, pins.SDPA_CASES + pins.MASK_CASES, mask="tree") <= 1e-12


def test_full_rows_equal_one_row_segments_over_all_keys():
    hq, hkv, d, n, kc = 4, 2, 8, 6, 19
    n_rows, kcs, q, kl, vl = pins.random_case(41, hq, hkv, d, [(n, kc)])
    kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, scale=1 / math.sqrt(d))
    a = oracle.attn(n_rows, kcs, q, kl, vl, mask="full", **kw)
    b = oracle.attn([1] * n, [kc] * n, q, kl * n, vl * n, **kw)
    np.testing.assert_array_equal(a, b)


def test_full_mask_ignores_key_order():
    hq, hkv, d, n, kc = 4, 2, 8, 5, 31
    n_rows, kcs, q, kl, vl = pins.random_case(42, hq, hkv, d, [(n, kc)])
    perm = np.random.Generator(np.random.PCG64(42)).permutation(kc)
    kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, scale=1 / math.sqrt(d), mask="full")
    a = oracle.attn(n_rows, kcs, q, kl, vl, **kw)
    b = oracle.attn(n_rows, kcs, q, [kl[0][perm]], [vl[0][perm]], **kw)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_chain_tree_equals_causal():
    # A tree whose rows form one chain is the causal count.
    hq, hkv, d = 4, 2, 8
    segs = [(7, 30), (1, 5), (3, 3)]
    n_rows, kcs, q, kl, vl = pins.random_case(43, hq, hkv, d, segs)
    kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, scale=1 / math.sqrt(d))
    tree = np.concatenate([synth.ancestor_masks(np.arange(-1, n - 1)) for n in n_rows])
    a = oracle.attn(n_rows, kcs, q, kl, vl, mask="tree", tree=tree, **kw)
    b = oracle.attn(n_rows, kcs, q, kl, vl, **kw)
    np.testing.assert_array_equal(a, b)


def test_tree_node_equals_its_chain():
    # Each node equals the last row of a causal segment holding the context,
    # its ancestors and itself, in key order.
    hq, hkv, d, n, kc = 4, 2, 8, 12, 40
    n_rows, kcs, q, kl, vl = pins.random_case(44, hq, hkv, d, [(n, kc)])
    par = synth.random_parents(np.random.Generator(np.random.PCG64(44)), n)
    kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, scale=1 / math.sqrt(d))
    a = oracle.attn(n_rows, kcs, q, kl, vl, mask="tree", tree=synth.ancestor_masks(par), **kw)
    for r in range(n):
        path, x = [], r
        while x >= 0:
            path.append(x)
            x = int(par[x])
        keys = list(range(kc - n)) + [kc - n + x for x in sorted(path)]
        b = oracle.attn([1], [len(keys)], q[r:r + 1], [kl[0][keys]], [vl[0][keys]], **kw)
        np.testing.assert_array_equal(a[r], b[0])


@pytest.mark.parametrize("mask", ["full", "tree"])
def test_masked_split_and_merge_equal_unsplit(mask):
    hq, hkv, d, split = 4, 2, 8, 5
    segs = [(9, 40), (4, 4), (1, 13)]
    n_rows, kcs, q, kl, vl = pins.random_case(45, hq, hkv, d, segs)
    kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, scale=1 / math.sqrt(d), mask=mask)
    if mask == "tree":
        rng = np.random.Generator(np.random.PCG64(45))
        kw["tree"] = np.concatenate([synth.ancestor_masks(synth.random_parents(rng, n))
                                     for n in n_rows])
    full = oracle.attn(n_rows, kcs, q, kl, vl, **kw)
    m, l, o = oracle.attn_partials(n_rows, kcs, q, kl, vl, split=split, **kw)
    np.testing.assert_allclose(oracle.merge(m, l, o), full, rtol=0, atol=1e-12)


def test_full_mask_reads_keys_past_the_causal_limit():
    hq, hkv, d, n, kc = 4, 2, 8, 3, 12
    n_rows, kcs, q, kl, vl = pins.random_case(46, hq, hkv, d, [(n, kc)])
    kl[0][kc - 1, :, 0] = synth.BF16_NAN
    out = oracle.attn(n_rows, kcs, q, kl, vl, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                      scale=1 / math.sqrt(d), mask="full")
    assert np.isnan(out).all()


def test_tree_never_reads_a_sibling_key():
    hq, hkv, d, n, kc = 4, 2, 8, 4, 10
    n_rows, kcs, q, kl, vl = pins.random_case(47, hq, hkv, d, [(n, kc)])
    par = np.array([-1, 0, 0, 1])        # rows 1 and 2 are siblings; 3 under 1
    kl[0][kc - n + 2] = synth.BF16_NAN   # row 2's key
    vl[0][kc - n + 2] = synth.BF16_NAN
    out = oracle.attn(n_rows, kcs, q, kl, vl, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                      scale=1 / math.sqrt(d), mask="tree", tree=synth.ancestor_masks(par))
    assert np.isnan(out[2]).all()
    assert np.isfinite(out[[0, 1, 3]]).all()


# --------------------------------------------------------------------------- NaN rule

def _nan_case():
    hq, hkv, d, n, kc = 4, 2, 8, 3, 12
    return (hq, hkv, d, n, kc) + pins.random_case(39, hq, hkv, d, [(n, kc)])


def _run(hq, hkv, d, n_rows, kcs, q, kl, vl):
    return oracle.attn(n_rows, kcs, q, kl, vl, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                       scale=1 / math.sqrt(d))


def test_nan_in_visible_key_poisons_its_group_only():
    hq, hkv, d, n, kc, n_rows, kcs, q, kl, vl = _nan_case()
    kl[0][2, 1, 3] = synth.BF16_NAN
    out = _run(hq, hkv, d, n_rows, kcs, q, kl, vl)
    assert np.isnan(out[:, 2:4]).all()          # heads 2, 3 read kv head 1
    assert np.isfinite(out[:, 0:2]).all()


def test_inf_in_query_gives_nan_row_head():
    hq, hkv, d, n, kc, n_rows, kcs, q, kl, vl = _nan_case()
    q[1, 0, 5] = synth.BF16_POS_INF
    out = _run(hq, hkv, d, n_rows, kcs, q, kl, vl)
    assert np.isnan(out[1, 0]).all()
    mask = np.ones(out.shape[:2], bool)
    mask[1, 0] = False
    assert np.isfinite(out[mask]).all()


def test_nan_in_newest_key_reaches_only_the_last_row():
    hq, hkv, d, n, kc, n_rows, kcs, q, kl, vl = _nan_case()
    kl[0][kc - 1, :, 0] = synth.BF16_NAN
    vl[0][kc - 1, :, :] = synth.BF16_NAN
    out = _run(hq, hkv, d, n_rows, kcs, q, kl, vl)
    assert np.isnan(out[n - 1]).all()
    assert np.isfinite(out[:n - 1]).all()


def test_nonfinite_value_poisons_only_its_lane():
    hq, hkv, d, n, kc, n_rows, kcs, q, kl, vl = _nan_case()
    vl[0][4, 0, 6] = synth.BF16_POS_INF
    out = _run(hq, hkv, d, n_rows, kcs, q, kl, vl)
    assert np.isnan(out[:, 0:2, 6]).all()       # +Inf is reported as NaN
    keep = np.ones(out.shape, bool)
    keep[:, 0:2, 6] = False
    assert np.isfinite(out[keep]).all()


# --------------------------------------------------------------------------- argmax

def test_argmax_matches_numpy_first_occurrence():
    x = pins.argmax_rows()
    ids, flags = oracle.argmax(x)
    ref_ids, ref_flags = pins.numpy_argmax(x)
    np.testing.assert_array_equal(ids, ref_ids)
    np.testing.assert_array_equal(flags, ref_flags)


def test_argmax_special_cases():
    x = pins.argmax_rows(vocab=3000)
    ids, flags = oracle.argmax(x)
    assert ids[0] == 0 and ids[1] == 5           # ties go to the lower id
    assert ids[3] == 0                           # all equal
    assert ids[4] == 2999                        # max at the last id
    assert ids[5] == 7                           # -0.0 == +0.0, lower id
    assert ids[6] == 0 and flags[6] == 1         # all NaN
    assert flags[7] == 1 and ids[7] != 0         # NaN at id 0 ranks as -inf
    assert flags[8] == 1 and flags[9] == 1 and flags[2] == 0
    assert ids[10] == 0 and flags[10] == 1       # all -inf, NaN in the middle
    assert ids[11] == 20 and flags[11] == 1


def test_argmax_respects_vocab_and_stride():
    x = pins.argmax_rows(seed=12, rows=12, vocab=500)
    wide = np.full((12, 512), synth.f32_to_bf16_bits(np.float32(99.0)), dtype=np.uint16)
    wide[:, :500] = x
    ids, flags = oracle.argmax(wide, vocab=500)
    assert (ids < 500).all()
    ref_ids, ref_flags = pins.numpy_argmax(x)
    np.testing.assert_array_equal(ids, ref_ids)
    np.testing.assert_array_equal(flags, ref_flags)


def test_oracle_reports_threads():
    n_rows, kcs, q, kl, vl = pins.random_case(40, 2, 1, 4, [(1, 5)])
    _, used = oracle.attn(n_rows, kcs, q, kl, vl, n_q_heads=2, n_kv_heads=1, head_dim=4,
                          scale=0.5, threads=3, return_threads=True)
    assert used == 3

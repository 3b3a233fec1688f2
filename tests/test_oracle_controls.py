"""Planted controls: each plausible mistake, edited into a temporary copy of the
oracle source, must turn one of the pins red.  Nothing here touches the shipped
oracle; the edits live only in a temporary directory."""
import functools
import math
import os
import subprocess

import numpy as np
import pytest

from oracle import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

ATTN_CONTROLS = [
    ("gqa groups interleaved", "const int g = t->head / group;", "const int g = t->head % hkv;"),
    ("scale dropped", "acc *= scale;", ";"),
    ("causal count off by one", "return j <= first_new + t->row;", "return j < first_new + t->row;"),
    ("max subtraction sign", "const double p = exp(s[j] - m);", "const double p = exp(m - s[j]);"),
    ("last key dropped from P.V",
     "for (int j = 0; j < t->key_count; ++j) {\n                if (!sees(t, j))\n                    continue;\n                const double p",
     "for (int j = 0; j + 1 < t->key_count; ++j) {\n                if (!sees(t, j))\n                    continue;\n                const double p"),
    ("k dims reversed", "acc += qd[x] * bf16_value(kr[x]);", "acc += qd[x] * bf16_value(kr[d - 1 - x]);"),
    ("v read from kv head 0", "const uint16_t *vr = vs + ((int64_t)j * hkv + g) * d;\n                l += p;",
     "const uint16_t *vr = vs + ((int64_t)j * hkv) * d;\n                l += p;"),
]
FULL_CONTROLS = [
    ("full read as causal", "case MASK_FULL:\n        return 1;", "case MASK_FULL:\n        return j <= first_new + t->row;"),
    ("full drops the newest key", "case MASK_FULL:\n        return 1;", "case MASK_FULL:\n        return j + 1 < t->key_count;"),
]
TREE_CONTROLS = [
    ("tree bit off by one", "(t->anc >> (j - first_new)) & 1u", "(t->anc >> (j - first_new + 1)) & 1u"),
    ("tree row misses its own key", "if (j < first_new || j == first_new + t->row)", "if (j < first_new)"),
    ("tree context dropped", "if (j < first_new || j == first_new + t->row)", "if (j == first_new + t->row)"),
    ("tree masks read from the segment's first row", "tree[row_offset[s] + r]", "tree[row_offset[s]]"),
]
ARGMAX_CONTROLS = [
    ("ties to the highest id", "if (i == 0 || key > best_key)", "if (i == 0 || key >= best_key)"),
    ("Inf not flagged", "if (!isfinite(x))\n                flag = 1;", "if (isnan(x))\n                flag = 1;"),
    ("NaN not ranked as -inf", "const double key = isnan(x) ? -INFINITY : x;", "const double key = x;"),
]
MERGE_CONTROLS = [
    ("merge skips the last split",
     "for (int t = 0; t < n_split; ++t) {\n            if (m[t] == -INFINITY)",
     "for (int t = 0; t + 1 < n_split; ++t) {\n            if (m[t] == -INFINITY)"),
]


def _build_variant(tmp_path, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"control anchor not found: {old!r}"
    path = tmp_path / "oracle_variant.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_variant.so"
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-fopenmp", "-o",
                           str(so), str(path), "-lm"])
    return oracle.load_library(str(so))


def _attention_red(lib):
    return pins.check_attention(functools.partial(oracle.attn, lib=lib)) > 1e-9


def _argmax_red(lib):
    x = pins.argmax_rows()
    ids, flags = oracle.argmax(x, lib=lib)
    ref_ids, ref_flags = pins.numpy_argmax(x)
    return not (np.array_equal(ids, ref_ids) and np.array_equal(flags, ref_flags))


def _merge_red(lib):
    hq, hkv, d = 4, 2, 8
    n_rows, kcs, q, kl, vl = pins.random_case(37, hq, hkv, d, [(1, 700), (3, 65)])
    kw = dict(n_q_heads=hq, n_kv_heads=hkv, head_dim=d, scale=1 / math.sqrt(d), lib=lib)
    full = oracle.attn(n_rows, kcs, q, kl, vl, **kw)
    m, l, o = oracle.attn_partials(n_rows, kcs, q, kl, vl, split=7, **kw)
    got = oracle.merge(m, l, o, lib=lib)
    return not np.allclose(got, full, rtol=0, atol=1e-12)


def test_unedited_source_is_green(tmp_path):
    lib = _build_variant(tmp_path, "#include <math.h>", "#include <math.h>")
    assert not _attention_red(lib) and not _argmax_red(lib) and not _merge_red(lib)


@pytest.mark.parametrize("name,old,new", ATTN_CONTROLS, ids=[c[0] for c in ATTN_CONTROLS])
def test_attention_control_goes_red(tmp_path, name, old, new):
    assert _attention_red(_build_variant(tmp_path, old, new)), name


@pytest.mark.parametrize("name,old,new", FULL_CONTROLS, ids=[c[0] for c in FULL_CONTROLS])
def test_full_control_goes_red(tmp_path, name, old, new):
    lib = _build_variant(tmp_path, old, new)
    cases = pins.SDPA_CASES + pins.MASK_CASES
    assert pins.check_attention(functools.partial(oracle.attn, lib=lib), cases, mask="full") > 1e-9, name


@pytest.mark.parametrize("name,old,new", TREE_CONTROLS, ids=[c[0] for c in TREE_CONTROLS])
def test_tree_control_goes_red(tmp_path, name, old, new):
    lib = _build_variant(tmp_path, old, new)
    cases = pins.SDPA_CASES + pins.MASK_CASES
    assert pins.check_attention(functools.partial(oracle.attn, lib=lib), cases, mask="tree") > 1e-9, name


@pytest.mark.parametrize("name,old,new", ARGMAX_CONTROLS, ids=[c[0] for c in ARGMAX_CONTROLS])
def test_argmax_control_goes_red(tmp_path, name, old, new):
    assert _argmax_red(_build_variant(tmp_path, old, new)), name


@pytest.mark.parametrize("name,old,new", MERGE_CONTROLS, ids=[c[0] for c in MERGE_CONTROLS])
def test_merge_control_goes_red(tmp_path, name, old, new):
    assert _merge_red(_build_variant(tmp_path, old, new)), name

"""Independent references the oracle is pinned to (CPU only).

None of these re-types the oracle's loops: the attention references go through
torch's float64 ``scaled_dot_product_attention`` (grouped-query mode, boolean
causal mask) and through scipy's softmax with numpy matmul; the argmax
reference is ``numpy.argmax`` (first occurrence) on NaN-masked rows.
"""
import math

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

from stream_paged_attention_amd import synth


def f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def causal_mask(n, kc):
    r = np.arange(n)[:, None]
    j = np.arange(kc)[None, :]
    return j < (kc - n + r + 1)


def full_mask(n, kc):
    return np.ones((n, kc), dtype=bool)


def tree_mask(n, kc, parents):
    """Context keys, the row's own key, and its ancestors' keys, found by
    walking the parent links."""
    m = np.zeros((n, kc), dtype=bool)
    m[:, :kc - n] = True
    for r in range(n):
        a = r
        while a >= 0:
            m[r, kc - n + a] = True
            a = int(parents[a])
    return m


def sdpa(n_rows, kcs, q, kl, vl, hq, hkv, d, masks=None):
    """torch float64 SDPA per segment, grouped-query mode, with a boolean mask
    per segment (the causal-count mask unless ``masks`` gives one)."""
    outs, off = [], 0
    for i, (n, kc, k, v) in enumerate(zip(n_rows, kcs, kl, vl)):
        qq = torch.from_numpy(f64(q[off:off + n])).permute(1, 0, 2)[None]
        kk = torch.from_numpy(f64(k)).permute(1, 0, 2)[None]
        vv = torch.from_numpy(f64(v)).permute(1, 0, 2)[None]
        mask = torch.from_numpy(causal_mask(n, kc) if masks is None else masks[i])
        o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask,
                                           scale=1.0 / math.sqrt(d), enable_gqa=hq != hkv)
        outs.append(o[0].permute(1, 0, 2).numpy())
        off += n
    return np.concatenate(outs)


def textbook_mha(n, kc, q, k, v, d):
    """softmax(QK^T / sqrt(d) + causal mask) V per head with scipy + numpy (Hq == Hkv)."""
    qq, kk, vv = f64(q), f64(k), f64(v)          # [n][H][d], [kc][H][d]
    out = np.empty_like(qq)
    mask = causal_mask(n, kc)
    for h in range(qq.shape[1]):
        s = qq[:, h, :] @ kk[:, h, :].T / math.sqrt(d)
        s = np.where(mask, s, -np.inf)
        out[:, h, :] = scipy.special.softmax(s, axis=1) @ vv[:, h, :]
    return out


def numpy_argmax(bits, vocab=None):
    x = synth.bf16_bits_to_f32(bits).astype(np.float64)
    if vocab is not None:
        x = x[:, :vocab]
    keyed = np.where(np.isnan(x), -np.inf, x)
    return np.argmax(keyed, axis=1).astype(np.int32), (~np.isfinite(x)).any(axis=1).astype(np.uint8)


def random_case(seed, hq, hkv, d, segs, qscale=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    n_rows = [n for n, _ in segs]
    kcs = [kc for _, kc in segs]
    q = synth.f32_to_bf16_bits(qscale * rng.standard_normal((sum(n_rows), hq, d), dtype=np.float32))
    kl = [synth.f32_to_bf16_bits(rng.standard_normal((kc, hkv, d), dtype=np.float32)) for kc in kcs]
    vl = [synth.f32_to_bf16_bits(rng.standard_normal((kc, hkv, d), dtype=np.float32)) for kc in kcs]
    return n_rows, kcs, q, kl, vl


SDPA_CASES = [
    # (seed, Hq, Hkv, D, [(rows, keys) per segment], q scale)
    (1, 1, 1, 1, [(1, 1), (2, 3)], 1.0),
    (2, 2, 1, 2, [(1, 5), (3, 5)], 1.0),
    (3, 4, 2, 4, [(1, 33), (3, 33), (2, 2)], 1.0),
    (4, 8, 2, 8, [(1, 7), (4, 40)], 1.0),
    (5, 6, 3, 5, [(2, 9)], 1.0),
    (6, 4, 4, 16, [(5, 64), (1, 1)], 1.0),
    (7, 4, 1, 8, [(3, 33)], 400.0),   # scores far past exp()'s range: needs the max subtraction
]

# Cases for the full and tree masks: blocks of several rows, some with no
# context (key count == rows), some with a long one.
MASK_CASES = [
    (51, 2, 1, 4, [(4, 4), (1, 6)], 1.0),
    (52, 4, 2, 8, [(9, 40), (3, 3), (6, 7)], 1.0),
    (53, 8, 2, 16, [(16, 100)], 1.0),
    (54, 4, 1, 8, [(5, 20)], 300.0),
]


def check_attention(attn_fn, cases=SDPA_CASES, tol=1e-12, mask="causal"):
    """Return the worst |oracle - sdpa| over the cases, under the causal, full
    or tree mask (trees: parents drawn per segment, passed to the oracle as
    ancestor bit masks and to torch as boolean masks)."""
    worst = 0.0
    for seed, hq, hkv, d, segs, qs in cases:
        n_rows, kcs, q, kl, vl = random_case(seed, hq, hkv, d, segs, qs)
        kw = {}
        masks = None
        if mask == "full":
            kw = dict(mask="full")
            masks = [full_mask(n, kc) for n, kc in zip(n_rows, kcs)]
        elif mask == "tree":
            rng = np.random.Generator(np.random.PCG64(seed + 1000))
            parents = [synth.random_parents(rng, n) for n in n_rows]
            kw = dict(mask="tree", tree=np.concatenate([synth.ancestor_masks(p) for p in parents]))
            masks = [tree_mask(n, kc, p) for n, kc, p in zip(n_rows, kcs, parents)]
        got = attn_fn(n_rows, kcs, q, kl, vl, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                      scale=1.0 / math.sqrt(d), **kw)
        ref = sdpa(n_rows, kcs, q, kl, vl, hq, hkv, d, masks)
        if not np.all(np.isfinite(got)):
            return math.inf
        worst = max(worst, float(np.max(np.abs(got - ref))))
    return worst


def argmax_rows(seed=11, rows=24, vocab=3000):
    """Random rows with planted ties, NaN/Inf plants and the special cases."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = synth.normal_logits(rng, rows, vocab)
    synth.plant_tie(x, 0, [0, vocab - 1])
    synth.plant_tie(x, 1, [5, 6])
    synth.plant_tie(x, 2, sorted(rng.choice(vocab, 3, replace=False).tolist()))
    x[3, :] = synth.f32_to_bf16_bits(np.float32(0.25))          # all equal -> 0
    x[4, :] = synth.f32_to_bf16_bits(np.float32(-1.0))
    x[4, vocab - 1] = synth.f32_to_bf16_bits(np.float32(2.0))    # max at the last id
    x[5, :] = synth.f32_to_bf16_bits(np.float32(-1.0))
    x[5, 7] = np.uint16(0x8000)                                   # -0.0 ties +0.0
    x[5, 9] = np.uint16(0x0000)
    x[6, :] = synth.BF16_NAN                                      # all NaN -> 0, flagged
    x[7, 0] = synth.BF16_NAN                                      # NaN first, then finite
    x[8, int(rng.integers(vocab))] = synth.BF16_POS_INF
    x[9, int(rng.integers(vocab))] = synth.BF16_NEG_INF
    x[10, :] = synth.BF16_NEG_INF                                 # all -inf -> 0
    x[10, 100] = synth.BF16_NAN                                   # NaN ranks as -inf: still 0
    x[11, 50] = synth.BF16_NAN
    synth.plant_tie(x, 11, [20, 60])
    return x

"""Seeded kept-state cases shared by the CPU pins and the GPU tests: a stream's
logical K/V rows per layer placed into a shuffled page list of a pool, and
state buffers holding random bits beforehand (so rows that must stay
untouched can be seen)."""
import dataclasses
from typing import List, Tuple

import numpy as np

from stream_paged_attention_amd import synth


@dataclasses.dataclass
class LayersCase:
    pools: List[Tuple[np.ndarray, np.ndarray]]     # per layer [pool_pages][Hkv][P][D]
    states: List[Tuple[np.ndarray, np.ndarray]]    # per layer [ceil(at/P)][Hkv][P][D]
    logical: List[Tuple[np.ndarray, np.ndarray]]   # per layer [n_pages*P][Hkv][D]
    pages: np.ndarray                              # int32, n_pages entries
    pool_pages: int
    page_size: int
    at: int


def layers_case(seed, n_layers, hkv, d, page_size, at, n_pages=None, pool_pages=None) -> LayersCase:
    rng = np.random.Generator(np.random.PCG64(seed))
    n_state = -(-at // page_size)
    n_pages = max(n_state, 1) if n_pages is None else n_pages
    pool_pages = 2 * n_pages + 3 if pool_pages is None else pool_pages
    pages = rng.permutation(pool_pages)[:n_pages].astype(np.int32)
    pools, states, logical = [], [], []
    for _ in range(n_layers):
        lk = synth.f32_to_bf16_bits(rng.standard_normal((n_pages * page_size, hkv, d), dtype=np.float32))
        lv = synth.f32_to_bf16_bits(rng.standard_normal((n_pages * page_size, hkv, d), dtype=np.float32))
        pk = synth.place_paged([lk], page_size, pool_pages, [pages])
        pv = synth.place_paged([lv], page_size, pool_pages, [pages])
        shape = (max(n_state, 1), hkv, page_size, d)
        sk = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        sv = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        pools.append((pk, pv))
        states.append((sk, sv))
        logical.append((lk, lv))
    return LayersCase(pools, states, logical, pages, pool_pages, page_size, at)

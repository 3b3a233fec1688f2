"""Seeded synthetic inputs for shared-round attention and greedy argmax.

This module draws values and places them; it holds none of the method's
arithmetic (no scores, no softmax, no merge, no argmax).  It is the one thing
the float64 oracle and the HIP path share: the oracle reads the *logical*
per-stream K/V copies it returns, the HIP path reads the same values after
they have been placed into pages of a shared pool, a wrapping ring or a
contiguous buffer.

Storage layouts (all bf16, kept as uint16 bit patterns on the host):

* logical copy (oracle input): ``[key][kv_head][dim]`` per stream;
* paged pool: ``[page][kv_head][page_size][dim]`` -- one page holds
  ``page_size`` consecutive logical keys of one stream, head-major so that a
  kv head's run of keys is one contiguous block;
* ring: ``[kv_head][slots][dim]`` per stream, logical key j in slot
  ``(first + j) mod slots``;
* contiguous: ``[kv_head][capacity][dim]`` per stream.

Every slot that no logical key occupies (unused pool pages, the tail of a
stream's last page, ring slots outside the valid range, contiguous capacity
past the key count) is filled with a bf16 NaN, so that a read outside the
visible range shows up in the output.

Values are float32 standard normals rounded to bf16 with round-to-nearest-even,
drawn from ``numpy.random.Generator(PCG64(seed))`` in a fixed order: structure
(row and key counts, ring heads), then the page permutation, then Q, then each
stream's K and V in stream order, then logits, then plants.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
BF16_POS_INF = np.uint16(0x7F80)
BF16_NEG_INF = np.uint16(0xFF80)

KIND_CONTIG = "contig"
KIND_PAGED = "paged"
KIND_RING = "ring"


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); NaN -> 0x7FC0."""
    x = np.asarray(x, dtype=np.float32)
    shape = x.shape
    x = np.ascontiguousarray(x.reshape(-1))
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = (r & 0xFFFF).astype(np.uint16)
    out[np.isnan(x)] = BF16_NAN
    return out.reshape(shape)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


@dataclasses.dataclass
class Segment:
    """One stream's span in a shared launch (host description)."""

    n_rows: int
    key_count: int
    row_offset: int
    capacity: int = 0          # paged: entries of ``pages``; ring: slots; contig: keys allocated
    first: int = 0             # ring: slot holding logical key 0
    pages: Optional[np.ndarray] = None   # paged: int32 logical page -> pool page


@dataclasses.dataclass
class Workload:
    name: str
    kind: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    split_keys: int
    scale: float
    segments: List[Segment]
    q: np.ndarray                      # uint16 [total_rows][Hq][D]
    k_logical: List[np.ndarray]        # uint16 [key_count][Hkv][D] per stream
    v_logical: List[np.ndarray]
    pool_k: Optional[np.ndarray] = None   # paged: uint16 [pool_pages][Hkv][P][D]
    pool_v: Optional[np.ndarray] = None
    store_k: Optional[List[np.ndarray]] = None  # ring/contig: uint16 [Hkv][capacity][D] per stream
    store_v: Optional[List[np.ndarray]] = None
    logits: Optional[np.ndarray] = None   # uint16 [rows][vocab]
    notes: str = ""
    mask: str = "causal"                  # "causal", "full" or "tree"
    tree: Optional[np.ndarray] = None     # tree: uint64 ancestor mask per packed row

    @property
    def total_rows(self) -> int:
        return int(sum(s.n_rows for s in self.segments))

    @property
    def max_rows(self) -> int:
        return int(max([s.n_rows for s in self.segments] or [0]))

    @property
    def max_keys(self) -> int:
        return int(max([s.key_count for s in self.segments] or [0]))

    @property
    def pool_pages(self) -> int:
        return 0 if self.pool_k is None else int(self.pool_k.shape[0])


# ----------------------------------------------------------------------------
# placement of logical K/V into storage
# ----------------------------------------------------------------------------

def place_paged(k_logical: Sequence[np.ndarray], page_size: int, pool_pages: int,
                page_lists: Sequence[np.ndarray], fill=BF16_NAN) -> np.ndarray:
    """Scatter each stream's logical rows into the pool pages its list names."""
    assert len(k_logical) == len(page_lists)
    hkv, d = k_logical[0].shape[1], k_logical[0].shape[2]
    pool = np.full((pool_pages, hkv, page_size, d), fill, dtype=np.uint16)
    for kl, pages in zip(k_logical, page_lists):
        kc = kl.shape[0]
        npg = -(-kc // page_size)
        assert len(pages) >= npg
        padded = np.full((npg * page_size, hkv, d), fill, dtype=np.uint16)
        padded[:kc] = kl
        blocks = padded.reshape(npg, page_size, hkv, d).transpose(0, 2, 1, 3)
        pool[np.asarray(pages[:npg], dtype=np.int64)] = blocks
    return pool


def place_ring(kl: np.ndarray, slots: int, first: int, fill=BF16_NAN) -> np.ndarray:
    """Put logical key j of one stream into ring slot (first + j) mod slots."""
    kc, hkv, d = kl.shape
    assert kc <= slots and 0 <= first < slots
    ring = np.full((hkv, slots, d), fill, dtype=np.uint16)
    idx = (first + np.arange(kc, dtype=np.int64)) % slots
    ring[:, idx, :] = kl.transpose(1, 0, 2)
    return ring


def place_contig(kl: np.ndarray, capacity: int, fill=BF16_NAN) -> np.ndarray:
    kc, hkv, d = kl.shape
    assert kc <= capacity
    buf = np.full((hkv, capacity, d), fill, dtype=np.uint16)
    buf[:, :kc, :] = kl.transpose(1, 0, 2)
    return buf


def consecutive_page_lists(key_counts: Sequence[int], page_size: int,
                           perm: np.ndarray) -> List[np.ndarray]:
    """Each stream takes the next ceil(kc/P) ids of a page permutation."""
    out, at = [], 0
    for kc in key_counts:
        npg = -(-int(kc) // page_size)
        out.append(np.ascontiguousarray(perm[at:at + npg], dtype=np.int32))
        at += npg
    assert at <= len(perm), "pool too small for the streams' pages"
    return out


def _segments(n_rows: Sequence[int], key_counts: Sequence[int]) -> List[Segment]:
    segs, off = [], 0
    for n, kc in zip(n_rows, key_counts):
        segs.append(Segment(n_rows=int(n), key_count=int(kc), row_offset=off))
        off += int(n)
    return segs


def restore(w: Workload, kind: str, *, seed: int = 0, pool_pages: Optional[int] = None,
            page_size: Optional[int] = None, ring_slots: Optional[int] = None,
            ring_first: Optional[Sequence[int]] = None,
            capacity: Optional[Sequence[int]] = None, fill=BF16_NAN) -> Workload:
    """Same logical K/V and Q, placed into another storage kind or permutation.

    Used for the equality checks (two page permutations, paged against
    contiguous, a wrapped ring against its contiguous copy).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    segs = [dataclasses.replace(s, pages=None, first=0, capacity=0) for s in w.segments]
    kcs = [s.key_count for s in segs]
    out = dataclasses.replace(w, kind=kind, segments=segs, pool_k=None, pool_v=None,
                              store_k=None, store_v=None)
    if kind == KIND_PAGED:
        p = page_size or w.page_size
        need = sum(-(-kc // p) for kc in kcs)
        npool = pool_pages or need
        perm = rng.permutation(npool).astype(np.int32)
        lists = consecutive_page_lists(kcs, p, perm)
        for s, pl in zip(segs, lists):
            s.pages, s.capacity = pl, len(pl)
        out.page_size = p
        out.pool_k = place_paged(w.k_logical, p, npool, lists, fill)
        out.pool_v = place_paged(w.v_logical, p, npool, lists, fill)
    elif kind == KIND_RING:
        out.store_k, out.store_v = [], []
        for i, s in enumerate(segs):
            slots = ring_slots or s.key_count
            first = int(ring_first[i]) if ring_first is not None else int(rng.integers(0, slots))
            s.capacity, s.first = slots, first
            out.store_k.append(place_ring(w.k_logical[i], slots, first, fill))
            out.store_v.append(place_ring(w.v_logical[i], slots, first, fill))
    elif kind == KIND_CONTIG:
        out.store_k, out.store_v = [], []
        for i, s in enumerate(segs):
            cap = int(capacity[i]) if capacity is not None else s.key_count
            s.capacity = cap
            out.store_k.append(place_contig(w.k_logical[i], cap, fill))
            out.store_v.append(place_contig(w.v_logical[i], cap, fill))
    else:
        raise ValueError(kind)
    return out


# ----------------------------------------------------------------------------
# general builder
# ----------------------------------------------------------------------------

def make_workload(name: str, kind: str, n_q_heads: int, n_kv_heads: int, head_dim: int,
                  n_rows: Sequence[int], key_counts: Sequence[int], *, seed: int,
                  page_size: int = 32, pool_pages: Optional[int] = None,
                  ring_slots: Optional[Sequence[int]] = None,
                  ring_heads: Optional[Sequence[int]] = None,
                  contig_capacity: Optional[Sequence[int]] = None,
                  split_keys: int = 512, rng: Optional[np.random.Generator] = None,
                  draw_perm: bool = True) -> Workload:
    """Draw Q and each stream's K/V and place them.

    Order of draws: page permutation (paged), Q, then K and V stream by stream.
    ``ring_heads`` gives each ring's write head; logical key 0 then sits at
    slot ``(head - key_count) mod slots``.
    """
    rng = rng if rng is not None else np.random.Generator(np.random.PCG64(seed))
    segs = _segments(n_rows, key_counts)
    for s in segs:
        assert 1 <= s.n_rows <= s.key_count
    perm = None
    if kind == KIND_PAGED:
        need = sum(-(-int(kc) // page_size) for kc in key_counts)
        npool = pool_pages if pool_pages is not None else need
        assert npool >= need
        perm = (rng.permutation(npool) if draw_perm else np.arange(npool)).astype(np.int32)
    total = sum(int(n) for n in n_rows)
    q = _normal_bf16(rng, (total, n_q_heads, head_dim))
    kl, vl = [], []
    for kc in key_counts:
        kl.append(_normal_bf16(rng, (int(kc), n_kv_heads, head_dim)))
        vl.append(_normal_bf16(rng, (int(kc), n_kv_heads, head_dim)))
    w = Workload(name=name, kind=kind, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                 head_dim=head_dim, page_size=page_size if kind == KIND_PAGED else 0,
                 split_keys=split_keys, scale=float(1.0 / np.sqrt(head_dim)),
                 segments=segs, q=q, k_logical=kl, v_logical=vl)
    if kind == KIND_PAGED:
        lists = consecutive_page_lists(key_counts, page_size, perm)
        for s, pl in zip(segs, lists):
            s.pages, s.capacity = pl, len(pl)
        w.pool_k = place_paged(kl, page_size, len(perm), lists)
        w.pool_v = place_paged(vl, page_size, len(perm), lists)
    elif kind == KIND_RING:
        w.store_k, w.store_v = [], []
        for i, s in enumerate(segs):
            slots = int(ring_slots[i]) if ring_slots is not None else s.key_count
            head = int(ring_heads[i]) if ring_heads is not None else 0
            s.capacity = slots
            s.first = (head - s.key_count) % slots
            w.store_k.append(place_ring(kl[i], slots, s.first))
            w.store_v.append(place_ring(vl[i], slots, s.first))
    elif kind == KIND_CONTIG:
        w.store_k, w.store_v = [], []
        for i, s in enumerate(segs):
            cap = int(contig_capacity[i]) if contig_capacity is not None else s.key_count
            s.capacity = cap
            w.store_k.append(place_contig(kl[i], cap))
            w.store_v.append(place_contig(vl[i], cap))
    else:
        raise ValueError(kind)
    return w


def random_parents(rng: np.random.Generator, n: int, chain: bool = False) -> np.ndarray:
    """A draft tree over a segment's n rows: parent[r] < r, or -1 for a row
    that hangs off the context alone.  Row 0 is the root; ``chain`` gives the
    degenerate tree parent[r] = r - 1."""
    if chain:
        return np.arange(-1, n - 1, dtype=np.int64)
    par = np.full(n, -1, dtype=np.int64)
    for r in range(1, n):
        par[r] = int(rng.integers(0, r))
    return par


def ancestor_masks(parents: Sequence[int]) -> np.ndarray:
    """The tree mask format the library takes: for each row, bit j set when
    row j lies on its path to the root (the row itself not included)."""
    n = len(parents)
    assert n <= 64
    out = np.zeros(n, dtype=np.uint64)
    for r in range(n):
        bits, a = 0, int(parents[r])
        while a >= 0:
            assert a < r
            bits |= 1 << a
            a = int(parents[a])
        out[r] = np.uint64(bits)
    return out


def with_trees(w: Workload, seed: int, chain: bool = False) -> Workload:
    """The same workload under a tree mask, one drawn tree per segment."""
    rng = np.random.Generator(np.random.PCG64(seed))
    tree = np.zeros(w.total_rows, dtype=np.uint64)
    for s in w.segments:
        tree[s.row_offset:s.row_offset + s.n_rows] = ancestor_masks(
            random_parents(rng, s.n_rows, chain))
    return dataclasses.replace(w, mask="tree", tree=tree)


def normal_logits(rng: np.random.Generator, rows: int, vocab: int) -> np.ndarray:
    return _normal_bf16(rng, (rows, vocab))


def plant_tie(logits: np.ndarray, row: int, idx: Sequence[int]) -> None:
    """Set the given ids of one row to one value above the row's largest finite logit."""
    vals = bf16_bits_to_f32(logits[row])
    top = float(np.max(vals[np.isfinite(vals)]))
    logits[row, np.asarray(idx, dtype=np.int64)] = f32_to_bf16_bits(np.float32(top + 0.5))


# ----------------------------------------------------------------------------
# the five synthetic workloads
# ----------------------------------------------------------------------------

# Names, in the order their seeds were assigned: every value a workload holds
# is drawn from numpy.random.Generator(PCG64(seed)) with this seed.
WORKLOADS = ("single64", "decode16", "verify8", "prompt512", "ring17")
WORKLOAD_SEED = {name: i + 1 for i, name in enumerate(WORKLOADS)}

WORKLOAD_TITLES = {
    "single64": "1 stream x 1 row, 8/2 heads, D64, 256 contiguous keys; argmax 1x1024 with a planted tie",
    "decode16": "16 one-row decode streams, 32/8 heads, D128, keys U[512,4096] in 32-token pages "
                "of a permuted 4096-page pool, split-K 512 + merge",
    "verify8": "verify round: 8 streams of 1-16 causal rows, 16/4 heads, D256, committed keys "
               "U[2048,16384] in 32-token pages; argmax over 128000 logits per row",
    "prompt512": "prompt chunk: 1 stream, 512 causal rows over 15000 keys (14488 + 512), 16/4 heads, "
                 "D256, 32-token pages",
    "ring17": "ring drafter: 17 streams of 1-16 rows, 4200-slot rings with a random write head, "
              "16/2 heads, D128; argmax 32x128000 with planted ties, a NaN row and a +Inf row",
}

# split_keys used for each workload (keys per partial; 0 = one partial per row-head)
# Split sizes: decode16 as its workload states; the others are the
# fastest measured for that workload (the prompt chunk: four equal splits
# of its 15 000 keys, one matrix-core workgroup a CU).
WORKLOAD_SPLIT = {"single64": 0, "decode16": 512, "verify8": 512, "prompt512": 3776, "ring17": 512}


def make_synthetic(name: str) -> Workload:
    """Build the named synthetic workload (one of WORKLOADS) from its seed."""
    if name not in WORKLOAD_SEED:
        raise ValueError(f"no synthetic workload {name!r}")
    n = WORKLOAD_SEED[name]
    rng = np.random.Generator(np.random.PCG64(n))
    if name == "single64":
        w = make_workload("single64", KIND_CONTIG, 8, 2, 64, [1], [256], seed=n, rng=rng,
                          split_keys=WORKLOAD_SPLIT["single64"])
        logits = normal_logits(rng, 1, 1024)
        idx = np.sort(rng.choice(1024, size=2, replace=False))
        plant_tie(logits, 0, idx)
        w.logits = logits
        w.notes = f"tie planted at ids {idx.tolist()}"
    elif name == "decode16":
        kcs = rng.integers(512, 4096, size=16, endpoint=True)
        w = make_workload("decode16", KIND_PAGED, 32, 8, 128, [1] * 16, kcs.tolist(), seed=n,
                          rng=rng, page_size=32, pool_pages=4096, split_keys=WORKLOAD_SPLIT["decode16"])
    elif name == "verify8":
        rows = rng.integers(1, 16, size=8, endpoint=True)
        committed = rng.integers(2048, 16384, size=8, endpoint=True)
        kcs = committed + rows
        w = make_workload("verify8", KIND_PAGED, 16, 4, 256, rows.tolist(), kcs.tolist(),
                          seed=n, rng=rng, page_size=32, pool_pages=4608,
                          split_keys=WORKLOAD_SPLIT["verify8"])
        total = int(rows.sum())
        logits = normal_logits(rng, total, 128000)
        row = int(rng.integers(0, total))
        idx = np.sort(rng.choice(128000, size=2, replace=False))
        plant_tie(logits, row, idx)
        w.logits = logits
        w.notes = f"tie planted in row {row} at ids {idx.tolist()}"
    elif name == "prompt512":
        w = make_workload("prompt512", KIND_PAGED, 16, 4, 256, [512], [15000], seed=n, rng=rng,
                          page_size=32, pool_pages=1024, split_keys=WORKLOAD_SPLIT["prompt512"])
    elif name == "ring17":
        heads = rng.integers(1, 4199, size=17, endpoint=True)
        rows = rng.integers(1, 16, size=17, endpoint=True)
        w = make_workload("ring17", KIND_RING, 16, 2, 128, rows.tolist(), [4200] * 17,
                          seed=n, rng=rng, ring_slots=[4200] * 17, ring_heads=heads.tolist(),
                          split_keys=WORKLOAD_SPLIT["ring17"])
        logits = normal_logits(rng, 32, 128000)
        plant_tie(logits, 0, [0, 127999])
        plant_tie(logits, 1, np.sort(rng.choice(128000, size=2, replace=False)))
        plant_tie(logits, 2, np.sort(rng.choice(128000, size=3, replace=False)))
        a = int(rng.integers(0, 127999))
        plant_tie(logits, 3, [a, a + 1])
        logits[4, int(rng.integers(0, 128000))] = BF16_NAN
        logits[5, int(rng.integers(0, 128000))] = BF16_POS_INF
        w.logits = logits
        w.notes = "ties in rows 0-3, NaN in row 4, +Inf in row 5"
    w.name = name
    return w


def gather_paged(pool: np.ndarray, pages: np.ndarray, key_count: int) -> np.ndarray:
    """Read a stream's logical rows back out of a pool (test helper)."""
    p = pool.shape[2]
    npg = -(-key_count // p)
    blocks = pool[np.asarray(pages[:npg], dtype=np.int64)]           # [npg][Hkv][P][D]
    rows = blocks.transpose(0, 2, 1, 3).reshape(npg * p, pool.shape[1], pool.shape[3])
    return rows[:key_count]


def gather_ring(ring: np.ndarray, first: int, key_count: int) -> np.ndarray:
    slots = ring.shape[1]
    idx = (first + np.arange(key_count)) % slots
    return ring[:, idx, :].transpose(1, 0, 2)


def row_map(segments: Sequence[Segment]) -> List[Tuple[int, int]]:
    """(segment, row-in-segment) of every packed query row."""
    out = []
    for si, s in enumerate(segments):
        out.extend((si, r) for r in range(s.n_rows))
    return out

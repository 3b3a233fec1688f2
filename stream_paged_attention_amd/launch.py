"""Put a synthetic workload into device memory and call the C ABI on it.

PyTorch is used only to allocate device memory, copy the host inputs in and
hand out the current stream; every step of the attention and argmax runs in
libtfattn.so through ``binding``.  bf16 data stays as 16-bit patterns
(int16 tensors).
"""
from __future__ import annotations

import ctypes
from typing import List, Optional

import numpy as np
import torch

from . import binding
from .synth import Workload


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def to_host_u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def check(rc: int, what: str) -> None:
    if rc != binding.TF_OK:
        raise RuntimeError(f"{what} failed: {rc} ({binding.tf_strerror(rc)})")


class DeviceWorkload:
    """Device copies of a workload's Q, K/V storage, tables and workspaces.

    ``copies`` > 1 keeps that many copies of the K/V storage (with their own
    segment tables) so a timing loop can rotate over them and read K/V from
    HBM rather than from the last-level cache.
    """

    def __init__(self, w: Workload, device="cuda:0", copies: int = 1,
                 split_keys: Optional[int] = None):
        self.w = w
        self.device = torch.device(device)
        self.kind = binding.KIND_CODE[w.kind]
        self.split_keys = w.split_keys if split_keys is None else split_keys
        self.q = _dev(w.q, self.device)
        self.out = torch.zeros(w.q.shape, dtype=torch.int16, device=self.device)
        self.err = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.mask = binding.MASK_CODE[w.mask]
        self.tree = (_dev(np.ascontiguousarray(w.tree, dtype=np.uint64).view(np.int64), self.device)
                     if w.mask == "tree" else None)
        self.copies = copies
        self.k_store: List[List[torch.Tensor]] = []
        self.v_store: List[List[torch.Tensor]] = []
        if w.kind == "paged":
            base_k, base_v = _dev(w.pool_k, self.device), _dev(w.pool_v, self.device)
            for c in range(copies):
                self.k_store.append([base_k if c == 0 else base_k.clone()])
                self.v_store.append([base_v if c == 0 else base_v.clone()])
            pages = np.concatenate([s.pages for s in w.segments]).astype(np.int32)
            self.pages = _dev(pages, self.device)
            self.page_off = np.concatenate([[0], np.cumsum([len(s.pages) for s in w.segments])])
        else:
            for c in range(copies):
                self.k_store.append([_dev(x, self.device) for x in w.store_k])
                self.v_store.append([_dev(x, self.device) for x in w.store_v])
            self.pages = None
        self.host_segs = self._host_segments(0)
        if self.split_keys > 0:
            rc, nbytes = binding.tf_plan_partials(self.host_segs, w.n_q_heads, w.head_dim,
                                                  self.split_keys)
            check(rc, "tf_plan_partials")
            self.partials = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32,
                                        device=self.device)
            self.partials_bytes = nbytes
        else:
            self.partials, self.partials_bytes = None, 0
        self.tables = []
        for c in range(copies):
            hs = self._host_segments(c)
            for i in range(len(hs)):
                hs[i].partial_offset = self.host_segs[i].partial_offset
            self.tables.append(self._upload(hs))

    # -- tables -----------------------------------------------------------------
    def _host_segments(self, copy: int):
        w = self.w
        arr = (binding.tf_segment * len(w.segments))()
        for i, s in enumerate(w.segments):
            e = arr[i]
            if w.kind == "paged":
                e.k = self.k_store[copy][0].data_ptr()
                e.v = self.v_store[copy][0].data_ptr()
                e.pages = self.pages.data_ptr() + 4 * int(self.page_off[i])
            else:
                e.k = self.k_store[copy][i].data_ptr()
                e.v = self.v_store[copy][i].data_ptr()
                e.pages = None
            e.capacity = s.capacity
            e.first = s.first
            e.row_offset = s.row_offset
            e.n_rows = s.n_rows
            e.key_count = s.key_count
            e.partial_offset = 0
        return arr

    def _upload(self, arr) -> torch.Tensor:
        raw = bytes(ctypes.string_at(ctypes.addressof(arr), ctypes.sizeof(arr)))
        return torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(self.device)

    # -- arguments ----------------------------------------------------------------
    def args(self, copy: int = 0) -> binding.tf_attn_args:
        w = self.w
        a = binding.tf_attn_args()
        a.kind = self.kind
        a.n_segments = len(w.segments)
        a.total_rows = w.total_rows
        a.max_rows = w.max_rows
        a.max_keys = w.max_keys
        a.min_rows = min((s.n_rows for s in w.segments), default=0)
        a.n_q_heads = w.n_q_heads
        a.n_kv_heads = w.n_kv_heads
        a.head_dim = w.head_dim
        a.page_size = w.page_size if w.kind == "paged" else 0
        a.pool_pages = w.pool_pages if w.kind == "paged" else 0
        a.split_keys = self.split_keys
        a.scale = w.scale
        a.mask = self.mask
        a.tree = self.tree.data_ptr() if self.tree is not None else None
        a.segs = self.tables[copy].data_ptr()
        a.q = self.q.data_ptr()
        a.out = self.out.data_ptr()
        a.partials = self.partials.data_ptr() if self.partials is not None else None
        a.partials_bytes = self.partials_bytes
        a.err = self.err.data_ptr()
        return a

    def check_table(self) -> int:
        return binding.tf_check_segments(self.args(0), self.host_segs)

    def run(self, copy: int = 0, stream: Optional[int] = None) -> None:
        """tf_attn_rows, then tf_attn_merge when there are split partials."""
        st = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        a = self.args(copy)
        check(binding.tf_attn_rows(a, st), "tf_attn_rows")
        if self.split_keys > 0:
            check(binding.tf_attn_merge(a, st), "tf_attn_merge")

    def output(self) -> np.ndarray:
        torch.cuda.synchronize(self.device)
        return to_host_u16(self.out)

    def error_word(self) -> int:
        torch.cuda.synchronize(self.device)
        return int(self.err.item())

    # -- one launch per segment ----------------------------------------------------
    def run_per_segment(self) -> np.ndarray:
        """Launch each segment alone (its own one-entry table, q, out, partials)."""
        w = self.w
        st = torch.cuda.current_stream(self.device).cuda_stream
        row_bytes = w.n_q_heads * w.head_dim * 2
        out = torch.zeros_like(self.out)
        keep = []
        for i, s in enumerate(w.segments):
            one = (binding.tf_segment * 1)()
            ctypes.memmove(ctypes.addressof(one), ctypes.addressof(self.host_segs[i]),
                           ctypes.sizeof(binding.tf_segment))
            one[0].row_offset = 0
            a = self.args(0)
            a.n_segments = 1
            a.total_rows = s.n_rows
            a.max_rows = s.n_rows
            a.max_keys = s.key_count
            a.min_rows = s.n_rows
            a.q = self.q.data_ptr() + s.row_offset * row_bytes
            a.out = out.data_ptr() + s.row_offset * row_bytes
            if self.tree is not None:
                a.tree = self.tree.data_ptr() + 8 * s.row_offset
            part = None
            if self.split_keys > 0:
                rc, nbytes = binding.tf_plan_partials(one, w.n_q_heads, w.head_dim,
                                                      self.split_keys)
                check(rc, "tf_plan_partials")
                part = torch.empty(max(nbytes, 16) // 4, dtype=torch.float32, device=self.device)
                a.partials = part.data_ptr()
                a.partials_bytes = nbytes
            table = self._upload(one)
            a.segs = table.data_ptr()
            check(binding.tf_check_segments(a, one), "tf_check_segments")
            check(binding.tf_attn_rows(a, st), "tf_attn_rows")
            if self.split_keys > 0:
                check(binding.tf_attn_merge(a, st), "tf_attn_merge")
            keep.append((table, part))
        torch.cuda.synchronize(self.device)
        return to_host_u16(out)

    def put_args(self, k_new: torch.Tensor, v_new: torch.Tensor, copy: int = 0) -> binding.tf_put_args:
        """tf_kv_put arguments writing packed new rows into this workload's storage."""
        w = self.w
        a = binding.tf_put_args()
        a.kind = self.kind
        a.n_segments = len(w.segments)
        a.total_rows = w.total_rows
        a.max_rows = w.max_rows
        a.n_kv_heads = w.n_kv_heads
        a.head_dim = w.head_dim
        a.page_size = w.page_size if w.kind == "paged" else 0
        a.pool_pages = w.pool_pages if w.kind == "paged" else 0
        a.segs = self.tables[copy].data_ptr()
        a.k_new = k_new.data_ptr()
        a.v_new = v_new.data_ptr()
        a.err = self.err.data_ptr()
        return a

    def kv_put(self, k_new: np.ndarray, v_new: np.ndarray, copy: int = 0) -> None:
        """tf_kv_put of packed new rows [total_rows][Hkv][D] (bf16 bits) into copy `copy`."""
        kn, vn = _dev(k_new, self.device), _dev(v_new, self.device)
        st = torch.cuda.current_stream(self.device).cuda_stream
        check(binding.tf_kv_put(self.put_args(kn, vn, copy), st), "tf_kv_put")
        torch.cuda.synchronize(self.device)

    def storage(self, copy: int = 0):
        """Host copies of (K, V) storage: the pools, or lists of per-stream buffers."""
        torch.cuda.synchronize(self.device)
        k = [to_host_u16(x) for x in self.k_store[copy]]
        v = [to_host_u16(x) for x in self.v_store[copy]]
        if self.w.kind == "paged":
            return k[0], v[0]
        return k, v

    def partial_records(self) -> np.ndarray:
        """The partials workspace as [records][head_dim + 4] float32 (host copy)."""
        torch.cuda.synchronize(self.device)
        d = self.w.head_dim
        n = self.partials_bytes // ((d + 4) * 4)
        return self.partials[: n * (d + 4)].view(n, d + 4).cpu().numpy()


def argmax(logits: np.ndarray, device="cuda:0", vocab: Optional[int] = None):
    """Run tf_argmax on host bf16 logits [rows][stride]; returns (ids, flags)."""
    dev = torch.device(device)
    rows, stride = logits.shape
    vocab = stride if vocab is None else vocab
    x = _dev(logits, dev)
    ids = torch.full((rows,), -1, dtype=torch.int32, device=dev)
    flags = torch.full((rows,), 7, dtype=torch.uint8, device=dev)
    nbytes = binding.tf_argmax_workspace_bytes(rows, vocab)
    ws = torch.zeros(max(nbytes, 8) // 8 + 1, dtype=torch.int64, device=dev)   # zero before first use
    st = torch.cuda.current_stream(dev).cuda_stream
    check(binding.tf_argmax(x.data_ptr(), rows, vocab, stride, ids.data_ptr(), flags.data_ptr(),
                            ws.data_ptr(), nbytes, st), "tf_argmax")
    torch.cuda.synchronize(dev)
    return ids.cpu().numpy(), flags.cpu().numpy()


class DeviceState:
    """Device copies of per-layer pools and kept-state buffers, and the
    tf_state_save / tf_state_restore calls on them.

    ``pools`` and ``states`` are lists of (K, V) host arrays per layer
    (bf16 bits, [pages][Hkv][P][D]); ``pages`` is the stream's page list.
    """

    def __init__(self, pools, states, pages, at: int, device="cuda:0"):
        self.device = torch.device(device)
        self.pk = [_dev(k, self.device) for k, _ in pools]
        self.pv = [_dev(v, self.device) for _, v in pools]
        self.sk = [_dev(k, self.device) for k, _ in states]
        self.sv = [_dev(v, self.device) for _, v in states]
        self.pool_pages, self.hkv, self.page_size, self.head_dim = pools[0][0].shape
        self.at = at
        self.err = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.set_pages(pages)
        table = (binding.tf_state_layer * len(pools))()
        for i in range(len(pools)):
            table[i].pool_k = self.pk[i].data_ptr()
            table[i].pool_v = self.pv[i].data_ptr()
            table[i].state_k = self.sk[i].data_ptr()
            table[i].state_v = self.sv[i].data_ptr()
        self.host_layers = table
        raw = bytes(ctypes.string_at(ctypes.addressof(table), ctypes.sizeof(table)))
        self.layers = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(self.device)

    def set_pages(self, pages) -> None:
        self.n_pages = len(pages)
        self.pages = _dev(np.ascontiguousarray(pages, dtype=np.int32), self.device)

    def args(self) -> binding.tf_state_args:
        a = binding.tf_state_args()
        a.n_layers = len(self.pk)
        a.n_kv_heads = self.hkv
        a.head_dim = self.head_dim
        a.page_size = self.page_size
        a.pool_pages = self.pool_pages
        a.at = self.at
        a.n_pages = self.n_pages
        a.pages = self.pages.data_ptr()
        a.layers = self.layers.data_ptr()
        a.err = self.err.data_ptr()
        return a

    def save(self, stream: Optional[int] = None) -> None:
        st = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        check(binding.tf_state_save(self.args(), st), "tf_state_save")

    def restore(self, stream: Optional[int] = None) -> None:
        st = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        check(binding.tf_state_restore(self.args(), st), "tf_state_restore")

    def host(self):
        """(pools, states) as lists of (K, V) host arrays."""
        torch.cuda.synchronize(self.device)
        pools = [(to_host_u16(k), to_host_u16(v)) for k, v in zip(self.pk, self.pv)]
        states = [(to_host_u16(k), to_host_u16(v)) for k, v in zip(self.sk, self.sv)]
        return pools, states

    def error_word(self) -> int:
        torch.cuda.synchronize(self.device)
        return int(self.err.item())

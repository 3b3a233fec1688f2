"""The C ABI: every declared symbol is exported; host-side checks (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

from stream_paged_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tf_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\**\s*(tf_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("tf_attn_rows", "tf_attn_merge", "tf_argmax"):
        assert must in names
    assert set(names) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = binding.load()
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (tf_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


STRUCTS = ("tf_segment", "tf_attn_args", "tf_put_args", "tf_state_layer", "tf_state_args")


def test_header_compiles_as_c_and_struct_layouts_match():
    # every field's offset and every struct's size, as a C compiler lays
    # them out, against the ctypes declarations of the binding
    lines = []
    for name in STRUCTS:
        cls = getattr(binding, name)
        lines.append(f'printf("{name} size %zu\\n", sizeof({name}));')
        for field, _ in cls._fields_:
            lines.append(f'printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    src = ("#include \"tf_attn.h\"\n#include <stdio.h>\n#include <stddef.h>\n"
           "int main(void){" + "".join(lines) + " return 0;}\n")
    tmp = os.path.join(ROOT, "_build")
    os.makedirs(tmp, exist_ok=True)
    c = os.path.join(tmp, "hdr_check.c")
    exe = os.path.join(tmp, "hdr_check")
    open(c, "w").write(src)
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                           c, "-o", exe])
    got = {}
    for line in subprocess.check_output([exe], text=True).splitlines():
        name, what, val = line.split()
        got[(name, what)] = int(val)
    for name in STRUCTS:
        cls = getattr(binding, name)
        assert got[(name, "size")] == ctypes.sizeof(cls), name
        for field, _ in cls._fields_:
            assert got[(name, field)] == getattr(cls, field).offset, (name, field)


def test_strerror_names_every_code():
    for code in (0, -1, -2, -3, -4, -5):
        assert binding.tf_strerror(code) != "unknown error"
    assert binding.tf_strerror(-99) == "unknown error"


def _segs(specs):
    arr = (binding.tf_segment * len(specs))()
    for i, (n, kc) in enumerate(specs):
        arr[i].n_rows, arr[i].key_count = n, kc
    return arr


def test_plan_partials_offsets_and_bytes():
    segs = _segs([(1, 512), (3, 513), (2, 40)])
    rc, nbytes = binding.tf_plan_partials(segs, 4, 128, 512)
    assert rc == binding.TF_OK
    # splits: 1, 2, 1; records: 1*4*1, 3*4*2, 2*4*1
    assert [s.partial_offset for s in segs] == [0, 4, 28]
    assert nbytes == (4 + 24 + 8) * (128 + 4) * 4


@pytest.mark.parametrize("args,rc", [
    (dict(head_dim=64, split=0), binding.TF_E_UNSUPPORTED),
    (dict(head_dim=96, split=512), binding.TF_E_UNSUPPORTED),
    (dict(head_dim=128, split=100), binding.TF_E_UNSUPPORTED),
    (dict(head_dim=128, hq=0), binding.TF_E_INVALID),
])
def test_plan_partials_refusals(args, rc):
    segs = _segs([(1, 10)])
    got, _ = binding.tf_plan_partials(segs, args.get("hq", 4), args["head_dim"],
                                      args.get("split", 512))
    assert got == rc


def _args(**kw):
    a = binding.tf_attn_args()
    a.kind = kw.get("kind", binding.TF_KV_PAGED)
    a.n_segments = kw.get("n_segments", 1)
    a.total_rows = kw.get("total_rows", 2)
    a.max_rows = kw.get("max_rows", 2)
    a.max_keys = kw.get("max_keys", 100)
    a.min_rows = kw.get("min_rows", 0)
    a.n_q_heads = kw.get("hq", 8)
    a.n_kv_heads = kw.get("hkv", 2)
    a.head_dim = kw.get("d", 128)
    a.page_size = kw.get("page_size", 32)
    a.pool_pages = kw.get("pool_pages", 10)
    a.split_keys = kw.get("split", 0)
    a.scale = kw.get("scale", 0.088)
    fake = 0x10000  # 16-byte aligned stand-in addresses: nothing is dereferenced
    a.segs = kw.get("segs", fake)
    a.q = kw.get("q", fake)
    a.out = kw.get("out", fake)
    a.partials = kw.get("partials", None)
    a.partials_bytes = kw.get("partials_bytes", 0)
    a.mask = kw.get("mask", binding.TF_MASK_CAUSAL)
    a.tree = kw.get("tree", None)
    return a


@pytest.mark.parametrize("kw,rc", [
    (dict(d=96), binding.TF_E_UNSUPPORTED),
    (dict(page_size=48), binding.TF_E_UNSUPPORTED),
    (dict(page_size=16), binding.TF_E_UNSUPPORTED),
    (dict(split=100), binding.TF_E_UNSUPPORTED),
    (dict(hq=6, hkv=4), binding.TF_E_INVALID),
    (dict(kind=7), binding.TF_E_INVALID),
    (dict(n_segments=-1), binding.TF_E_INVALID),
    (dict(q=None), binding.TF_E_INVALID),
    (dict(q=0x10008), binding.TF_E_INVALID),          # misaligned
    (dict(max_keys=1, max_rows=2), binding.TF_E_INVALID),
    (dict(pool_pages=0), binding.TF_E_INVALID),
    (dict(split=512), binding.TF_E_WORKSPACE),        # partials missing
    (dict(min_rows=3, max_rows=2), binding.TF_E_INVALID),
    (dict(min_rows=-1), binding.TF_E_INVALID),
    (dict(scale=0.0), binding.TF_E_INVALID),
    (dict(scale=-0.1), binding.TF_E_INVALID),
    (dict(scale=float("inf")), binding.TF_E_INVALID),
    (dict(scale=float("nan")), binding.TF_E_INVALID),
    (dict(mask=3), binding.TF_E_INVALID),
    (dict(mask=-1), binding.TF_E_INVALID),
    (dict(mask=binding.TF_MASK_TREE), binding.TF_E_INVALID),                    # tree masks missing
    (dict(mask=binding.TF_MASK_TREE, tree=0x50004), binding.TF_E_INVALID),      # misaligned
    (dict(mask=binding.TF_MASK_TREE, tree=0x50000, max_rows=65, max_keys=100),
     binding.TF_E_INVALID),                                                     # more than 64 rows
    # grids past the launch limit are refused before any launch
    (dict(split=32, max_keys=2**31 - 1, partials=0x10000, partials_bytes=1 << 40), binding.TF_E_UNSUPPORTED),
    (dict(hq=2**30, hkv=2**30), binding.TF_E_UNSUPPORTED),
    (dict(hq=2**30, hkv=1, max_rows=2, max_keys=100), binding.TF_E_UNSUPPORTED),   # matrix-core grid
])
def test_rows_refuses_bad_scalars_without_launching(kw, rc):
    # stream 0 and fake pointers: a refused call must return before any launch
    assert binding.tf_attn_rows(_args(**kw), 0) == rc


def test_tree_mask_limits_on_the_host_table():
    t = _host_table([(4, 0, 0, 64, 100), (4, 0, 64, 1, 40)])
    a = _args(total_rows=65, n_segments=2, max_rows=64, mask=binding.TF_MASK_TREE, tree=0x50000)
    assert binding.tf_check_segments(a, t) == binding.TF_OK
    big = _host_table([(4, 0, 0, 65, 100)])
    a = _args(total_rows=65, max_rows=65, mask=binding.TF_MASK_TREE, tree=0x50000)
    assert binding.tf_check_segments(a, big) == binding.TF_E_INVALID
    a.mask = binding.TF_MASK_FULL
    assert binding.tf_check_segments(a, big) == binding.TF_OK


def test_merge_needs_split_partials():
    assert binding.tf_attn_merge(_args(split=0), 0) == binding.TF_E_INVALID
    assert binding.tf_attn_merge(_args(split=512), 0) == binding.TF_E_WORKSPACE


def test_empty_launch_is_ok():
    assert binding.tf_attn_rows(_args(n_segments=0, segs=None, q=None, out=None), 0) == 0


def _host_table(specs, kind=binding.TF_KV_PAGED):
    arr = (binding.tf_segment * len(specs))()
    for i, sp in enumerate(specs):
        e = arr[i]
        e.k = e.v = 0x20000
        e.pages = 0x30000 if kind == binding.TF_KV_PAGED else None
        e.capacity, e.first, e.row_offset, e.n_rows, e.key_count = sp
        e.partial_offset = 0
    return arr


def test_check_segments_host_rules():
    ok = _host_table([(4, 0, 0, 1, 100), (2, 0, 1, 2, 40)])
    assert binding.tf_check_segments(_args(total_rows=3, n_segments=2), ok) == binding.TF_OK
    past = _host_table([(3, 0, 0, 1, 100)])        # 3 pages of 32 < 100 keys
    assert binding.tf_check_segments(_args(total_rows=1), past) == binding.TF_E_PAST_PAGES
    overlap = _host_table([(4, 0, 0, 2, 100), (4, 0, 1, 1, 40)])
    assert binding.tf_check_segments(_args(total_rows=3, n_segments=2), overlap) == binding.TF_E_INVALID
    too_many_rows = _host_table([(4, 0, 0, 3, 100)])
    assert binding.tf_check_segments(_args(total_rows=3, max_rows=2), too_many_rows) == binding.TF_E_INVALID
    # a segment with fewer rows than the min_rows hint
    assert binding.tf_check_segments(_args(total_rows=3, n_segments=2, min_rows=2), ok) == binding.TF_E_INVALID
    assert binding.tf_check_segments(_args(total_rows=3, n_segments=2, min_rows=1), ok) == binding.TF_OK
    ring_bad = _host_table([(50, 50, 0, 1, 40)], kind=binding.TF_KV_RING)
    assert binding.tf_check_segments(_args(kind=binding.TF_KV_RING, total_rows=1), ring_bad) == binding.TF_E_INVALID
    ring_past = _host_table([(30, 3, 0, 1, 40)], kind=binding.TF_KV_RING)
    assert binding.tf_check_segments(_args(kind=binding.TF_KV_RING, total_rows=1), ring_past) == binding.TF_E_PAST_PAGES


def test_check_segments_storage_limit():
    # one kv head's run of a CONTIG / RING buffer must stay below 4 GiB (the
    # kernels address it with 32-bit offsets): 2^23 slots at D 256 is 4 GiB
    for kind in (binding.TF_KV_CONTIG, binding.TF_KV_RING):
        big = _host_table([(1 << 23, 0, 0, 1, 40)], kind=kind)
        a = _args(kind=kind, total_rows=1)
        a.head_dim = 256
        assert binding.tf_check_segments(a, big) == binding.TF_E_UNSUPPORTED
        fits = _host_table([((1 << 23) - 1, 0, 0, 1, 40)], kind=kind)
        assert binding.tf_check_segments(a, fits) == binding.TF_OK


def test_check_segments_workspace():
    t = _host_table([(4, 0, 0, 1, 100)])
    t[0].partial_offset = 0
    a = _args(total_rows=1, split=32, partials=0x40000, partials_bytes=(128 + 4) * 4 * 8 * 3)
    # 100 keys at 32 a split = 4 splits x 8 heads = 32 records needed, 24 given
    assert binding.tf_check_segments(a, t) == binding.TF_E_WORKSPACE
    a.partials_bytes = (128 + 4) * 4 * 32
    assert binding.tf_check_segments(a, t) == binding.TF_OK


def test_argmax_refusals():
    assert binding.tf_argmax(0x100, 2, 0, 10, 0x200, 0x300, 0x400, 10 ** 6, 0) == binding.TF_E_INVALID
    assert binding.tf_argmax(0x100, 2, 10, 5, 0x200, 0x300, 0x400, 10 ** 6, 0) == binding.TF_E_INVALID
    assert binding.tf_argmax(0x100, 2, 10, 10, 0x200, 0x300, 0x400, 1, 0) == binding.TF_E_WORKSPACE
    assert binding.tf_argmax(0, 0, 10, 10, 0, 0, 0, 0, 0) == binding.TF_OK   # no rows: nothing to do
    assert binding.tf_argmax_workspace_bytes(32, 128000) == 32 * 16     # one 16-byte slot a row
    # a row's chunk count must fit 16 bits: at most 65535 chunks of 16384 logits
    big = 65536 * 16384
    assert binding.tf_argmax(0x100, 1, big, big, 0x200, 0x300, 0x400, 16, 0) == binding.TF_E_UNSUPPORTED


def test_put_refusals():
    # refused before any launch: no GPU needed
    a = binding.tf_put_args()
    a.kind = binding.TF_KV_PAGED
    a.n_segments, a.total_rows, a.max_rows, a.n_kv_heads, a.head_dim = 1, 1, 1, 2, 96
    a.page_size, a.pool_pages = 32, 4
    a.segs = a.k_new = a.v_new = 0x10000
    assert binding.tf_kv_put(a, 0) == binding.TF_E_UNSUPPORTED
    a.head_dim, a.page_size = 128, 48
    assert binding.tf_kv_put(a, 0) == binding.TF_E_UNSUPPORTED
    a.page_size, a.k_new = 32, 0x10008
    assert binding.tf_kv_put(a, 0) == binding.TF_E_INVALID


def _state_args(**kw):
    a = binding.tf_state_args()
    a.n_layers = kw.get("n_layers", 2)
    a.n_kv_heads = kw.get("hkv", 8)
    a.head_dim = kw.get("d", 64)
    a.page_size = kw.get("page_size", 512)
    a.pool_pages = kw.get("pool_pages", 100)
    a.at = kw.get("at", 1000)
    a.n_pages = kw.get("n_pages", 2)
    a.pages = kw.get("pages", 0x10000)
    a.layers = kw.get("layers", 0x20000)
    a.err = None
    return a


@pytest.mark.parametrize("kw,rc", [
    (dict(d=96), binding.TF_E_UNSUPPORTED),
    (dict(page_size=48), binding.TF_E_UNSUPPORTED),
    (dict(page_size=2048), binding.TF_E_UNSUPPORTED),
    (dict(n_layers=-1), binding.TF_E_INVALID),
    (dict(hkv=0), binding.TF_E_INVALID),
    (dict(at=-1), binding.TF_E_INVALID),
    (dict(pool_pages=0), binding.TF_E_INVALID),
    (dict(at=1025, n_pages=2), binding.TF_E_PAST_PAGES),
    (dict(pages=None), binding.TF_E_INVALID),
    (dict(layers=None), binding.TF_E_INVALID),
    (dict(at=0, pages=None, layers=None), binding.TF_OK),           # nothing to copy
    (dict(n_layers=0, pages=None, layers=None), binding.TF_OK),
])
def test_state_copy_refusals(kw, rc):
    # refused (or empty) before any launch: no GPU needed
    assert binding.tf_state_save(_state_args(**kw), 0) == rc
    assert binding.tf_state_restore(_state_args(**kw), 0) == rc

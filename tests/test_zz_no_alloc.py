"""tf_attn_static: the entry point that allocates nothing.

Its output must equal the workspace path's (tf_attn_rows + tf_attn_merge with
a caller workspace) byte for byte, on two calls in a row, the second with a
smaller input, since both run the same kernels; the smaller case is also
held to the oracle bar (2e-3).  It refuses a caller workspace and a planned
size beyond its array without launching.
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from stream_paged_attention_amd import binding, launch, synth

pytestmark = pytest.mark.gpu


def _workspace_path(dw):
    dw.out.fill_(0x7FA5)
    dw.run()
    assert dw.error_word() == 0
    return dw.output().copy()


def _static_path(dw):
    a = dw.args(0)
    a.partials = None
    a.partials_bytes = dw.partials_bytes
    dw.out.fill_(0x7FA5)
    rc = binding.tf_attn_static(a, torch.cuda.current_stream(dw.device).cuda_stream)
    assert rc == binding.TF_OK, binding.tf_strerror(rc)
    assert dw.error_word() == 0
    return dw.output().copy()


def test_static_partials_match_the_workspace_path(gpu):
    big = synth.make_synthetic("decode16")
    small = synth.make_workload("static-small", synth.KIND_PAGED, 8, 2, 128, [1, 6, 1], [900, 300, 70],
                                seed=51, page_size=32, pool_pages=60, split_keys=128)
    dbig = launch.DeviceWorkload(big, gpu)
    dsmall = launch.DeviceWorkload(small, gpu)
    assert dsmall.partials_bytes < dbig.partials_bytes <= binding.TF_STATIC_PARTIALS_BYTES
    want_big = _workspace_path(dbig)
    want_small = _workspace_path(dsmall)
    # two calls in a row on the shared array, the second with a smaller input
    got_big = _static_path(dbig)
    got_small = _static_path(dsmall)
    assert np.array_equal(got_big, want_big), "decode16: static partials differ from the workspace path"
    assert np.array_equal(got_small, want_small), "small: static partials differ from the workspace path"
    ref = oracle.attn_workload(small)
    got = synth.bf16_bits_to_f32(got_small).astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 2e-3 + 2.0 ** -8 * np.max(np.abs(ref))


def test_static_refusals(gpu):
    w = synth.make_workload("static-ref", synth.KIND_PAGED, 8, 2, 128, [1], [300], seed=52,
                            page_size=32, pool_pages=20, split_keys=128)
    dw = launch.DeviceWorkload(w, gpu)
    st = torch.cuda.current_stream(gpu).cuda_stream
    a = dw.args(0)                      # a caller workspace: refused
    assert binding.tf_attn_static(a, st) == binding.TF_E_INVALID
    a.partials = None
    a.partials_bytes = binding.TF_STATIC_PARTIALS_BYTES + 4
    assert binding.tf_attn_static(a, st) == binding.TF_E_WORKSPACE
    a.partials_bytes = dw.partials_bytes
    assert binding.tf_attn_static(a, st) == binding.TF_OK
    assert dw.error_word() == 0

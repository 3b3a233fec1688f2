"""Guard regions around every buffer the kernels write.

The pages' drafter gate (TensorFold PR #1562, its Gate section) repeats the
shared-round kernels with guard regions around their outputs and requires
them untouched.  Here `out`, the split partials, the argmax ids / flags and
the argmax workspace each sit inside a larger allocation whose 4 KiB (or
more) on both sides hold a NaN bit pattern no kernel writes (0x7FA5 for bf16,
0x7FA5A5A5 for fp32 and int32, 0xA5 for bytes).  After all five synthetic
workloads (attention and, where they have logits, the argmax) the guards must
still hold that pattern, and inside the buffers no element may still hold it
(every element is written).
"""
import numpy as np
import pytest
import torch

from oracle import oracle
from stream_paged_attention_amd import binding, launch, synth

pytestmark = pytest.mark.gpu

GUARD_BYTES = 4096
PAT16 = 0x7FA5
PAT32 = 0x7FA5A5A5
PAT8 = 0xA5


def guarded(n, dtype, pattern, device):
    """(whole, inner): a tensor of n elements with GUARD_BYTES of pattern on both sides."""
    g = GUARD_BYTES // torch.empty(0, dtype=dtype).element_size()
    whole = torch.full((n + 2 * g,), pattern, dtype=dtype, device=device)
    return whole, whole[g:g + n], g


def guards_intact(whole, g, pattern):
    h = whole.cpu().numpy()
    return bool(np.all(h[:g] == pattern) and np.all(h[-g:] == pattern))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_guards_untouched(gpu, name):
    print(f"guards: {name}", flush=True)
    w = synth.make_synthetic(name)
    dw = launch.DeviceWorkload(w, gpu)
    out_whole, out_in, g_out = guarded(dw.out.numel(), torch.int16, PAT16, gpu)
    dw.out = out_in.view(dw.out.shape)
    part_whole = None
    if dw.partials is not None:
        n = dw.partials.numel()
        part_whole, part_in, g_part = guarded(n, torch.int32, PAT32, gpu)
        dw.partials = part_in.view(torch.float32)
    assert dw.check_table() == binding.TF_OK
    for _ in range(2):
        dw.run()
    torch.cuda.synchronize()
    assert dw.error_word() == 0
    assert guards_intact(out_whole, g_out, PAT16), f"{name}: a write landed next to out"
    assert not np.any(launch.to_host_u16(dw.out) == PAT16), f"{name}: output elements left unwritten"
    if part_whole is not None:
        assert guards_intact(part_whole, g_part, PAT32), f"{name}: a write landed next to the partials"
        recs = dw.partial_records()
        # m, l and o of every planned record are written (fields 2..3 are unused)
        bits = np.concatenate([recs[:, :2], recs[:, 4:]], axis=1).view(np.uint32)
        assert not np.any(bits == PAT32), f"{name}: partial records left unwritten"

    if w.logits is not None:
        rows, vocab = w.logits.shape
        x = launch._dev(w.logits, gpu)
        ids_whole, ids_in, g_ids = guarded(rows, torch.int32, PAT32, gpu)
        fl_whole, fl_in, g_fl = guarded(rows, torch.uint8, PAT8, gpu)
        nbytes = binding.tf_argmax_workspace_bytes(rows, vocab)
        ws_whole, ws_in, g_ws = guarded(max(nbytes, 1), torch.uint8, PAT8, gpu)
        ws_in.zero_()   # the workspace holds zeros before its first use
        st = torch.cuda.current_stream(gpu).cuda_stream
        for _ in range(2):
            rc = binding.tf_argmax(x.data_ptr(), rows, vocab, vocab, ids_in.data_ptr(), fl_in.data_ptr(),
                                   ws_in.data_ptr(), nbytes, st)
            assert rc == binding.TF_OK
        torch.cuda.synchronize()
        assert guards_intact(ids_whole, g_ids, PAT32), f"{name}: a write landed next to the argmax ids"
        assert guards_intact(fl_whole, g_fl, PAT8), f"{name}: a write landed next to the argmax flags"
        assert guards_intact(ws_whole, g_ws, PAT8), f"{name}: a write landed next to the argmax workspace"
        assert not ws_in.cpu().numpy().any(), f"{name}: the argmax workspace was not left zero"
        rids, rflags = oracle.argmax(w.logits)
        np.testing.assert_array_equal(ids_in.cpu().numpy(), rids)
        np.testing.assert_array_equal(fl_in.cpu().numpy(), rflags)

"""pisa_select_prefill_noalloc (the selection on the library's static device scratch)
against pisa_select_prefill with a caller workspace: identical outputs on two calls in a
row, the second on a smaller problem, and a problem past the scratch size rejected on the
host."""
import numpy as np
import pytest

from block_selection_pyramid_amd import synth

pytestmark = pytest.mark.gpu


def _run(torch, pisa, w):
    p = pisa.Problem(**w.shape())
    q, k, _ = synth.make_inputs(w)
    qd = torch.from_numpy(q).view(torch.bfloat16).cuda()
    kd = torch.from_numpy(k).view(torch.bfloat16).cuda()
    pyr = pisa.build_pyramid(p, kd)
    ref_i, ref_s = pisa.select_prefill(p, qd, kd, pyr)
    shape = ref_i.shape
    out_i = torch.full(shape, -7, dtype=torch.int32, device="cuda")
    out_s = torch.full(shape, 7.0, dtype=torch.float32, device="cuda")
    pisa.select_prefill_noalloc(p, qd, kd, pyr, out_i, out_s)
    torch.cuda.synchronize()
    return ref_i.cpu().numpy(), ref_s.cpu().numpy(), out_i.cpu().numpy(), out_s.cpu().numpy()


def test_noalloc_matches_workspace_call_twice():
    import torch
    from block_selection_pyramid_amd import pisa
    assert torch.cuda.is_available()
    pisa.load()
    # first call: 78K tokens, 16/4 heads, K = 8 (61 MiB of workspace; level 2 gathered);
    # second: a smaller, ragged problem whose lists and counters reuse the same scratch
    big = synth.custom(name="noalloc-64k", batch=1, seq_len=65536 + 64 * 200, n_q_heads=16, n_kv_heads=4,
                       head_dim=128, top_k=8, seed=41, needles=64)
    small = synth.custom(name="noalloc-small", batch=2, seq_len=5000 + 13, n_q_heads=8, n_kv_heads=2,
                         head_dim=128, top_k=5, seed=42, needles=8)
    for w in (big, small):
        p = pisa.Problem(**w.shape())
        assert pisa.prefill_workspace_min_bytes(p) <= pisa.NOALLOC_SCRATCH_BYTES
        print("[noalloc]", w.name, "N=%d: launching" % w.seq_len, flush=True)
        ri, rs, oi, os_ = _run(torch, pisa, w)
        assert np.array_equal(ri, oi), w.name
        assert np.array_equal(rs.view(np.int32), os_.view(np.int32)), w.name


def test_noalloc_rejects_problems_past_the_scratch():
    import torch
    from block_selection_pyramid_amd import pisa
    pisa.load()
    p = pisa.Problem(1, 262144, 16, 4, 128, 64, 8, 2)
    assert pisa.prefill_workspace_min_bytes(p) > pisa.NOALLOC_SCRATCH_BYTES
    # host-side rejection: no kernel runs, so tiny placeholder tensors suffice for the shapes
    # the binding checks are bypassed by calling the C entry point directly
    lib = pisa.load()
    import ctypes
    buf = torch.empty(256, dtype=torch.uint8, device="cuda")
    ptr = buf.data_ptr()
    rc = lib.pisa_select_prefill_noalloc(ctypes.byref(p.c()), ptr, ptr, ptr, ptr, ptr, None)
    assert rc == 3  # PISA_ERR_WORKSPACE

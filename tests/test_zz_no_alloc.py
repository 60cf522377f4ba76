"""The Split-K forward without allocation (flex_attn_fwd_splitk_noalloc)
against the Split-K forward with a caller workspace, through the C ABI.

Both run the same split and merge kernels with the same part count, so their
outputs must be identical bit for bit; two calls in a row (the second on a
smaller problem) check that the shared static scratch needs no clearing, the
device's free memory must not move across a call once the library is loaded,
and a problem whose partial states exceed the scratch is refused before any
launch."""
import numpy as np
import pytest
import torch

import mask_planned_block_amd as mpb
import workloads as W
from tests import gpu_support as G

pytestmark = pytest.mark.gpu


def _run_both(w, num_splits):
    print("CASE no_alloc", w.name, w.total_q, w.total_k, num_splits, flush=True)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    kw = dict(scale=w.scale, softcap=w.softcap if w.softcap > 0 else None,
              alibi_slopes=d["slopes"], alibi_before_softcap=w.alibi_before_softcap)
    sp = num_splits if num_splits else mpb.flex_attn_fwd_num_splits(plan)
    ws = torch.empty(max(mpb.flex_attn_fwd_splitk_workspace_size(plan, sp), 256),
                     dtype=torch.uint8, device="cuda")
    o_ref, l_ref = mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], workspace=ws,
                                     num_splits=sp, **kw)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((w.heads_q, w.total_q), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    mpb.flex_attn_fwd_splitk_noalloc(plan, d["q"], d["k"], d["v"], out, lse, num_splits=sp,
                                     **kw)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return plan, sp, (o_ref, l_ref), (out, lse), free0, free1


def test_noalloc_splitk_matches_workspace_splitk():
    # warm the static scratch up (first use on this device loads the library
    # code object that holds it)
    w0 = W.make("chunk_long_kv", small=True)
    _run_both(w0, 2)
    # full long-K chunk at the library's part count, then a smaller problem
    # with another part count: the second call reuses what the first left
    for w, sp in ((W.make("chunk_long_kv"), 0), (W.make("chunk_long_kv", small=True), 3)):
        plan, used, ref, got, free0, free1 = _run_both(w, sp)
        assert used > 1
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1]), (w.name, used)
        assert free0 == free1, "the no-allocation call changed the device's free memory"


def test_noalloc_refuses_oversized_partial_states():
    # 64 parts of a 16 x 4096-row problem at d = 128: 64 * 4096 * 16 * 128 * 4 B
    # = 2 GiB of partial states, far above the static scratch
    S = 4096
    mf = np.full((1, 1, S), S, np.int32)
    w = W.custom(mf, batch=1, seqlen_q=S, seqlen_k=S, heads_q=16, head_dim=128,
                 dtype=W.DTYPE_BF16, seed=3)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    out = torch.empty_like(d["q"])
    lse = torch.empty((w.heads_q, w.total_q), dtype=torch.float32, device="cuda")
    with pytest.raises(mpb.MPBError) as ei:
        mpb.flex_attn_fwd_splitk_noalloc(plan, d["q"], d["k"], d["v"], out, lse, num_splits=64)
    assert ei.value.name == "MPB_ERR_WORKSPACE"

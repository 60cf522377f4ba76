"""GPU tests of plans built with a deferred header read-back.

A deferred build ("Flex Attention Mask Plan Design" §4.5 reads the header
back once; here that read is moved from the build to the first call that
needs it) runs the same planner kernels, so its plan arrays must equal those
of a build that waited for the header, and a forward launched before anything
read the header -- the upper bound of workgroups, each reading the task count
on the device -- must equal the forward over the waited-for plan bit for bit
(same kernels, same tile lists, same order).  Endpoint errors found on the GPU
surface at the first call that reads the header; a forward launched on such a
plan writes nothing.
"""
import numpy as np
import pytest
import torch

import mask_planned_block_amd as mpb
import oracle
import workloads as W
from tests import gpu_support as G

pytestmark = pytest.mark.gpu

NAMES = ["tiny_causal", "window_sink", "varlen_doc", "block_sparse", "prefix_softcap",
         "chunk_long_kv"]


@pytest.fixture(scope="module", autouse=True)
def require_gpu():
    assert torch.cuda.is_available(), "no GPU visible to a GPU test"


def _case(case, **kw):
    print("CASE", case, kw, flush=True)


def _same_exports(a, b):
    for key in ("cu_rows", "seqdesc", "p_off", "p_idx", "p_masks", "f_off", "f_idx",
                "work_desc", "section_off", "header", "launch"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("name", NAMES)
def test_deferred_forward_equals_waited(name):
    w = W.make(name, small=True)
    _case("deferred", name=name)
    d = G.device_inputs(w)
    lazy = G.build_plan(w, d, defer_header=True)
    o_lazy, l_lazy = G.run_attention(w, d, lazy)     # before anything reads the header
    o_abl, l_abl = G.run_attention(w, d, lazy, force_partial=True)
    ref = G.build_plan(w, d)
    o_ref, l_ref = G.run_attention(w, d, ref)
    torch.cuda.synchronize()
    assert torch.equal(o_lazy, o_ref) and torch.equal(l_lazy, l_ref)
    assert torch.equal(o_abl, o_ref) and torch.equal(l_abl, l_ref)
    info = lazy.info
    assert info.build_mode == mpb.BUILD_SINGLE_PASS_DEFERRED
    assert ref.info.build_mode == mpb.BUILD_SINGLE_PASS
    assert list(info.header) == list(ref.info.header)
    assert info.num_tasks == ref.info.num_tasks and info.rows_total == ref.info.rows_total
    ge = lazy.export()
    _same_exports(ge, ref.export())
    pl = info.problem
    op = oracle.build_plan(w, pl.tile_q // info.signature.pack_gqa, pl.tile_k)
    G.compare_plan(ge, op)


def _gqa_workload(kind):
    """Deferred builds small enough that every item ranks its own row (at most
    256 mask rows) with Q heads grouped over fewer KV heads.  "shared": one
    window+sink mask, 24 Q heads on 12 KV heads over 3 samples, so that
    sample 1's KV heads run past 16 in the snake order of the sections
    ((b * Hk) mod 16 = 0, 12, 8).  "per_head": a different window per Q head
    (mask heads = Q heads), 8 Q heads on 4 KV heads."""
    if kind == "shared":
        return W.window_sink(seed=3, batch=3, heads=24, heads_k=12, seqlen=384, sink=32,
                             window=100)
    batch, seqlen, hq, hk = 3, 384, 8, 4
    ql = np.arange(seqlen, dtype=np.int64)
    mf = np.stack([np.tile(W.window_sink_endpoints(ql, 16, 40 + 37 * h), (1, batch))
                   for h in range(hq)])
    return W.custom(mf, layout=W.LAYOUT_BSHD, batch=batch, seqlen_q=seqlen, seqlen_k=seqlen,
                    heads_q=hq, heads_k=hk, head_dim=128, dtype=W.DTYPE_BF16, seed=4,
                    name="per_head_windows")


@pytest.mark.parametrize("kind", ["shared", "per_head"])
def test_deferred_ranked_schedule_gqa(kind):
    w = _gqa_workload(kind)
    _case("deferred gqa", kind=kind, hq=w.heads_q, hk=w.heads_k, hmask=w.mask_heads)
    d = G.device_inputs(w)
    lazy = G.build_plan(w, d, defer_header=True)
    o_lazy, l_lazy = G.run_attention(w, d, lazy)
    ref = G.build_plan(w, d)
    o_ref, l_ref = G.run_attention(w, d, ref)
    torch.cuda.synchronize()
    assert torch.equal(o_lazy, o_ref) and torch.equal(l_lazy, l_ref)
    info = lazy.info
    assert info.build_mode == mpb.BUILD_SINGLE_PASS_DEFERRED
    assert list(info.header) == list(ref.info.header)
    ge = lazy.export()
    _same_exports(ge, ref.export())
    pl = info.problem
    op = oracle.build_plan(w, pl.tile_q // info.signature.pack_gqa, pl.tile_k)
    G.compare_plan(ge, op)
    if info.signature.pack_gqa == 1:   # a packed plan's tasks follow the packed view
        G.check_schedule(w, ge, pl.tile_q)


def test_deferred_large_plan_schedules_in_its_own_launch():
    """Past the fused schedule's size (block-sparse: 24 x 64 items) a deferred
    build keeps its schedule launch; its plan and forward equal those of the
    build that read the header back."""
    w = W.make("block_sparse")
    _case("deferred_large")
    d = G.device_inputs(w)
    lazy = G.build_plan(w, d, defer_header=True)
    o_lazy, l_lazy = G.run_attention(w, d, lazy)
    ref = G.build_plan(w, d)
    o_ref, l_ref = G.run_attention(w, d, ref)
    torch.cuda.synchronize()
    assert torch.equal(o_lazy, o_ref) and torch.equal(l_lazy, l_ref)
    assert lazy.info.build_mode == mpb.BUILD_SINGLE_PASS_DEFERRED
    _same_exports(lazy.export(), ref.export())


def test_back_to_back_deferred_builds():
    """Several deferred builds of one host thread in a row, each followed by
    its forward, before any header is read: every build reuses the thread's
    workspace, look-back words and header slot in stream order."""
    _case("deferred_chain")
    runs = []
    for name in NAMES:
        w = W.make(name, small=True)
        d = G.device_inputs(w)
        plan = G.build_plan(w, d, defer_header=True)
        runs.append((w, d, plan, G.run_attention(w, d, plan)))
    torch.cuda.synchronize()
    for w, d, plan, (o, lse) in runs:
        assert plan.info.build_mode == mpb.BUILD_SINGLE_PASS_DEFERRED
        O, L = oracle.attention(w)
        G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64),
                            w.name)


@pytest.mark.parametrize("name", ["window_sink", "chunk_long_kv"])
def test_deferred_splitk_and_paged(name):
    """Split-K and paged forwards read a deferred plan's header first; their
    results equal those over the waited-for plan."""
    from tests.test_gpu_paged import make_pool, run_paged
    w = W.make(name, small=True)
    _case("deferred_split_paged", name=name)
    d = G.device_inputs(w)
    lazy = G.build_plan(w, d, defer_header=True)
    ref = G.build_plan(w, d)
    for sp in (3, 0):
        o, lse = G.run_attention(w, d, lazy, num_splits=sp)
        o_r, l_r = G.run_attention(w, d, ref, num_splits=sp)
        torch.cuda.synchronize()
        assert torch.equal(o, o_r) and torch.equal(lse, l_r), sp
    lazy2 = G.build_plan(w, d, defer_header=True)
    pool = make_pool(w, 2 * ref.problem.tile_k, seed=2)
    o, lse = run_paged(w, d, lazy2, pool, 2 * ref.problem.tile_k)
    o_r, l_r = G.run_attention(w, d, ref)
    torch.cuda.synchronize()
    assert torch.equal(o, o_r) and torch.equal(lse, l_r)


def test_deferred_errors_surface_at_first_header_read():
    """An endpoint past k_len: the deferred build returns a plan, a forward
    on it writes nothing, and mask_plan_info, the Split-K forward and the
    exports all report MPB_ERR_ENDPOINT_RANGE; the same for bad THD prefixes
    (MPB_ERR_SEQLENS)."""
    _case("deferred_errors")
    w = W.make("window_sink", small=True)
    d = G.device_inputs(w)
    mf = d["mask_func"].clone()
    mf[0, 2, 37] = w.seqlen_k + 5
    bad = mpb.mask_plan_build(G.problem(w), mf, None, None, defer_header=True)
    o = torch.full_like(d["q"], 7.0)
    lse = torch.full((w.heads_q, w.total_q), 3.0, dtype=torch.float32, device="cuda")
    mpb.flex_attn_fwd(bad, d["q"], d["k"], d["v"], scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 3.0).all()), "a failed plan wrote output"
    for call in (lambda: mpb.mask_plan_info(bad), lambda: mpb.mask_plan_export(bad),
                 lambda: G.run_attention(w, d, bad, num_splits=2)):
        with pytest.raises(mpb.MPBError) as e:
            call()
        assert e.value.status == 2   # MPB_ERR_ENDPOINT_RANGE
    bad.close()
    v = W.make("varlen_doc", small=True)
    dv = G.device_inputs(v)
    cq = dv["cu_q"].clone()
    cq[2] = cq[1] - 1   # decreasing prefix
    badv = mpb.mask_plan_build(G.problem(v), dv["mask_func"], cq, dv["cu_k"],
                               defer_header=True)
    with pytest.raises(mpb.MPBError) as e:
        mpb.mask_plan_info(badv)
    assert e.value.status == 4   # MPB_ERR_SEQLENS
    badv.close()


def test_defer_ignored_where_the_build_is_not_single_pass():
    """A plan with the backward view is not built in a single pass: it reads
    its header back during the build whatever defer_header says."""
    w = W.make("window_sink", small=True)
    _case("deferred_bwd")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, build_backward=True, defer_header=True)
    assert plan.info.build_mode in (mpb.BUILD_IN_PLACE, mpb.BUILD_EXACT)

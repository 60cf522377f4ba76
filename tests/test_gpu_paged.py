"""GPU parity of the paged K/V forward.

FlexAttention's paged attention folds the page table into the block indices
(physical block = page_table[batch][logical block]), so the attention itself
is unchanged: the paged forward over a page pool must equal the contiguous
forward over the same logical K/V bit for bit (same kernels, same
arithmetic), and the oracle within the forward's tolerances.  Every pool row
that does not hold a sample's key -- spare pages and the tail of each
sample's last page -- is NaN, so a read outside a sample's keys would show
up in the output.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_support as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def require_gpu():
    assert torch.cuda.is_available(), "no GPU visible to a GPU test"


def _case(case, **kw):
    print("CASE", case, kw, flush=True)


def make_pool(w, page_size, seed=0, spare=3):
    """Scatter the workload's logical K/V into a NaN-filled page pool under a
    random page table.  Returns (k_pool, v_pool, page_table) as device
    tensors: pools [num_pages, page_size, Hk, D], table int32 [B, pages_per_seq]
    with -1 past each sample's pages."""
    rng = np.random.default_rng(seed)
    need = [-(-w.sample_bounds(b)[3] // page_size) for b in range(w.batch)]
    pps = max(max(need), -(-w.seqlen_k // page_size), 1)
    num_pages = sum(need) + spare
    perm = rng.permutation(num_pages)
    table = np.full((w.batch, pps), -1, np.int32)
    kp = np.full((num_pages * page_size, w.heads_k, w.head_dim), np.nan, np.float32)
    vp = kp.copy()
    nxt = 0
    for b in range(w.batch):
        _, _, k_off, k_len = w.sample_bounds(b)
        for lp in range(need[b]):
            pg = int(perm[nxt])
            nxt += 1
            table[b, lp] = pg
            lo, hi = lp * page_size, min((lp + 1) * page_size, k_len)
            kp[pg * page_size:pg * page_size + hi - lo] = w.k[k_off + lo:k_off + hi]
            vp[pg * page_size:pg * page_size + hi - lo] = w.v[k_off + lo:k_off + hi]
    dt = G.torch_dtype(w)
    shape = (num_pages, page_size, w.heads_k, w.head_dim)
    k_pool = torch.from_numpy(kp).to(dt).reshape(shape).cuda()
    v_pool = torch.from_numpy(vp).to(dt).reshape(shape).cuda()
    return k_pool, v_pool, torch.from_numpy(table).cuda()


def run_paged(w, d, plan, pool, page_size, **kw):
    import mask_planned_block_amd as mpb
    k_pool, v_pool, table = pool
    return mpb.flex_attn_fwd_paged(plan, d["q"], k_pool, v_pool, table, page_size,
                                   scale=w.scale, softcap=w.softcap if w.softcap > 0 else None,
                                   alibi_slopes=d["slopes"],
                                   alibi_before_softcap=w.alibi_before_softcap, **kw)


@pytest.mark.parametrize("name", ["window_sink", "varlen_doc", "block_sparse", "prefix_softcap",
                                  "chunk_long_kv"])
@pytest.mark.parametrize("pages_per_tile", [1, 2, 4])
def test_paged_equals_contiguous_and_oracle(name, pages_per_tile):
    w = W.make(name, small=True)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    ps = plan.problem.tile_k * pages_per_tile
    _case("paged", name=name, page_size=ps)
    pool = make_pool(w, ps, seed=pages_per_tile)
    import mask_planned_block_amd as mpb
    ws = torch.empty(mpb.flex_attn_fwd_paged_workspace_size(plan, 1) + 256, dtype=torch.uint8,
                     device="cuda")
    o, lse = run_paged(w, d, plan, pool, ps, workspace=ws)
    o_ref, l_ref = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "paged != contiguous"
    # a second call reuses the lists the first one remapped into the workspace
    o2, l2 = run_paged(w, d, plan, pool, ps, workspace=ws, remap=False)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_ref) and torch.equal(l2, l_ref), "reused remap differs"
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), name)


@pytest.mark.parametrize("pack", [None, False])   # the library's choice (packed), unpacked
@pytest.mark.parametrize("tq,tk", [(64, 64), (128, 32), (64, 32)])
def test_paged_other_tiles_and_splitk(tq, tk, pack):
    w = W.make("chunk_long_kv", small=True)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, tq, tk, pack_gqa=pack)
    ps = 2 * tk
    _case("paged_tiles_split", tq=tq, tk=tk, pack=pack)
    pool = make_pool(w, ps, seed=7)
    for sp in (1, 3):
        o, lse = run_paged(w, d, plan, pool, ps, num_splits=sp)
        o_ref, l_ref = G.run_attention(w, d, plan, num_splits=sp)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "S=%d" % sp


def test_paged_full_size_chunk_long_kv():
    """The long-K chunk shape at full size with 256-token pages and the
    library's Split-K choice: identical to the contiguous Split-K forward."""
    w = W.make("chunk_long_kv")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    _case("paged_full")
    pool = make_pool(w, 256, seed=3, spare=17)
    o, lse = run_paged(w, d, plan, pool, 256, num_splits=0)
    o_ref, l_ref = G.run_attention(w, d, plan, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    rows = G.sample_rows(w, n_random=100)
    O, L = oracle.attention(w, rows=rows)
    lse_np = lse.cpu().numpy().astype(np.float64)
    G.compare_attention(w, O, L, G.flat_o(w, o)[rows[:, 0], rows[:, 1]],
                        lse_np[rows[:, 1], rows[:, 0]], "paged full")


def test_paged_errors():
    import mask_planned_block_amd as mpb
    w = W.make("window_sink", small=True)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    tk = plan.problem.tile_k
    pool = make_pool(w, 2 * tk)

    def expect(name, fn):
        with pytest.raises(mpb.MPBError) as ei:
            fn()
        assert ei.value.name == name, str(ei.value)

    k_pool, v_pool, table = pool
    # a page that is not a multiple of the K tile
    kp2 = k_pool.reshape(-1, w.heads_k, w.head_dim)[: (k_pool.shape[0] * k_pool.shape[1]) //
                                                     (tk + 32) * (tk + 32)]
    expect("MPB_ERR_UNSUPPORTED", lambda: mpb.flex_attn_fwd_paged(
        plan, d["q"], kp2, kp2, table, tk + 32))
    # too few pages per sequence for seqlen_k
    expect("MPB_ERR_INVALID_ARGUMENT", lambda: mpb.flex_attn_fwd_paged(
        plan, d["q"], k_pool, v_pool, table[:, :1].contiguous(), 2 * tk))
    # workspace too small
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    expect("MPB_ERR_WORKSPACE", lambda: mpb.flex_attn_fwd_paged(
        plan, d["q"], k_pool, v_pool, table, 2 * tk, workspace=small))
    # fp32 plans have no paged consumer
    wf = W.make("tiny_causal", small=True)
    df = G.device_inputs(wf)
    pf = G.build_plan(wf, df)
    poolf = make_pool(wf, 64)
    expect("MPB_ERR_UNSUPPORTED", lambda: mpb.flex_attn_fwd_paged(
        pf, df["q"], poolf[0], poolf[1], poolf[2], 64))

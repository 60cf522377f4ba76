"""GPU parity of PackGQA plans and forwards.

PackGQA ("Flex Attention Mask Plan Design", §4.1 consumer resolution and
§6.2) packs the G = Hq/Hk Q heads that share one K/V head into one forward
tile: a tile of T_Q rows holds T_Q/G tokens of all G heads, so the plan's rows
are blocks of T_Q/G tokens, its tasks are (row, K/V head) and every partial
tile keeps one payload word row per token.  The block relation and the
predicate words are those of an unpacked plan with T_Q/G-token rows, so the
packed export is compared bit for bit with the oracle's plan at tile
(T_Q/G, T_KV); the schedule with the K/V heads as task heads; the attention,
which packing does not change, with the oracle's fp64 attention at the
forward's tolerances (fp32 1e-4; bf16 2e-2 on O, 1e-2 on LSE), rows with
nothing visible exactly O = 0 and LSE = -inf.
"""
import dataclasses

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


def _causal_offset_thd(lens_q, lens_k, heads_q, heads_k, seed, **kw):
    """THD samples whose queries are the last q_len of k_len causal tokens
    (appending a chunk to a cache): row q of sample b sees [0, k_len - q_len
    + q + 1)."""
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    mf = np.zeros((1, 1, int(cq[-1])), np.int32)
    for b, (lq, lk) in enumerate(zip(lens_q, lens_k)):
        mf[0, 0, cq[b]:cq[b + 1]] = lk - lq + np.arange(lq) + 1
    return W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=cq, cu_seqlens_k=ck,
                    heads_q=heads_q, heads_k=heads_k, head_dim=128, dtype=W.DTYPE_BF16,
                    seed=seed, **kw)


def _ragged_fp32(heads_q, heads_k, seed):
    B, Sq, Sk = 2, 150, 97
    rng = np.random.default_rng(seed)
    mf = np.sort(rng.integers(0, Sk + 1, size=(1, 7, B * Sq)), axis=1).astype(np.int32)
    mf[:, :, 5:9] = 0   # rows with nothing visible
    return W.custom(mf, batch=B, seqlen_q=Sq, seqlen_k=Sk, heads_q=heads_q, heads_k=heads_k,
                    head_dim=64, dtype=W.DTYPE_FP32, seed=seed)


CASES = {
    # chunk of 200 queries against 3000 cached keys, G = 2
    "chunk_g2": lambda: W.make("chunk_long_kv", small=True),
    # 16-token decode chunks, G = 8: 16-token plan rows
    "decode_g8": lambda: W.chunk_long_kv(batch=3, heads_q=32, heads_k=4, seqlen_q=16,
                                         seqlen_k=1500),
    "window_g4": lambda: W.window_sink(batch=2, heads=8, heads_k=2, seqlen=700),
    "varlen_g4": lambda: W.varlen_doc(total=1500, nseq=5, min_len=100, heads=8, heads_k=2),
    # softcap then ALiBi: every lane of a packed tile has its own head's slope
    "prefix_softcap_g4": lambda: W.prefix_softcap(batch=2, heads=8, heads_k=2, seqlen=600,
                                                  prefix=150),
    # ALiBi inside the softcap, THD chunks of 0..64 queries
    "thd_chunks_g4": lambda: _causal_offset_thd([1, 5, 16, 0, 33, 64], [300, 1000, 64, 200, 700,
                                                                        129], 16, 4, seed=4,
                                                softcap=20.0, alibi=True,
                                                alibi_before_softcap=True),
    "fp32_g2": lambda: _ragged_fp32(4, 2, 21),
    "fp32_g4": lambda: _ragged_fp32(8, 2, 22),
}


def _tiles(name, w):
    """Physical tiles with a forward consumer whose packed rows keep >= 16
    tokens."""
    g = w.heads_q // w.heads_k
    if w.dtype == W.DTYPE_FP32:
        cand = [(64, 64), (64, 32)]
    else:
        cand = [(128, 64), (128, 32), (64, 64)]
    return [(tq, tk) for tq, tk in cand if tq // g >= 16]


PARAMS = [(name, tq, tk) for name, f in CASES.items() for tq, tk in _tiles(name, f())]


def task_view(w):
    """The workload as the packed schedule sees it: one task head per K/V
    head (group 1)."""
    return dataclasses.replace(w, heads_q=w.heads_k)


def check_packed_plan(w, plan, tq, tk):
    g = w.heads_q // w.heads_k
    info = plan.info
    assert info.signature.pack_gqa == g
    assert info.problem.tile_q == tq and info.problem.tile_k == tk
    assert info.num_tasks == info.rows_total * w.heads_k
    gp = plan.export()
    G.compare_plan(gp, oracle.build_plan(w, tq // g, tk))
    G.check_schedule(task_view(w), gp, tq // g)
    G.check_launch_order(task_view(w), gp, tq // g)


@pytest.mark.parametrize("name,tq,tk", PARAMS)
def test_packed_plan_and_forward(name, tq, tk):
    w = CASES[name]()
    _case("packgqa", name=name, tq=tq, tk=tk)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, tq, tk, pack_gqa=True)
    check_packed_plan(w, plan, tq, tk)
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64),
                        "%s %dx%d" % (name, tq, tk))


@pytest.mark.parametrize("name", ["chunk_g2", "decode_g8", "thd_chunks_g4", "fp32_g4"])
@pytest.mark.parametrize("num_splits", [3, 8])
def test_packed_splitk(name, num_splits):
    w = CASES[name]()
    _case("packgqa_splitk", name=name, num_splits=num_splits)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, pack_gqa=True)
    assert plan.info.signature.pack_gqa == w.heads_q // w.heads_k
    o, lse = G.run_attention(w, d, plan, num_splits=num_splits)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64),
                        "%s S=%d" % (name, num_splits))


@pytest.mark.parametrize("name", ["chunk_g2", "decode_g8"])
def test_packed_paged_equals_contiguous(name):
    """Paged K/V under a packed plan: bit-identical to the contiguous packed
    forward (the page table only moves where K/V tiles are read)."""
    from tests.test_gpu_paged import make_pool, run_paged
    w = CASES[name]()
    _case("packgqa_paged", name=name)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, pack_gqa=True)
    o_ref, l_ref = G.run_attention(w, d, plan)
    pool = make_pool(w, 128, seed=5)
    o, lse = run_paged(w, d, plan, pool, 128)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), name)


def test_library_choice():
    """Left to the library, a plan packs whenever the mask and tile allow it;
    pack_gqa=False keeps it unpacked, and both forwards match the oracle."""
    w = CASES["decode_g8"]()
    _case("packgqa_auto")
    d = G.device_inputs(w)
    O, L = oracle.attention(w)
    auto = G.build_plan(w, d)
    assert auto.info.signature.pack_gqa == 8
    off = G.build_plan(w, d, pack_gqa=False)
    assert off.info.signature.pack_gqa == 1 and off.info.num_tasks == off.info.rows_total * 32
    for plan, what in ((auto, "auto"), (off, "off")):
        o, lse = G.run_attention(w, d, plan)
        torch.cuda.synchronize()
        G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), what)
    long_q = W.make("chunk_long_kv", small=True)        # 200 queries, G = 2
    dl = G.device_inputs(long_q)
    assert G.build_plan(long_q, dl).info.signature.pack_gqa == 2
    # a plan with the backward view is never packed
    assert G.build_plan(long_q, dl, build_backward=True).info.signature.pack_gqa == 1
    # one mask per Q head (here all equal): the heads of a group may differ,
    # so the library does not pack
    ph = dataclasses.replace(w, mask_heads=w.heads_q, mask_func=np.ascontiguousarray(
        np.repeat(w.mask_func, w.heads_q, axis=0)))
    assert G.build_plan(ph, G.device_inputs(ph)).info.signature.pack_gqa == 1


def test_packed_full_chunk_long_kv_sampled_rows():
    """The long-K chunk at full size (Hq 32, Hk 8, 512 queries, 32768 keys),
    packed, through the library's Split-K choice and unsplit: sampled rows
    against the oracle and agreement of the two forwards."""
    w = W.make("chunk_long_kv")
    _case("packgqa_full")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, pack_gqa=True)
    check_packed_plan(w, plan, plan.info.problem.tile_q, plan.info.problem.tile_k)
    o, lse = G.run_attention(w, d, plan, num_splits=0)
    o1, l1 = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    lse_np = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(lse_np).all() and not torch.isnan(o.float()).any().item()
    assert float((o.float() - o1.float()).abs().max()) <= 2e-2
    assert float((lse - l1).abs().max()) <= 1e-3
    rows = G.sample_rows(w, n_random=300, tile_q=plan.info.problem.tile_q // 4)
    O, L = oracle.attention(w, rows=rows)
    og = G.flat_o(w, o)[rows[:, 0], rows[:, 1]]
    lg = lse_np[rows[:, 1], rows[:, 0]]
    G.compare_attention(w, O, L, og, lg, "chunk_long_kv packed")

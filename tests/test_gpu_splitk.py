"""GPU parity of the Split-K forward and of the partial-state merge.

Split-K (Tessera page, "Split-K") cuts every task's tile list into parts run
by separate workgroups and merges their partial states; the result is the
same attention, so it is compared with the oracle's attention at the
forward's tolerances (fp32 1e-4; bf16 2e-2 on O, 1e-2 on LSE), rows with
nothing visible exactly O = 0 and LSE = -inf.  The merge entry point is
compared with the oracle's merge on random partial states (fp32 arithmetic
on both sides of the rounding: 1e-5 relative to the output scale for fp32
output, the bf16 rounding step 2^-8 of |O| for bf16 output).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_support as G

pytestmark = pytest.mark.gpu

SMALL = ["tiny_causal", "window_sink", "varlen_doc", "block_sparse", "prefix_softcap",
         "chunk_long_kv"]


@pytest.fixture(scope="module", autouse=True)
def require_gpu():
    assert torch.cuda.is_available(), "no GPU visible to a GPU test"


def _case(case, **kw):
    print("CASE", case, kw, flush=True)


def _run_split(w, d, plan, num_splits):
    return G.run_attention(w, d, plan, num_splits=num_splits)


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("num_splits", [2, 3, 7])
def test_splitk_small_all_rows(name, num_splits):
    w = W.make(name, small=True)
    _case("splitk_small", name=name, num_splits=num_splits)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    o, lse = _run_split(w, d, plan, num_splits)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64),
                        "%s S=%d" % (name, num_splits))


@pytest.mark.parametrize("pack", [None, False])   # the library's choice (packed), unpacked
@pytest.mark.parametrize("tq,tk", [(64, 64), (128, 32), (64, 32)])
def test_splitk_other_tiles(tq, tk, pack):
    w = W.make("chunk_long_kv", small=True)
    _case("splitk_tiles", tq=tq, tk=tk, pack=pack)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, tq, tk, pack_gqa=pack)
    o, lse = _run_split(w, d, plan, 5)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64))


def test_splitk_more_parts_than_tiles_and_auto():
    """64 parts leave most parts of every task empty (LSE = -inf partial
    states that the merge must skip); 0 = the library's choice."""
    w = W.make("window_sink", small=True)
    _case("splitk_64_and_auto")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    O, L = oracle.attention(w)
    for sp in (64, 0, 1):
        o, lse = _run_split(w, d, plan, sp)
        torch.cuda.synchronize()
        G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64),
                            "S=%d" % sp)


def test_splitk_empty_rows_empty_samples_gqa():
    lens_q = [130, 0, 77, 1, 256]
    lens_k = [700, 5, 0, 64, 900]
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    rng = np.random.default_rng(31)
    Hq = 4
    mf = np.zeros((Hq, 5, int(cq[-1])), np.int32)
    for b in range(5):
        for t in range(cq[b], cq[b + 1]):
            mf[:, :, t] = np.sort(rng.integers(0, lens_k[b] + 1, size=(Hq, 5)), axis=1)
    mf[:, :, 0:3] = 0          # fully masked rows
    w = W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=cq, cu_seqlens_k=ck, heads_q=Hq,
                 heads_k=2, head_dim=128, dtype=W.DTYPE_BF16, seed=9)
    _case("splitk_edge_thd")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    O, L = oracle.attention(w)
    for sp in (2, 4, 9):
        o, lse = _run_split(w, d, plan, sp)
        torch.cuda.synchronize()
        G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64),
                            "edge S=%d" % sp)


def test_splitk_fp32_ragged():
    B, Sq, Sk = 2, 150, 700
    rng = np.random.default_rng(13)
    mf = np.sort(rng.integers(0, Sk + 1, size=(1, 7, B * Sq)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=Sq, seqlen_k=Sk, heads_q=3, head_dim=64,
                 dtype=W.DTYPE_FP32, seed=3)
    _case("splitk_fp32")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    o, lse = _run_split(w, d, plan, 3)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), "fp32")


def test_splitk_full_chunk_long_kv_sampled_rows():
    """The Split-K benchmark shape at full size, in the benchmark's launch
    configuration (the library's split count): sampled rows against the
    oracle, whole-tensor properties, and agreement with the unsplit forward."""
    import mask_planned_block_amd as mpb
    w = W.make("chunk_long_kv")
    _case("splitk_full")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    sp = mpb.flex_attn_fwd_num_splits(plan)
    assert sp > 1, "the long-K shape should be split"
    o, lse = _run_split(w, d, plan, 0)
    o1, l1 = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    lse_np = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(lse_np).all() and not torch.isnan(o.float()).any().item()
    # split and unsplit compute the same rows with different rounding orders
    assert float((o.float() - o1.float()).abs().max()) <= 2e-2
    assert float((lse - l1).abs().max()) <= 1e-3
    rows = G.sample_rows(w, n_random=300)
    O, L = oracle.attention(w, rows=rows)
    og = G.flat_o(w, o)[rows[:, 0], rows[:, 1]]
    lg = lse_np[rows[:, 1], rows[:, 0]]
    G.compare_attention(w, O, L, og, lg, "chunk_long_kv S=%d" % sp)


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_entry_point_against_oracle(hd, out_dtype):
    import mask_planned_block_amd as mpb
    rng = np.random.default_rng(hd)
    P, T, H = 5, 37, 3
    o_parts = rng.standard_normal((P, T, H, hd)).astype(np.float32)
    lse_parts = (3.0 * rng.standard_normal((P, H, T))).astype(np.float32)
    lse_parts[rng.random((P, H, T)) < 0.3] = -np.inf     # empty parts
    lse_parts[:, 1, 5] = -np.inf                         # a row with every part empty
    o_parts[lse_parts.transpose(0, 2, 1) == -np.inf] = np.nan   # never read
    _case("merge", hd=hd, out=str(out_dtype))
    o, lse = mpb.flex_attn_fwd_merge(torch.from_numpy(o_parts).cuda(),
                                     torch.from_numpy(lse_parts).cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    n = T * H
    # oracle rows follow O's (token, head) order
    op = o_parts.reshape(P, n, hd).astype(np.float64)
    lp = lse_parts.transpose(0, 2, 1).reshape(P, n).astype(np.float64)
    op = np.where(np.isfinite(lp)[:, :, None], op, 0.0)
    O, L = oracle.merge(op, lp)
    og = o.float().cpu().numpy().reshape(n, hd).astype(np.float64)
    lg = lse.cpu().numpy().T.reshape(n).astype(np.float64)
    empty = ~np.isfinite(L)
    assert empty.sum() == 1 and np.array_equal(~np.isfinite(lg), empty)
    assert np.all(og[empty] == 0.0) and not np.isnan(og).any()
    scale = float(np.max(np.abs(O)))
    tol = 1e-5 * scale if out_dtype == torch.float32 else 2.0 ** -8 * scale
    assert float(np.max(np.abs(og - O))) <= tol
    assert float(np.max(np.abs(lg[~empty] - L[~empty]))) <= 1e-5 * max(1.0, np.abs(L[~empty]).max())


def test_splitk_errors():
    import mask_planned_block_amd as mpb
    w = W.make("window_sink", small=True)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)

    def expect(name, fn):
        with pytest.raises(mpb.MPBError) as ei:
            fn()
        assert ei.value.name == name, str(ei.value)

    expect("MPB_ERR_INVALID_ARGUMENT", lambda: mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"],
                                                                  num_splits=65))
    need = mpb.flex_attn_fwd_splitk_workspace_size(plan, 4)
    assert need > 0 and mpb.flex_attn_fwd_splitk_workspace_size(plan, 1) == 0
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    expect("MPB_ERR_WORKSPACE", lambda: mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"],
                                                          num_splits=4, workspace=small))
    expect("MPB_ERR_UNSUPPORTED", lambda: mpb.flex_attn_fwd_merge(
        torch.zeros((2, 3, 1, 96), device="cuda"), torch.zeros((2, 1, 3), device="cuda")))

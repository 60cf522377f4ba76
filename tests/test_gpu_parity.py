"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Plan arrays (classes, offsets, indices, payload words, header) must match
bit-exactly; O/LSE within max-abs 1e-4 (fp32 inputs) or 2e-2 / 1e-2 (bf16
inputs) of the fp64 oracle; rows with nothing visible exactly O = 0 and
LSE = -inf.  Reduced shapes are compared on every row; the full benchmark
shapes on the whole plan and on sampled rows (random rows plus sample and tile
edges) plus whole-tensor properties.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_support as G

pytestmark = pytest.mark.gpu

CONFIGS = ["tiny_causal", "window_sink", "varlen_doc", "block_sparse", "prefix_softcap"]


@pytest.fixture(scope="module", autouse=True)
def require_gpu():
    # Fail, do not skip, when a GPU run has no device.
    assert torch.cuda.is_available(), "no GPU visible to a GPU test"
    import mask_planned_block_amd as mpb
    assert mpb.library_path.endswith("libmpb.so")


def default_tiles(w):
    """The library's tile for a workload whose plan leaves it open: 128x32 for
    bf16 d=128 once the plan has at least 3 tasks per CU, else 128x64; fp32
    64x64 (d=64)."""
    if w.dtype != W.DTYPE_BF16:
        return (64, 64) if w.head_dim == 64 else (64, 32)
    if w.head_dim != 128:
        return (128, 64)
    rows = w.batch * -(-w.seqlen_q // 128) if w.layout == W.LAYOUT_BSHD else w.total_q // 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return (128, 32) if rows * w.heads_q >= 3 * cus else (128, 64)


def _print_case(case, **kw):
    print("CASE", case, kw, flush=True)


# ------------------------------------------------------------------ plan

@pytest.mark.parametrize("name", CONFIGS)
@pytest.mark.parametrize("tiles", ["default", "alt"])
def test_plan_bit_exact_small(name, tiles):
    w = W.make(name, small=True, with_values=False)
    tq, tk = default_tiles(w) if tiles == "default" else (64, 32)
    _print_case("plan_small", name=name, tq=tq, tk=tk)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, tq, tk)
    gp = plan.export()
    op = oracle.build_plan(w, tq, tk)
    G.compare_plan(gp, op)
    G.check_schedule(w, gp, tq)
    G.check_launch_order(w, gp, tq)


@pytest.mark.parametrize("name", CONFIGS)
def test_plan_bit_exact_full(name):
    w = W.make(name, with_values=False)
    tq, tk = default_tiles(w)
    _print_case("plan_full", name=name, tq=tq, tk=tk)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    assert (plan.problem.tile_q, plan.problem.tile_k) == (tq, tk), "library tile choice"
    gp = plan.export()
    op = oracle.build_plan(w, tq, tk)
    G.compare_plan(gp, op)
    G.check_schedule(w, gp, tq)
    G.check_launch_order(w, gp, tq)


# ------------------------------------------------------------------ attention

@pytest.mark.parametrize("name", CONFIGS)
def test_attention_small_all_rows(name):
    w = W.make(name, small=True)
    _print_case("attn_small", name=name)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), name)


@pytest.mark.parametrize("name", CONFIGS)
def test_attention_full_sampled_rows(name):
    w = W.make(name)
    _print_case("attn_full", name=name)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    lse_np = lse.cpu().numpy().astype(np.float64)
    # properties at full size: every row of these workloads sees >= 1 key
    assert np.isfinite(lse_np).all()
    assert not torch.isnan(o.float()).any().item()
    rows = G.sample_rows(w, tile_q=plan.problem.tile_q)
    O, L = oracle.attention(w, rows=rows)
    og = G.flat_o(w, o)[rows[:, 0], rows[:, 1]]
    lg = lse_np[rows[:, 1], rows[:, 0]]
    G.compare_attention(w, O, L, og, lg, name)


@pytest.mark.parametrize("tq,tk", [(64, 64), (128, 32), (64, 32)])
@pytest.mark.parametrize("name", ["window_sink", "varlen_doc", "block_sparse"])
def test_attention_other_tiles(name, tq, tk):
    w = W.make(name, small=True)
    _print_case("attn_tiles", name=name, tq=tq, tk=tk)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, tq, tk)
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), name)


@pytest.mark.parametrize("variant", ["softcap", "alibi", "alibi_first", "both"])
def test_score_mod_variants(variant):
    w = W.make("prefix_softcap", small=True)
    if variant == "softcap":
        w.alibi_slopes = None
    elif variant == "alibi":
        w.softcap = 0.0
    elif variant == "alibi_first":
        w.alibi_before_softcap = True
    _print_case("score_mod", variant=variant)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), variant)


@pytest.mark.parametrize("dtype,hd", [(W.DTYPE_BF16, 64), (W.DTYPE_FP32, 128)])
def test_other_head_dims(dtype, hd):
    w = W.window_sink(batch=1, heads=2, seqlen=300, head_dim=hd, dtype=dtype, seed=4)
    _print_case("head_dim", dtype=dtype, hd=hd)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64))


# ------------------------------------------------------------------ edge cases

def test_empty_samples_empty_rows_gqa_hmask():
    lens_q = [130, 0, 77, 1, 256]
    lens_k = [100, 5, 0, 64, 300]
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    rng = np.random.default_rng(3)
    Hq = 4
    mf = np.zeros((Hq, 5, int(cq[-1])), np.int32)
    for b in range(5):
        for t in range(cq[b], cq[b + 1]):
            mf[:, :, t] = np.sort(rng.integers(0, lens_k[b] + 1, size=(Hq, 5)), axis=1)
    mf[:, :, cq[0]:cq[0] + 3] = 0          # fully masked rows
    w = W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=cq, cu_seqlens_k=ck, heads_q=Hq,
                 heads_k=2, head_dim=128, dtype=W.DTYPE_BF16, seed=8)
    _print_case("edge_thd")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    pl = plan.problem
    G.compare_plan(plan.export(), oracle.build_plan(w, pl.tile_q, pl.tile_k))
    G.check_schedule(w, plan.export(), 128)
    G.check_launch_order(w, plan.export(), 128)
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), "edge")


def test_ragged_fixed_length_fp32():
    # Sq, Sk not tile multiples; fp32 path; random multi-interval endpoints.
    B, Sq, Sk = 2, 150, 97
    rng = np.random.default_rng(12)
    mf = np.sort(rng.integers(0, Sk + 1, size=(1, 7, B * Sq)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=Sq, seqlen_k=Sk, heads_q=3, head_dim=64,
                 dtype=W.DTYPE_FP32, seed=2)
    _print_case("ragged_fp32")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    pl = plan.problem
    G.compare_plan(plan.export(), oracle.build_plan(w, pl.tile_q, pl.tile_k))
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), "ragged")


def test_force_partial_is_identical_and_plan_reuse():
    w = W.make("window_sink", small=True)
    _print_case("force_partial")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    o1, l1 = G.run_attention(w, d, plan)
    o2, l2 = G.run_attention(w, d, plan, force_partial=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # new Q/K/V values reuse the plan (geometry unchanged)
    w2 = W.make("window_sink", small=True, seed=5)
    d2 = G.device_inputs(w2)
    o3, l3 = G.run_attention(w2, d2, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w2)
    G.compare_attention(w2, O, L, G.flat_o(w2, o3), l3.cpu().numpy().astype(np.float64))


def test_one_plan_two_streams():
    w = W.make("block_sparse", small=True)
    _print_case("two_streams")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s in (s1, s2):
        with torch.cuda.stream(s):
            outs.append(G.run_attention(w, d, plan, stream=s))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_builds_alternating_streams():
    """Consecutive builds on different streams (the build workspace is shared
    by one host thread's builds) give the oracle's plans."""
    ws = [W.make("varlen_doc", small=True), W.make("block_sparse", small=True)]
    _print_case("alternating_streams")
    ds = [G.device_inputs(w) for w in ws]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    plans = []
    for r in range(2):
        for w, d, s in ((ws[0], ds[0], s1), (ws[1], ds[1], s2)):
            plans.append((w, G.build_plan(w, d, stream=s)))
    torch.cuda.synchronize()
    for w, plan in plans:
        pl = plan.problem
        G.compare_plan(plan.export(), oracle.build_plan(w, pl.tile_q, pl.tile_k))


# ------------------------------------------------------------------ errors

def _expect(status_name, fn):
    import mask_planned_block_amd as mpb
    with pytest.raises(mpb.MPBError) as ei:
        fn()
    assert ei.value.name == status_name, str(ei.value)


def test_device_side_validation_errors():
    import mask_planned_block_amd as mpb
    w = W.make("window_sink", small=True, with_values=False)
    d = G.device_inputs(w)
    cases = []
    bad = w.mask_func.copy()
    bad[0, 0, 17], bad[0, 1, 17] = 9, 3              # F0 > F1
    cases.append((bad, "MPB_ERR_ENDPOINT_ORDER", oracle.ERR_ORDER))
    bad = w.mask_func.copy()
    bad[0, 2, 40] = w.seqlen_k + 1                    # beyond k_len
    cases.append((bad, "MPB_ERR_ENDPOINT_RANGE", oracle.ERR_RANGE))
    bad = w.mask_func.copy()
    bad[0, 0, 5] = -1                                 # negative (and F0 > F1 no longer)
    cases.append((bad, "MPB_ERR_ENDPOINT_RANGE", oracle.ERR_RANGE))
    for mf, name, bit in cases:
        wb = W.custom(mf, batch=w.batch, seqlen_q=w.seqlen_q, seqlen_k=w.seqlen_k,
                      heads_q=w.heads_q, head_dim=w.head_dim, with_values=False)
        assert oracle.validate(wb) & bit
        _expect(name, lambda: mpb.mask_plan_build(G.problem(w), torch.from_numpy(mf).cuda()))
    wv = W.make("varlen_doc", small=True, with_values=False)
    dv = G.device_inputs(wv)
    for mutate in (lambda c: c.__setitem__(0, 1), lambda c: c.__setitem__(-1, c[-1] + 1),
                   lambda c: c.__setitem__(2, c[1] - 1)):
        cu = wv.cu_seqlens_q.copy()
        mutate(cu)
        wb = W.custom(wv.mask_func, layout=W.LAYOUT_THD, cu_seqlens_q=cu,
                      cu_seqlens_k=wv.cu_seqlens_k, seqlen_q=wv.seqlen_q, seqlen_k=wv.seqlen_k,
                      head_dim=wv.head_dim, with_values=False)
        wb.total_q = wv.total_q
        assert oracle.validate(wb) == oracle.ERR_SEQLENS
        _expect("MPB_ERR_SEQLENS", lambda: mpb.mask_plan_build(
            G.problem(wv), dv["mask_func"], torch.from_numpy(cu).cuda(), dv["cu_k"]))
    # a valid build still works after the failures (nothing leaked or stuck)
    G.build_plan(w, d)


def test_signature_and_workspace_errors():
    import mask_planned_block_amd as mpb
    w = W.make("window_sink", small=True)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    q2 = d["q"][:, :, :1].contiguous()   # fewer heads than the plan binds
    _expect("MPB_ERR_SIGNATURE_MISMATCH", lambda: mpb.flex_attn_fwd(
        plan, q2, d["k"][:, :, :1].contiguous(), d["v"][:, :, :1].contiguous()))
    _expect("MPB_ERR_SIGNATURE_MISMATCH", lambda: mpb.flex_attn_fwd(
        plan, d["q"].float(), d["k"].float(), d["v"].float()))
    assert mpb.flex_attn_fwd_workspace_size(plan) == 0
    _expect("MPB_ERR_INVALID_ARGUMENT", lambda: mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"],
                                                                   scale=-1.0))


def test_library_tile_choice():
    """tile 0x0 resolves from the task count: bf16 d=128 plans with at least
    three tasks per CU get 128x32 tiles, smaller ones 128x64, and plans with
    the backward view 128x64; an explicit tile is kept."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for heads, want in ((3 * cus // 16, (128, 32)), (3 * cus // 16 - 1, (128, 64))):
        w = W.custom(np.full((1, 1, 2048), 2048, np.int32), batch=1, seqlen_q=2048,
                     seqlen_k=2048, heads_q=heads, head_dim=128, dtype=W.DTYPE_BF16,
                     with_values=False)
        _print_case("tile_choice", heads=heads)
        plan = G.build_plan(w, G.device_inputs(w))
        assert (plan.problem.tile_q, plan.problem.tile_k) == want, (heads, want)
        plan = G.build_plan(w, G.device_inputs(w), 64, 64)
        assert (plan.problem.tile_q, plan.problem.tile_k) == (64, 64)
        # a plan with the backward view keeps 64-wide K tiles
        plan = G.build_plan(w, G.device_inputs(w), build_backward=True)
        assert (plan.problem.tile_q, plan.problem.tile_k) == (128, 64)


@pytest.mark.parametrize("sign", [1.0, -1.0])
@pytest.mark.parametrize("dtype", [W.DTYPE_FP32, W.DTYPE_BF16])
@pytest.mark.parametrize("softcap", [0.0, 20.0])
def test_steep_alibi_negligible_tiles(dtype, softcap, sign):
    """Steep ALiBi slopes put most K tiles far below each row's max: their
    softmax weights are exactly zero in fp32 and the kernel skips them (after
    the scores, or before them when a softcap bounds the scores).  With
    positive slopes the far keys vanish, with negative ones the near keys
    (the row max sits at key 0).  The result must match the oracle, fully
    masked rows included, and equal bit for bit the ablation run that skips
    nothing (and the one that runs full tiles through the predicate path).
    The negative slopes are milder: with them the row max carries the largest
    bias (slope * -q, up to 350 here), and a bias of thousands would leave
    fp32 scores only 2^-11-exact, which the 1e-4 fp32 tolerance presumes
    they are not; 350 still puts most tiles 200 log2 units below the max."""
    B, S, H = 2, 700, 4
    q_local = np.tile(np.arange(S), B)
    mf = np.stack([np.minimum(q_local + 1, 16), np.minimum(q_local + 1, 16), q_local + 1])
    mf[:, :3] = 0                       # three fully masked rows
    slopes = [8.0, 2.0, 0.5, 0.01] if sign > 0 else [-0.5, -0.25, -0.1, -0.01]
    w = W.custom(mf[None].astype(np.int32), batch=B, seqlen_q=S, seqlen_k=S, heads_q=H,
                 head_dim=64 if dtype == W.DTYPE_FP32 else 128, dtype=dtype, seed=46,
                 softcap=softcap, alibi=np.array(slopes, np.float32))
    _print_case("steep_alibi", dtype=dtype, softcap=softcap, sign=sign)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    o, lse = G.run_attention(w, d, plan)
    o2, l2 = G.run_attention(w, d, plan, force_partial=True)
    o3, l3 = G.run_attention(w, d, plan, no_skip=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    assert torch.equal(o, o3) and torch.equal(lse, l3), "a skipped block had nonzero weight"
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64), "steep")


@pytest.mark.parametrize("name", ["block_sparse", "window_sink", "prefix_softcap"])
def test_skips_change_nothing(name):
    """The exact-zero skips (predicate words all zero for a wavefront's rows,
    negligible blocks) leave O and LSE unchanged bit for bit: the ablation
    run that computes every listed tile and block gives the same bytes."""
    w = W.make(name, small=True)
    _print_case("no_skip", name=name)
    d = G.device_inputs(w)
    for tq, tk in ((0, 0), (128, 64), (64, 32)):
        plan = G.build_plan(w, d, tq, tk)
        o, lse = G.run_attention(w, d, plan)
        o3, l3 = G.run_attention(w, d, plan, no_skip=True)
        torch.cuda.synchronize()
        assert torch.equal(o, o3) and torch.equal(lse, l3), (tq, tk)

"""GPU parity of the backward K2Q view (mask_plan_build_ex with
build_backward = 1, exported through mask_plan_export_k2q) against the CPU
oracle's brute-force K2Q view: cu_krows, offsets, Q-tile lists and K-major
payload words bit-exact, header slots 3..6 equal.  The forward part of the
same plan must still equal the oracle's forward plan, and the forward
attention must not change when the plan also holds the K2Q view."""
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
    assert torch.cuda.is_available(), "no GPU visible to a GPU test"


def default_tiles(w):
    return (128, 64) if w.dtype == W.DTYPE_BF16 else (64, 64)


def _case(case, **kw):
    print("CASE", case, kw, flush=True)


def _check_both_views(w, d, tq, tk):
    plan = G.build_plan(w, d, tq, tk, build_backward=True)
    gp = plan.export()
    G.compare_plan(gp, oracle.build_plan(w, tq, tk), with_k2q=True)
    gk = plan.export_k2q()
    G.compare_k2q(gk, oracle.build_k2q(w, tq, tk))
    G.check_k2q_order(gk, w.mask_heads)
    return plan


# every tile geometry with a forward consumer at the workload's dtype and head size
SMALL_CASES = [(n, t) for n in CONFIGS if n != "tiny_causal"
               for t in ((128, 64), (64, 64), (128, 32), (64, 32))] + \
              [("tiny_causal", (64, 64)), ("tiny_causal", (64, 32))]


@pytest.mark.parametrize("name,tiles", SMALL_CASES)
def test_k2q_bit_exact_small(name, tiles):
    w = W.make(name, small=True, with_values=False)
    tq, tk = tiles
    _case("k2q_small", name=name, tq=tq, tk=tk)
    _check_both_views(w, G.device_inputs(w), tq, tk)


@pytest.mark.parametrize("name", CONFIGS)
def test_k2q_bit_exact_full(name):
    # block_sparse (24 mask heads) needs more than the in-place block bound and
    # takes the exact-allocation path; the others are built in place.
    w = W.make(name, with_values=False)
    tq, tk = default_tiles(w)
    _case("k2q_full", name=name, tq=tq, tk=tk)
    _check_both_views(w, G.device_inputs(w), tq, tk)


def test_k2q_random_intervals_exact_path():
    # Eight mask heads of random two-interval rows at S = 4096: the upper-bound
    # block of both views is above 32 MiB, so the counts are read back first.
    S, Hm = 4096, 8
    rng = np.random.default_rng(21)
    mf = np.sort(rng.integers(0, S + 1, size=(Hm, 5, S)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=1, seqlen_q=S, seqlen_k=S, heads_q=Hm, head_dim=128,
                 dtype=W.DTYPE_BF16, with_values=False)
    _case("k2q_exact_random")
    _check_both_views(w, G.device_inputs(w), 128, 64)


def test_k2q_empty_samples_empty_rows_gqa_hmask():
    lens_q = [130, 0, 77, 1, 256]
    lens_k = [100, 5, 0, 64, 300]
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    rng = np.random.default_rng(4)
    Hq = 4
    mf = np.zeros((Hq, 5, int(cq[-1])), np.int32)
    for b in range(5):
        for t in range(cq[b], cq[b + 1]):
            mf[:, :, t] = np.sort(rng.integers(0, lens_k[b] + 1, size=(Hq, 5)), axis=1)
    mf[:, :, 0:3] = 0
    w = W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=cq, cu_seqlens_k=ck, heads_q=Hq,
                 heads_k=2, head_dim=128, dtype=W.DTYPE_BF16, with_values=False)
    _case("k2q_edge_thd")
    d = G.device_inputs(w)
    for tq, tk in ((128, 64), (64, 32)):
        _check_both_views(w, d, tq, tk)


def test_k2q_ragged_fixed_length_fp32():
    B, Sq, Sk = 2, 150, 97
    rng = np.random.default_rng(13)
    mf = np.sort(rng.integers(0, Sk + 1, size=(1, 7, B * Sq)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=Sq, seqlen_k=Sk, heads_q=3, head_dim=64,
                 dtype=W.DTYPE_FP32, with_values=False)
    _case("k2q_ragged_fp32")
    _check_both_views(w, G.device_inputs(w), 64, 64)


def test_forward_unchanged_by_k2q_view():
    w = W.make("varlen_doc", small=True)
    _case("k2q_forward_unchanged")
    d = G.device_inputs(w)
    p1 = G.build_plan(w, d, build_backward=True)
    p0 = G.build_plan(w, d, p1.problem.tile_q, p1.problem.tile_k)
    o0, l0 = G.run_attention(w, d, p0)
    o1, l1 = G.run_attention(w, d, p1)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert p1.info.device_bytes > p0.info.device_bytes


def test_k2q_export_refused_without_view_and_errors():
    import mask_planned_block_amd as mpb
    w = W.make("window_sink", small=True, with_values=False)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    with pytest.raises(mpb.MPBError) as ei:
        plan.export_k2q()
    assert ei.value.name == "MPB_ERR_INVALID_ARGUMENT"
    bad = w.mask_func.copy()
    bad[0, 0, 17], bad[0, 1, 17] = 9, 3
    with pytest.raises(mpb.MPBError) as ei:
        mpb.mask_plan_build(G.problem(w), torch.from_numpy(bad).cuda(), build_backward=True)
    assert ei.value.name == "MPB_ERR_ENDPOINT_ORDER"
    # builds with and without the view alternate on two streams afterwards
    ws = [W.make("block_sparse", small=True, with_values=False), w]
    ds = [G.device_inputs(ws[0]), d]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    plans = []
    for r in range(2):
        for i, s in ((0, s1), (1, s2)):
            plans.append((ws[i], G.build_plan(ws[i], ds[i], stream=s,
                                              build_backward=bool((r + i) % 2 == 0))))
    torch.cuda.synchronize()
    for k, (wk, plan) in enumerate(plans):
        pl = plan.problem
        with_k2q = (k // 2 + k % 2) % 2 == 0
        G.compare_plan(plan.export(), oracle.build_plan(wk, pl.tile_q, pl.tile_k), with_k2q)
        if with_k2q:
            G.compare_k2q(plan.export_k2q(), oracle.build_k2q(wk, pl.tile_q, pl.tile_k))


def test_k2q_no_k_rows():
    # every sample has an empty K: no K plan rows, cu_krows all zero
    cq = np.array([0, 5, 14], np.int32)
    ck = np.array([0, 0, 0], np.int32)
    mf = np.zeros((1, 1, 14), np.int32)
    w = W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=cq, cu_seqlens_k=ck, heads_q=2,
                 head_dim=128, dtype=W.DTYPE_BF16, with_values=False)
    _case("k2q_no_k_rows")
    plan = _check_both_views(w, G.device_inputs(w), 128, 64)
    assert int(plan.info.header[4]) == 0


@pytest.mark.parametrize("name,small", [("window_sink", True), ("block_sparse", False)])
def test_stage_times(name, small):
    import mask_planned_block_amd as mpb
    w = W.make(name, small=small, with_values=False)
    _case("stage_times", name=name, small=small)
    d = G.device_inputs(w)
    for bwd in (False, True):
        plan = G.build_plan(w, d, build_backward=bwd, time_stages=True)
        tq, tk = plan.problem.tile_q, plan.problem.tile_k
        t = plan.stage_times()
        assert t["classify"] > 0 and t["schedule"] > 0, t
        # forward plans are built in a single pass, backward ones in place
        # (small) or with the exact block allocated after the header
        mode = plan.info.build_mode
        assert mode == (mpb.BUILD_SINGLE_PASS if not bwd else
                        mpb.BUILD_IN_PLACE if small else mpb.BUILD_EXACT), (bwd, mode)
        assert (t["materialize"] == -1) == (mode != mpb.BUILD_EXACT), t
        for k in ("k2q_count", "k2q_materialize"):
            assert (t[k] > 0) if bwd else (t[k] == -1), t
        assert t["span"] >= max(t[k] for k in mpb.STAGE_NAMES[:-1]), t
        # the event records change nothing in the plan
        G.compare_plan(plan.export(), oracle.build_plan(w, tq, tk), with_k2q=bwd)
        if bwd:
            G.compare_k2q(plan.export_k2q(), oracle.build_k2q(w, tq, tk))
    with pytest.raises(mpb.MPBError) as ei:
        G.build_plan(w, d).stage_times()
    assert ei.value.name == "MPB_ERR_INVALID_ARGUMENT"


def _exact_single_pass_bytes(w, tq, tk, header):
    """Bytes of a single-pass plan's block after the cut: every array rounded
    to 256 bytes (an empty one still takes 256), the per-row metadata at the
    rows' upper bound, then the payload and the two index lists at their
    exact sizes."""
    def take(count):
        return -(-max(count, 1) * 4 // 256) * 256
    thd = w.layout == W.LAYOUT_THD
    upper = w.batch * -(-w.seqlen_q // tq) if not thd else (w.total_q + w.batch * (tq - 1)) // tq
    tasks = upper * w.heads_q
    n_off = w.mask_heads * upper + 1
    pn, fn = int(header[1]), int(header[2])
    return (take(8) + take(8 * w.batch) + take(w.batch + 1) +
            2 * take(w.batch + 1 if thd else 0) + take(4 * tasks) + take(10) + take(16 * tasks) +
            2 * take(n_off) + take(pn * tq * tk // 32) + take(pn) + take(fn))


@pytest.mark.parametrize("name", ["window_sink", "varlen_doc", "block_sparse"])
def test_single_pass_block_is_cut_to_exact_size(name):
    """A forward plan built in one pass holds exactly its arrays: the block
    allocated at the upper bound of every count is cut after the header, so
    no padded list or payload is kept (only the per-row metadata is sized by
    the rows' upper bound, which is exact for BSHD)."""
    import mask_planned_block_amd as mpb
    w = W.make(name, small=True, with_values=False)
    _case("single_pass_exact", name=name)
    plan = G.build_plan(w, G.device_inputs(w))
    info = plan.info
    assert info.build_mode == mpb.BUILD_SINGLE_PASS
    tq, tk = plan.problem.tile_q, plan.problem.tile_k
    assert info.device_bytes == _exact_single_pass_bytes(w, tq, tk, info.header)
    G.compare_plan(plan.export(), oracle.build_plan(w, tq, tk))

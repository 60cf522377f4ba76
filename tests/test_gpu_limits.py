"""GPU parity at the limits the C ABI accepts and at degenerate sizes.

  * nfunc = 4095 (the largest accepted): 2048 intervals per row, most of them
    empty (repeated endpoints), so the classifier walks 256 batches per row
    and the materializer reads endpoints from HBM (too many to stage in LDS).
  * a sample of 8191 K tiles (the largest accepted at tile_k = 64): one Q
    tile against 524224 keys, classified over 32 windows, the whole K list in
    one task; the Split-K forward splits it 64 ways.
  * zero-length sequences: Sq = 0 (no plan rows, the forward is a no-op) and
    Sk = 0 (every row fully masked: O = 0, LSE = -inf).
Plans are compared bit-exactly with the oracle's, O/LSE at the forward's
tolerances (bf16: 2e-2 / 1e-2).
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


def test_max_nfunc():
    B, Sq, Sk, nfunc = 1, 200, 3000, 4095
    rng = np.random.default_rng(40)
    mf = np.sort(rng.integers(0, Sk + 1, size=(1, nfunc, B * Sq)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=Sq, seqlen_k=Sk, heads_q=2, head_dim=128,
                 dtype=W.DTYPE_BF16, seed=41)
    _case("max_nfunc", nfunc=nfunc)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    pl = plan.problem
    G.compare_plan(plan.export(), oracle.build_plan(w, pl.tile_q, pl.tile_k))
    o, lse = G.run_attention(w, d, plan)
    torch.cuda.synchronize()
    O, L = oracle.attention(w)
    G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64),
                        "nfunc 4095")


def test_max_k_tiles():
    tk = 64
    Sk = 8191 * tk
    Sq = 128
    ql = np.arange(Sq, dtype=np.int64)
    # the last Sq tokens of a causal sequence, plus a sink-only row pattern
    f0 = (Sk - Sq + ql + 1).astype(np.int32)
    f0[:8] = 64
    mf = f0[None, None, :]
    w = W.custom(mf, batch=1, seqlen_q=Sq, seqlen_k=Sk, heads_q=1, head_dim=128,
                 dtype=W.DTYPE_BF16, seed=42)
    _case("max_k_tiles", nk=8191)
    d = G.device_inputs(w)
    plan = G.build_plan(w, d, 128, tk)
    assert plan.info.nk_max == 8191
    G.compare_plan(plan.export(), oracle.build_plan(w, 128, tk))
    rows = np.array([[q, 0] for q in (0, 3, 7, 8, 9, 64, 126, 127)], np.int64)
    O, L = oracle.attention(w, rows=rows)
    for sp in (None, 0):
        o, lse = G.run_attention(w, d, plan, **({} if sp is None else {"num_splits": sp}))
        torch.cuda.synchronize()
        lse_np = lse.cpu().numpy().astype(np.float64)
        assert np.isfinite(lse_np).all()
        G.compare_attention(w, O, L, G.flat_o(w, o)[rows[:, 0], rows[:, 1]],
                            lse_np[rows[:, 1], rows[:, 0]], "8191 K tiles S=%s" % sp)


def test_zero_length_sequences():
    import mask_planned_block_amd as mpb
    # Sq = 0: no plan rows; the forward and the Split-K forward are no-ops
    w = W.custom(np.zeros((1, 1, 0), np.int32), batch=2, seqlen_q=0, seqlen_k=300, heads_q=2,
                 head_dim=128, dtype=W.DTYPE_BF16, seed=43)
    _case("sq0")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    assert int(plan.info.header[0]) == 0 and plan.info.num_tasks == 0
    o, lse = G.run_attention(w, d, plan)
    o2, l2 = G.run_attention(w, d, plan, num_splits=4)
    torch.cuda.synchronize()
    assert o.numel() == 0 and lse.numel() == 0 and o2.numel() == 0
    # Sk = 0: every row sees nothing (all endpoints 0): O = 0, LSE = -inf
    w = W.custom(np.zeros((1, 3, 2 * 150), np.int32), batch=2, seqlen_q=150, seqlen_k=0,
                 heads_q=2, head_dim=128, dtype=W.DTYPE_BF16, seed=44)
    _case("sk0")
    d = G.device_inputs(w)
    plan = G.build_plan(w, d)
    pl = plan.problem
    G.compare_plan(plan.export(), oracle.build_plan(w, pl.tile_q, pl.tile_k))
    O, L = oracle.attention(w)
    for sp in (None, 3):
        o, lse = G.run_attention(w, d, plan, **({} if sp is None else {"num_splits": sp}))
        torch.cuda.synchronize()
        assert torch.all(o == 0).item() and torch.all(lse == -float("inf")).item()
        G.compare_attention(w, O, L, G.flat_o(w, o), lse.cpu().numpy().astype(np.float64),
                            "Sk=0 S=%s" % sp)


def test_backward_zero_length_sides():
    """Backward with no Q rows: every K row sees nothing, dK = dV = 0; with
    no keys: every row is empty, dQ = 0."""
    import mask_planned_block_amd as mpb
    for sq, sk in ((0, 300), (150, 0)):
        nf = np.zeros((1, 1, 2 * sq), np.int32)
        w = W.custom(nf, batch=2, seqlen_q=sq, seqlen_k=sk, heads_q=2, head_dim=128,
                     dtype=W.DTYPE_BF16, seed=45)
        _case("bwd_empty_side", sq=sq, sk=sk)
        d = G.device_inputs(w)
        plan = G.build_plan(w, d, build_backward=True)
        o, lse = G.run_attention(w, d, plan)
        dout = torch.from_numpy(W.grad_output(w)).to(torch.bfloat16).reshape(d["q"].shape).cuda()
        dq, dk, dv = mpb.flex_attn_bwd(plan, d["q"], d["k"], d["v"], o, lse, dout, scale=w.scale)
        torch.cuda.synchronize()
        for t in (dq, dk, dv):
            assert torch.all(t == 0).item()

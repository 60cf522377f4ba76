"""Pins of the oracle's attention backward (CPU only).

The backward is the gradient of FlexAttention Eq. 1 (softmax(mod(Q K^T *
scale)) V) for an incoming dO, with the score_mod's own derivative (softcap:
1 - tanh^2 of its argument; ALiBi: a constant shift).  It is pinned by
things other than its own formula:
  * central differences of the oracle's forward (L = sum dO . O), with
    Richardson extrapolation, on tiny varlen GQA cases for every score_mod
    combination;
  * torch autograd in float64 through a dense masked softmax written with
    library primitives (a different computation of the same derivative);
  * closed forms: a row that sees one key contributes nothing to dQ and its
    dO to that key's dV; without a score_mod the per-row softmax gradient
    sums to zero, so dK summed over a sample's keys vanishes.
"""
import numpy as np
import pytest

import oracle
import workloads as W


def _tiny(variant, seed=3):
    lens_q, lens_k = [5, 3, 4], [6, 4, 1]
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    rng = np.random.default_rng(seed)
    mf = np.zeros((2, 3, int(cq[-1])), np.int32)
    for b in range(3):
        for t in range(cq[b], cq[b + 1]):
            mf[:, :, t] = np.sort(rng.integers(0, lens_k[b] + 1, size=(2, 3)), axis=1)
    mf[:, :, 1] = 0                     # a fully masked row
    mf[:, :, 2] = [1, 2, 2]             # a row that sees key 0 only
    kw = dict(layout=W.LAYOUT_THD, cu_seqlens_q=cq, cu_seqlens_k=ck, heads_q=2, heads_k=1,
              head_dim=4, dtype=W.DTYPE_FP32, seed=seed, scale=0.7)
    if variant in ("softcap", "both", "both_first"):
        kw["softcap"] = 1.5
    if variant in ("alibi", "both", "both_first"):
        kw["alibi"] = np.array([0.25, -0.5], np.float32)
    if variant == "both_first":
        kw["alibi_before_softcap"] = True
    w = W.custom(mf, **kw)
    return w, W.grad_output(w).astype(np.float32)


def _loss(w, do):
    o, _ = oracle.attention(w, nthreads=1)
    return float(np.sum(o * do))


@pytest.mark.parametrize("variant", ["none", "softcap", "alibi", "both", "both_first"])
def test_bwd_matches_central_differences(variant):
    w, do = _tiny(variant)
    dq, dk, dv = oracle.attention_bwd(w, do, nthreads=1)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        x = getattr(w, name)
        fd = np.zeros_like(grad)
        for idx in np.ndindex(x.shape):
            est = []
            for h in (2.0 ** -7, 2.0 ** -8):   # exact float32 perturbations
                old = x[idx]
                x[idx] = old + h
                lp = _loss(w, do)
                x[idx] = old - h
                lm = _loss(w, do)
                x[idx] = old
                est.append((lp - lm) / (2 * h))
            fd[idx] = (4 * est[1] - est[0]) / 3   # Richardson: O(h^4)
        err = float(np.max(np.abs(fd - grad)))
        assert err < 1e-7 * (1 + float(np.max(np.abs(grad)))), (variant, name, err)


def _dense_visible(w):
    """[Hm][total_q][total_k] bool from the endpoints (the interval union of
    the mask representation: column k visible iff an even number of a row's
    endpoints are <= k), within the row's own sample."""
    vis = np.zeros((w.mask_heads, w.total_q, w.total_k), bool)
    for b in range(w.batch):
        qo, ql, ko, kl = w.sample_bounds(b)
        cols = np.arange(kl)
        for t in range(qo, qo + ql):
            for hm in range(w.mask_heads):
                cnt = (w.mask_func[hm, :, t][:, None] <= cols[None, :]).sum(axis=0)
                vis[hm, t, ko:ko + kl] = cnt % 2 == 0
    return vis


@pytest.mark.parametrize("variant", ["none", "softcap", "alibi", "both", "both_first"])
def test_bwd_matches_torch_autograd(variant):
    torch = pytest.importorskip("torch")
    B, S, Sk, Hq, Hk, d = 2, 40, 33, 4, 2, 16
    rng = np.random.default_rng(11)
    mf = np.sort(rng.integers(0, Sk + 1, size=(Hq, 5, B * S)), axis=1).astype(np.int32)
    mf[:, :, 7] = 0
    kw = dict(batch=B, seqlen_q=S, seqlen_k=Sk, heads_q=Hq, heads_k=Hk, head_dim=d,
              dtype=W.DTYPE_FP32, seed=5)
    if variant in ("softcap", "both", "both_first"):
        kw["softcap"] = 2.0
    if variant in ("alibi", "both", "both_first"):
        kw["alibi"] = True
    if variant == "both_first":
        kw["alibi_before_softcap"] = True
    w = W.custom(mf, **kw)
    do = W.grad_output(w)
    dq, dk, dv = oracle.attention_bwd(w, do)

    vis = torch.from_numpy(_dense_visible(w))
    q = torch.tensor(w.q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(w.k, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(w.v, dtype=torch.float64, requires_grad=True)
    grp = Hq // Hk
    kx = k.repeat_interleave(grp, dim=1)           # [Tk, Hq, d]
    vx = v.repeat_interleave(grp, dim=1)
    s = torch.einsum("qhd,khd->hqk", q, kx) * w.scale
    qpos = torch.tensor([t % S for t in range(B * S)], dtype=torch.float64)
    kpos = torch.tensor([t % Sk for t in range(B * Sk)], dtype=torch.float64)
    bias = None
    if w.alibi_slopes is not None:
        sl = torch.tensor(w.alibi_slopes, dtype=torch.float64)
        bias = sl[:, None, None] * (kpos[None, None, :] - qpos[None, :, None])
    if bias is not None and w.alibi_before_softcap:
        s = s + bias
    if w.softcap > 0:
        s = w.softcap * torch.tanh(s / w.softcap)
    if bias is not None and not w.alibi_before_softcap:
        s = s + bias
    m = vis if w.mask_heads == Hq else vis.expand(Hq, -1, -1)
    s = s.masked_fill(~m, float("-inf"))
    any_row = m.any(dim=-1, keepdim=True)
    p = torch.softmax(torch.where(any_row, s, torch.zeros_like(s)), dim=-1)
    p = torch.where(m, p, torch.zeros_like(p))
    o = torch.einsum("hqk,khd->qhd", p, vx)
    (o * torch.from_numpy(do.astype(np.float64))).sum().backward()
    for name, mine, ref in (("q", dq, q.grad), ("k", dk, k.grad), ("v", dv, v.grad)):
        err = float(np.max(np.abs(mine - ref.numpy())))
        assert err < 1e-11 * (1 + float(np.max(np.abs(mine)))), (variant, name, err)


def test_single_visible_key_and_zero_row_sums():
    # causal: row 0 of each sample sees key 0 only
    B, S, d = 2, 24, 8
    q_local = np.tile(np.arange(S), B)
    mf = (q_local + 1).reshape(1, 1, -1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=S, seqlen_k=S, heads_q=3, head_dim=d,
                 dtype=W.DTYPE_FP32, seed=9)
    do = W.grad_output(w)
    dq, dk, dv = oracle.attention_bwd(w, do)
    for b in range(B):
        assert np.all(dq[b * S] == 0.0)          # P = 1: dS = P (dP - D) = 0
    # dV of the last key of a sample only gets the last row's weight
    o, lse = oracle.attention(w)
    for b in range(B):
        last = b * S + S - 1
        for h in range(3):
            qv = w.q[last, h].astype(np.float64)
            kv = w.k[last, h].astype(np.float64)
            p = np.exp(w.scale * qv @ kv - lse[h, last])
            np.testing.assert_allclose(dv[last, h], p * do[last, h], rtol=1e-12, atol=1e-14)
    # no score_mod: every row's softmax gradient sums to zero, so does dK
    # summed over the keys of a sample
    for b in range(B):
        np.testing.assert_allclose(dk[b * S:(b + 1) * S].sum(axis=0), 0.0, atol=1e-12)


@pytest.mark.parametrize("variant", ["none", "both_first"])
def test_selected_dq_rows_match_full_backward(variant):
    w, do = _tiny(variant)
    _, _, _ = oracle.attention_bwd(w, do, nthreads=1)
    dq = oracle.attention_bwd(w, do, nthreads=2)[0]
    rows = np.array([[t, h] for t in range(w.total_q) for h in range(w.heads_q)][::-1])
    got = oracle.attention_bwd_dq_rows(w, do, rows, nthreads=3)
    for n, (t, h) in enumerate(rows):
        assert np.array_equal(got[n], dq[t, h])


@pytest.mark.parametrize("variant", ["none", "softcap", "alibi", "both", "both_first"])
def test_selected_dkdv_rows_match_full_backward(variant):
    """dK/dV of selected K rows (recomputing each Q row that sees the key)
    equal the full backward's rows bit for bit, for every key of a varlen
    case with empty, fully masked and single-key rows, in any row order."""
    w, do = _tiny(variant)
    _, dk, dv = oracle.attention_bwd(w, do, nthreads=1)
    rows = np.array([[t, g] for t in range(w.total_k) for g in range(w.heads_k)])[::-1]
    gk, gv = oracle.attention_bwd_dkdv_rows(w, do, rows, nthreads=3)
    for n, (t, g) in enumerate(rows):
        assert np.array_equal(gk[n], dk[t, g]) and np.array_equal(gv[n], dv[t, g]), (t, g)


def test_selected_dkdv_rows_gqa_bshd():
    """The same on a fixed-length GQA case (four Q heads on two K/V heads,
    per-head masks) with the rows sampled unevenly over samples and heads."""
    B, S, Sk, Hq, Hk = 2, 30, 26, 4, 2
    rng = np.random.default_rng(21)
    mf = np.sort(rng.integers(0, Sk + 1, size=(Hq, 5, B * S)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=S, seqlen_k=Sk, heads_q=Hq, heads_k=Hk, head_dim=8,
                 dtype=W.DTYPE_FP32, seed=13, softcap=3.0, alibi=True)
    do = W.grad_output(w)
    _, dk, dv = oracle.attention_bwd(w, do)
    rows = np.array([[0, 0], [25, 1], [26, 1], [51, 0], [13, 1], [13, 0], [40, 1]])
    gk, gv = oracle.attention_bwd_dkdv_rows(w, do, rows)
    for n, (t, g) in enumerate(rows):
        assert np.array_equal(gk[n], dk[t, g]) and np.array_equal(gv[n], dv[t, g]), (t, g)
    with pytest.raises(ValueError):
        oracle.attention_bwd_dkdv_rows(w, do, np.array([[B * Sk, 0]]))

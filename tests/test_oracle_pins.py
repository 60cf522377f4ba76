"""Pins for the CPU oracle (no GPU).

The oracle is checked against what the pages and the mathematics fix, never
against itself: the worked endpoint example of the mask plan design page,
set-union semantics by exhaustive enumeration, tile classes by brute force on a
dense boolean matrix, closed forms for causal tiles, and a textbook dense
softmax attention (numpy, additive 0/-inf bias) for the attention rows.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W


# ------------------------------------------------------------------ helpers

def set_union_visible(endpoints, k_len):
    """visible(q) = [0,F0) U [F1,F2) U ... as a Python set."""
    F = list(endpoints)
    s = set(range(0, F[0]))
    for i in range(1, len(F) - 1, 2):
        s |= set(range(F[i], F[i + 1]))
    return {k for k in s if k < k_len}


def dense_mask(w):
    """Dense boolean [mask_heads][total_q][k_len of owner] as a list of arrays
    per (hm, token), built from Python set unions."""
    out = {}
    for hm in range(w.mask_heads):
        for b in range(w.batch):
            qo, ql, ko, kl = w.sample_bounds(b)
            for q in range(ql):
                F = w.mask_func[hm, :, qo + q]
                row = np.zeros(kl, dtype=bool)
                for kk in set_union_visible(F, kl):
                    row[kk] = True
                out[(hm, qo + q)] = row
    return out


def textbook_attention(w, bias_fn=None, mask=None):
    """Dense softmax attention per sample/head with numpy in float64:
    S = scale*Q K^T (+ score_mod), additive 0/-inf mask bias, softmax, P V."""
    d = w.head_dim
    O = np.zeros((w.total_q, w.heads_q, d))
    L = np.zeros((w.heads_q, w.total_q))
    mask = dense_mask(w) if mask is None else mask
    g = w.heads_q // w.heads_k
    for b in range(w.batch):
        qo, ql, ko, kl = w.sample_bounds(b)
        for h in range(w.heads_q):
            hm = 0 if w.mask_heads == 1 else h
            Q = w.q[qo:qo + ql, h, :].astype(np.float64)
            K = w.k[ko:ko + kl, h // g, :].astype(np.float64)
            V = w.v[ko:ko + kl, h // g, :].astype(np.float64)
            S = w.scale * (Q @ K.T)
            qi = np.arange(ql)[:, None]
            ki = np.arange(kl)[None, :]
            if bias_fn is not None:
                S = bias_fn(S, h, qi, ki)
            M = np.stack([mask[(hm, qo + q)] for q in range(ql)]) if ql else np.zeros((0, kl), bool)
            S = np.where(M, S, -np.inf)
            for q in range(ql):
                row = S[q]
                if not np.isfinite(row).any():
                    O[qo + q, h] = 0.0
                    L[h, qo + q] = -np.inf
                    continue
                m = row.max()
                e = np.exp(row - m)
                O[qo + q, h] = (e @ V) / e.sum()
                L[h, qo + q] = m + math.log(e.sum())
    return O, L


def brute_force_classes(w, tile_q, tile_k):
    """Tile classes from the dense boolean matrix: 0 empty, 1 partial, 2 full."""
    mask = dense_mask(w)
    out = []
    for hm in range(w.mask_heads):
        per = []
        for b in range(w.batch):
            qo, ql, ko, kl = w.sample_bounds(b)
            M = np.zeros((max(ql, 0), kl), bool)
            for q in range(ql):
                M[q] = mask[(hm, qo + q)]
            for i in range(-(-ql // tile_q)):
                row = []
                for j in range(-(-kl // tile_k)):
                    blk = M[i * tile_q:(i + 1) * tile_q, j * tile_k:(j + 1) * tile_k]
                    whole = blk.shape == (tile_q, tile_k)
                    if not blk.any():
                        row.append(0)
                    elif whole and blk.all():
                        row.append(2)
                    else:
                        row.append(1)
                per.append((b, i, row))
        out.append(per)
    return out


# ------------------------------------------------------------------ expand

def test_p1_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p1_interval_example.json")))
    for k_len in (96, 128):
        vis = oracle.expand_row(g["endpoints"], k_len)
        want = np.zeros(k_len, bool)
        for a, b in g["visible_intervals"]:
            want[a:b] = True
        assert np.array_equal(vis, want)


@pytest.mark.parametrize("nfunc", [1, 3, 5])
def test_expand_exhaustive_set_union(nfunc):
    for k_len in range(0, 7):
        for F in itertools.combinations_with_replacement(range(k_len + 1), nfunc):
            vis = oracle.expand_row(F, k_len)
            want = set_union_visible(F, k_len)
            assert set(np.flatnonzero(vis).tolist()) == want, (F, k_len)


def test_equal_endpoint_pairs_are_empty():
    base = [3, 7, 11]
    k_len = 16
    ref = oracle.expand_row(base, k_len)
    for pos in range(1, len(base) + 1):
        for val in range(0, 17):
            F = base[:pos] + [val, val] + base[pos:]
            if all(F[i] <= F[i + 1] for i in range(len(F) - 1)):
                assert np.array_equal(oracle.expand_row(F, k_len), ref), F


# ------------------------------------------------------------------ validate

def _one_row(endpoints, k_len, layout=W.LAYOUT_BSHD):
    mf = np.asarray(endpoints, np.int32).reshape(1, -1, 1)
    return W.custom(mf, batch=1, seqlen_q=1, seqlen_k=k_len, head_dim=32, with_values=False)


@pytest.mark.parametrize("ep,k_len,err", [
    ([4], 8, 0), ([0], 8, 0), ([8], 8, 0), ([9], 8, oracle.ERR_RANGE), ([-1], 8, oracle.ERR_RANGE),
    ([2, 5, 7], 8, 0), ([5, 2, 7], 8, oracle.ERR_ORDER), ([2, 5, 9], 8, oracle.ERR_RANGE),
    ([5, -1, 2], 8, oracle.ERR_RANGE | oracle.ERR_ORDER), ([3, 3, 3], 8, 0),
    ([0, 0, 0], 0, 0), ([1], 0, oracle.ERR_RANGE),
])
def test_validate_endpoints(ep, k_len, err):
    assert oracle.validate(_one_row(ep, k_len)) == err


@pytest.mark.parametrize("cu_q,cu_k,maxq,maxk,bad", [
    ([0, 3, 5], [0, 4, 6], 3, 4, False),
    ([1, 3, 5], [0, 4, 6], 3, 4, True),        # does not start at 0
    ([0, 3, 5], [0, 4, 7], 3, 4, True),        # does not end at total_k (6)
    ([0, 4, 3], [0, 4, 6], 4, 4, True),        # decreasing
    ([0, 3, 5], [0, 4, 6], 2, 4, True),        # longer than max_seqlen_q
    ([0, 0, 5], [0, 0, 6], 5, 6, False),       # empty sample is legal
])
def test_validate_seqlens(cu_q, cu_k, maxq, maxk, bad):
    total_q = 5
    mf = np.zeros((1, 1, total_q), np.int32)
    w = W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=[0, 3, 5], cu_seqlens_k=[0, 4, 6],
                 head_dim=32, with_values=False)
    w.cu_seqlens_q = np.asarray(cu_q, np.int32)
    w.cu_seqlens_k = np.asarray(cu_k, np.int32)
    w.total_k = 6
    w.seqlen_q, w.seqlen_k = maxq, maxk
    e = oracle.validate(w)
    assert (e == oracle.ERR_SEQLENS) == bad


# ------------------------------------------------------------------ classify / pack / CSR

def _check_plan_against_brute_force(w, tq, tk):
    P = oracle.build_plan(w, tq, tk, nthreads=2)
    assert P.err == 0
    bf = brute_force_classes(w, tq, tk)
    words = tk // 32
    mask = dense_mask(w)
    for hm in range(w.mask_heads):
        for (b, i, row) in bf[hm]:
            grow = int(P.cu_rows[b]) + i
            flat = hm * P.rows_total + grow
            got = P.cls[hm, grow, :len(row)].tolist()
            assert got == row, (hm, b, i)
            assert all(c == 0 for c in P.cls[hm, grow, len(row):])
            pidx = P.p_idx[P.p_off[flat]:P.p_off[flat + 1]].tolist()
            fidx = P.f_idx[P.f_off[flat]:P.f_off[flat + 1]].tolist()
            assert pidx == [j for j, c in enumerate(row) if c == 1]
            assert fidx == [j for j, c in enumerate(row) if c == 2]
            qo, ql, ko, kl = w.sample_bounds(b)
            for n, j in enumerate(pidx):
                words_arr = P.p_masks[P.p_off[flat] + n]
                for r in range(tq):
                    for c in range(tk):
                        bit = (int(words_arr[r, c // 32]) >> (c % 32)) & 1
                        q, kk = i * tq + r, j * tk + c
                        want = q < ql and kk < kl and bool(mask[(hm, qo + q)][kk])
                        assert bit == int(want), (hm, b, i, j, r, c)
    assert P.p_masks.shape[1:] == (tq, words)
    return P


@pytest.mark.parametrize("tq,tk", [(32, 32), (64, 32), (32, 64)])
def test_classify_pack_brute_force_random_intervals(tq, tk):
    rng = np.random.default_rng(5)
    B, Sq, Sk, nfunc = 2, 75, 101, 5
    mf = np.sort(rng.integers(0, Sk + 1, size=(2, nfunc, B * Sq)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=Sq, seqlen_k=Sk, heads_q=2, head_dim=32, with_values=False)
    _check_plan_against_brute_force(w, tq, tk)


def test_classify_pack_brute_force_varlen():
    rng = np.random.default_rng(11)
    lens = [40, 0, 97, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    mf = np.zeros((1, 3, total), np.int32)
    for b, L in enumerate(lens):
        if L:
            mf[0, :, cu[b]:cu[b + 1]] = np.sort(rng.integers(0, L + 1, size=(3, L)), axis=0)
    w = W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=cu, cu_seqlens_k=cu, head_dim=32,
                 with_values=False)
    P = _check_plan_against_brute_force(w, 32, 32)
    assert P.cu_rows.tolist() == [0, 2, 2, 6, 8]
    # per-sample descriptor {q_off, k_off, q_len, k_len, row_begin, rows, k_tiles, 0},
    # written out by hand from the prefix: rows = ceil(q_len/32), k_tiles = ceil(k_len/32)
    assert P.seqdesc.tolist() == [[0, 0, 40, 40, 0, 2, 2, 0],
                                  [40, 40, 0, 0, 2, 0, 0, 0],
                                  [40, 40, 97, 97, 2, 4, 4, 0],
                                  [137, 137, 33, 33, 6, 2, 2, 0]]


def test_seqdesc_closed_form():
    """The per-sample descriptor for Q and K split differently (THD, an
    empty Q side, an empty K side, ragged lengths, tile_q != tile_k) and for
    fixed-length BSHD, against values written out by hand: offsets from the
    prefixes, row_begin the running sum of ceil(q_len / T_Q), rows =
    ceil(q_len / T_Q), k_tiles = ceil(k_len / T_KV)."""
    rng = np.random.default_rng(4)
    cq = np.array([0, 5, 75, 75], np.int32)
    ck = np.array([0, 64, 64, 97], np.int32)
    klen = [64, 0, 33]
    mf = np.zeros((1, 3, 75), np.int32)
    for b in range(3):
        for t in range(cq[b], cq[b + 1]):
            mf[0, :, t] = np.sort(rng.integers(0, klen[b] + 1, size=3))
    w = W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=cq, cu_seqlens_k=ck, head_dim=32,
                 with_values=False)
    P = oracle.build_plan(w, 64, 32, nthreads=2)
    assert P.err == 0
    assert P.seqdesc.tolist() == [[0, 0, 5, 64, 0, 1, 2, 0],
                                  [5, 64, 70, 0, 1, 2, 0, 0],
                                  [75, 64, 0, 33, 3, 0, 2, 0]]
    assert P.cu_rows.tolist() == [0, 1, 3, 3]
    # fixed length: B=3, Sq=50, Sk=70 at 32x32
    mfb = np.sort(rng.integers(0, 71, size=(1, 3, 150)), axis=1).astype(np.int32)
    wb = W.custom(mfb, batch=3, seqlen_q=50, seqlen_k=70, head_dim=32, with_values=False)
    Pb = oracle.build_plan(wb, 32, 32, nthreads=2)
    assert Pb.seqdesc.tolist() == [[0, 0, 50, 70, 0, 2, 3, 0],
                                   [50, 70, 50, 70, 2, 2, 3, 0],
                                   [100, 140, 50, 70, 4, 2, 3, 0]]
    assert Pb.cu_rows.tolist() == [0, 2, 4, 6]


def test_causal_closed_form():
    # Square causal mask, T_Q = T_KV = T, S a multiple of T: tile (i, j) is full
    # iff j < i, partial iff j == i, empty iff j > i.
    for S, T in [(256, 64), (256, 32), (128, 128)]:
        w = W.tiny_causal(seqlen=S, heads=1, with_values=False)
        P = oracle.build_plan(w, T, T, nthreads=2)
        n = S // T
        assert int(P.header[1]) == n and int(P.header[2]) == n * (n - 1) // 2
        for i in range(n):
            assert P.cls[0, i].tolist() == [2] * i + [1] + [0] * (n - i - 1)
    # 256-token causal at 64x64 tiles: 4 partial, 6 full, 6 empty.
    P = oracle.build_plan(W.tiny_causal(with_values=False), 64, 64)
    assert (int(P.header[1]), int(P.header[2])) == (4, 6)
    assert int((P.cls == 0).sum()) == 6


# ------------------------------------------------------------------ K2Q view

def _check_k2q_against_brute_force(w, tq, tk):
    """Backward K2Q view (mask plan design §4.4, §4.7) against tile classes
    and visibility taken from the dense boolean matrix."""
    V = oracle.build_k2q(w, tq, tk, nthreads=2)
    assert V is not None
    bf = brute_force_classes(w, tq, tk)
    mask = dense_mask(w)
    wq = tq // 32
    nks = [-(-w.sample_bounds(b)[3] // tk) for b in range(w.batch)]
    nqs = [-(-w.sample_bounds(b)[1] // tq) for b in range(w.batch)]
    assert V.cu_krows.tolist() == np.concatenate([[0], np.cumsum(nks)]).tolist()
    K = int(V.cu_krows[-1])
    assert int(V.header[0]) == sum(nqs) and int(V.header[1]) == K
    tot_p = tot_f = 0
    for hm in range(w.mask_heads):
        for b in range(w.batch):
            qo, ql, ko, kl = w.sample_bounds(b)
            rows = [row for (bb, i, row) in bf[hm] if bb == b]
            for j in range(nks[b]):
                flat = hm * K + int(V.cu_krows[b]) + j
                col = [row[j] for row in rows]
                pidx = V.p_idx[V.p_off[flat]:V.p_off[flat + 1]].tolist()
                fidx = V.f_idx[V.f_off[flat]:V.f_off[flat + 1]].tolist()
                assert pidx == [i for i, c in enumerate(col) if c == 1], (hm, b, j)
                assert fidx == [i for i, c in enumerate(col) if c == 2], (hm, b, j)
                tot_p += len(pidx)
                tot_f += len(fidx)
                for n, i in enumerate(pidx):
                    words = V.p_masks[V.p_off[flat] + n]
                    for r in range(tk):
                        for c in range(tq):
                            bit = (int(words[r, c // 32]) >> (c % 32)) & 1
                            q, kk = i * tq + c, j * tk + r
                            want = q < ql and kk < kl and bool(mask[(hm, qo + q)][kk])
                            assert bit == int(want), (hm, b, i, j, r, c)
    assert (int(V.header[2]), int(V.header[3])) == (tot_p, tot_f)
    assert V.p_masks.shape[1:] == (tk, wq)
    return V


@pytest.mark.parametrize("tq,tk", [(32, 32), (64, 32), (32, 64)])
def test_k2q_brute_force_random_intervals(tq, tk):
    rng = np.random.default_rng(7)
    B, Sq, Sk, nfunc = 2, 75, 101, 5
    mf = np.sort(rng.integers(0, Sk + 1, size=(2, nfunc, B * Sq)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=Sq, seqlen_k=Sk, heads_q=2, head_dim=32, with_values=False)
    _check_k2q_against_brute_force(w, tq, tk)


def test_k2q_brute_force_varlen():
    rng = np.random.default_rng(13)
    lq, lk = [40, 0, 97, 33], [50, 20, 0, 70]
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    mf = np.zeros((1, 3, int(cq[-1])), np.int32)
    for b, L in enumerate(lq):
        if L:
            mf[0, :, cq[b]:cq[b + 1]] = np.sort(rng.integers(0, lk[b] + 1, size=(3, L)), axis=0)
    w = W.custom(mf, layout=W.LAYOUT_THD, cu_seqlens_q=cq, cu_seqlens_k=ck, head_dim=32,
                 with_values=False)
    V = _check_k2q_against_brute_force(w, 32, 32)
    assert V.cu_krows.tolist() == [0, 2, 3, 3, 6]


def test_k2q_is_the_q2k_relation_transposed():
    # Design invariant 7: Q2K and K2Q describe the same block relation, and a
    # partial pair's K-major word bits are its Q-major bits transposed.
    rng = np.random.default_rng(17)
    B, S, nfunc, T = 2, 130, 7, 32
    mf = np.sort(rng.integers(0, S + 1, size=(1, nfunc, B * S)), axis=1).astype(np.int32)
    w = W.custom(mf, batch=B, seqlen_q=S, seqlen_k=S, heads_q=1, head_dim=32, with_values=False)
    P = oracle.build_plan(w, 64, T, nthreads=2)
    V = oracle.build_k2q(w, 64, T, nthreads=2)
    assert (int(P.header[1]), int(P.header[2])) == (int(V.header[2]), int(V.header[3]))
    K = int(V.cu_krows[-1])
    for b in range(B):
        for i in range(int(P.cu_rows[b + 1] - P.cu_rows[b])):
            qflat = int(P.cu_rows[b]) + i
            plist = P.p_idx[P.p_off[qflat]:P.p_off[qflat + 1]].tolist()
            for n, j in enumerate(plist):
                kflat = int(V.cu_krows[b]) + j
                kp = V.p_idx[V.p_off[kflat]:V.p_off[kflat + 1]].tolist()
                assert i in kp
                m = kp.index(i)
                qm = P.p_masks[P.p_off[qflat] + n]        # [64][1]
                km = V.p_masks[V.p_off[kflat] + m]        # [32][2]
                for r in range(64):
                    for c in range(T):
                        assert ((int(qm[r, c // 32]) >> (c % 32)) & 1) == \
                            ((int(km[c, r // 32]) >> (r % 32)) & 1)
            flist = P.f_idx[P.f_off[qflat]:P.f_off[qflat + 1]].tolist()
            for j in flist:
                kflat = int(V.cu_krows[b]) + j
                assert i in V.f_idx[V.f_off[kflat]:V.f_off[kflat + 1]].tolist()
    assert K == B * (-(-S // T))


def test_k2q_causal_closed_form():
    # Square causal mask, T_Q = T_KV = T, S a multiple of T: K row j is
    # partial for Q tile j alone and full for every Q tile after it.
    for S, T in [(256, 64), (256, 32)]:
        w = W.tiny_causal(seqlen=S, heads=1, with_values=False)
        V = oracle.build_k2q(w, T, T, nthreads=2)
        n = S // T
        for j in range(n):
            assert V.p_idx[V.p_off[j]:V.p_off[j + 1]].tolist() == [j]
            assert V.f_idx[V.f_off[j]:V.f_off[j + 1]].tolist() == list(range(j + 1, n))
        # the diagonal tile's K-major predicate: column (Q row) c sees K row r iff r <= c
        for j in range(n):
            km = V.p_masks[V.p_off[j]]
            for r in range(T):
                bits = [(int(km[r, c // 32]) >> (c % 32)) & 1 for c in range(T)]
                assert bits == [int(r <= c) for c in range(T)]


def test_tail_tile_never_full():
    # Every in-bound element visible, but the tile sticks out past k_len: partial.
    w = W.custom(np.full((1, 1, 64), 40, np.int32), batch=1, seqlen_q=64, seqlen_k=40,
                 head_dim=32, with_values=False)
    P = oracle.build_plan(w, 64, 64)
    assert P.cls[0, 0].tolist() == [1]
    # ... and past q_len (q_len=40 < T_Q=64) likewise.
    w = W.custom(np.full((1, 1, 40), 64, np.int32), batch=1, seqlen_q=40, seqlen_k=64,
                 head_dim=32, with_values=False)
    P = oracle.build_plan(w, 64, 64)
    assert P.cls[0, 0].tolist() == [1]


def test_payload_invariants_and_size(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p1_payload_size.json")))
    tq, tk = g["tile_q"], g["tile_k"]
    w = W.make("window_sink", small=True, with_values=False)
    P = oracle.build_plan(w, tq, tk)
    assert P.p_masks.shape[1] * P.p_masks.shape[2] * 4 == g["payload_bytes_per_partial_tile"]
    # popcount of all payloads + full tiles * T_Q*T_KV == number of visible pairs
    pop = sum(bin(int(x)).count("1") for x in P.p_masks.ravel())
    visible = sum(int(r.sum()) for r in dense_mask(w).values())
    assert pop + int(P.header[2]) * tq * tk == visible


def test_hmask_one_equals_replicated():
    w1 = W.make("window_sink", small=True, with_values=False)
    wr = W.custom(np.repeat(w1.mask_func, w1.heads_q, axis=0), batch=w1.batch,
                  seqlen_q=w1.seqlen_q, seqlen_k=w1.seqlen_k, heads_q=w1.heads_q,
                  head_dim=w1.head_dim, with_values=False)
    P1 = oracle.build_plan(w1, 64, 64)
    Pr = oracle.build_plan(wr, 64, 64)
    n = P1.rows_total
    for h in range(w1.heads_q):
        assert np.array_equal(Pr.cls[h], P1.cls[0])
    assert int(Pr.header[1]) == w1.heads_q * int(P1.header[1])


# ------------------------------------------------------------------ attention

def _rel(a, b):
    return np.max(np.abs(a - b))


def test_all_visible_equals_textbook():
    S, H, d = 70, 2, 32
    mf = np.full((1, 1, 2 * S), S, np.int32)
    w = W.custom(mf, batch=2, seqlen_q=S, seqlen_k=S, heads_q=H, head_dim=d, seed=3)
    O, L = oracle.attention(w)
    # textbook softmax attention without any mask code
    for b in range(2):
        for h in range(H):
            Q = w.q[b * S:(b + 1) * S, h].astype(np.float64)
            K = w.k[b * S:(b + 1) * S, h].astype(np.float64)
            V = w.v[b * S:(b + 1) * S, h].astype(np.float64)
            Sc = w.scale * Q @ K.T
            P = np.exp(Sc - Sc.max(1, keepdims=True))
            ref = (P / P.sum(1, keepdims=True)) @ V
            lse = np.log(np.exp(Sc).sum(1))
            assert _rel(O[b * S:(b + 1) * S, h], ref) < 1e-12
            assert _rel(L[h, b * S:(b + 1) * S], lse) < 1e-12


def test_causal_equals_triangular_and_first_row():
    w = W.tiny_causal(seqlen=50, heads=2, head_dim=16, seed=1)
    O, L = oracle.attention(w)
    for h in range(2):
        Q = w.q[:, h].astype(np.float64)
        K = w.k[:, h].astype(np.float64)
        V = w.v[:, h].astype(np.float64)
        Sc = w.scale * Q @ K.T
        Sc = np.where(np.tril(np.ones((50, 50), bool)), Sc, -np.inf)
        P = np.exp(Sc - Sc.max(1, keepdims=True))
        ref = (P / P.sum(1, keepdims=True)) @ V
        assert _rel(O[:, h], ref) < 1e-12
        # row 0 sees only key 0
        assert np.array_equal(O[0, h], V[0])
        assert abs(L[h, 0] - w.scale * float(Q[0] @ K[0])) < 1e-12


def test_random_intervals_equal_dense_bias_and_normalise():
    rng = np.random.default_rng(7)
    B, S, H, d = 2, 45, 2, 16
    mf = np.sort(rng.integers(0, S + 1, size=(H, 5, B * S)), axis=1).astype(np.int32)
    mf[:, :, 3] = 0  # a fully masked row
    w = W.custom(mf, batch=B, seqlen_q=S, seqlen_k=S, heads_q=H, head_dim=d, seed=9)
    O, L = oracle.attention(w)
    Oref, Lref = textbook_attention(w)
    fin = np.isfinite(Lref)
    assert np.array_equal(np.isfinite(L), fin)
    assert _rel(O, Oref) < 1e-12 and _rel(L[fin], Lref[fin]) < 1e-12
    assert np.all(O[3] == 0.0) and np.all(L[:, 3] == -np.inf)
    # sum over visible keys of exp(score - LSE) == 1
    mask = dense_mask(w)
    for (hm, t), row in mask.items():
        if not row.any():
            continue
        b = t // S
        Sc = w.scale * w.k[b * S:(b + 1) * S, hm].astype(np.float64) @ w.q[t, hm].astype(np.float64)
        assert abs(np.exp(Sc[row] - L[hm, t]).sum() - 1.0) < 1e-12


def test_alibi_sign_and_row_shift():
    # slope*(k-q) differs from slope*k by a per-row constant: O unchanged,
    # LSE shifted by +slope*q relative to the slope*k reference.
    w = W.tiny_causal(seqlen=40, heads=2, head_dim=16, seed=4)
    w.alibi_slopes = np.asarray([0.5, 0.125], np.float32)
    O, L = oracle.attention(w)
    Oref, Lref = textbook_attention(
        w, bias_fn=lambda S, h, qi, ki: S + float(w.alibi_slopes[h]) * ki)
    assert _rel(O, Oref) < 1e-12
    q = np.arange(40)
    for h in range(2):
        assert _rel(L[h] + float(w.alibi_slopes[h]) * q, Lref[h]) < 1e-12


def test_softcap_limits_and_single_key_closed_form():
    w = W.tiny_causal(seqlen=30, heads=1, head_dim=16, seed=2)
    O0, L0 = oracle.attention(w)
    w.softcap = 1e12
    O1, L1 = oracle.attention(w)
    assert _rel(O0, O1) < 1e-12 and _rel(L0, L1) < 1e-9
    # row 0 sees only key 0: LSE = c*tanh(s/c) (softcap first) + slope*(0-0)
    c = 0.7
    w.softcap = c
    w.alibi_slopes = np.asarray([0.3], np.float32)
    s = w.scale * float(w.q[0, 0].astype(np.float64) @ w.k[0, 0].astype(np.float64))
    O, L = oracle.attention(w)
    assert abs(L[0, 0] - c * math.tanh(s / c)) < 1e-12
    assert np.all(np.abs(L[0, 1:] - np.log(np.arange(2, 31))) <= c + 0.3 * 30 + 1e-9)
    # ALiBi first: row 1, key 0 has bias slope*(0-1); order matters
    w.alibi_before_softcap = True
    Oa, La = oracle.attention(w)
    w.alibi_before_softcap = False
    s10 = w.scale * float(w.q[1, 0].astype(np.float64) @ w.k[0, 0].astype(np.float64))
    s11 = w.scale * float(w.q[1, 0].astype(np.float64) @ w.k[1, 0].astype(np.float64))
    sl = float(w.alibi_slopes[0])  # the float32 value the oracle reads
    first = np.logaddexp(c * math.tanh((s10 - sl) / c), c * math.tanh(s11 / c))
    after = np.logaddexp(c * math.tanh(s10 / c) - sl, c * math.tanh(s11 / c))
    assert abs(La[0, 1] - first) < 1e-9 and abs(L[0, 1] - after) < 1e-9


def test_varlen_equals_per_sample_fixed():
    w = W.make("varlen_doc", small=True)
    O, L = oracle.attention(w)
    for b in range(w.batch):
        qo, ql, ko, kl = w.sample_bounds(b)
        ws = W.custom(w.mask_func[:, :, qo:qo + ql], batch=1, seqlen_q=ql, seqlen_k=kl,
                      heads_q=w.heads_q, head_dim=w.head_dim, with_values=False)
        ws.q, ws.k, ws.v = w.q[qo:qo + ql], w.k[ko:ko + kl], w.v[ko:ko + kl]
        Os, Ls = oracle.attention(ws)
        assert np.array_equal(Os, O[qo:qo + ql]) and np.array_equal(Ls, L[:, qo:qo + ql])


def test_gqa_head_mapping():
    w = W.custom(np.full((1, 1, 20), 20, np.int32), batch=1, seqlen_q=20, seqlen_k=20, heads_q=4,
                 heads_k=2, head_dim=8, seed=6)
    O, L = oracle.attention(w)
    wr = W.custom(w.mask_func, batch=1, seqlen_q=20, seqlen_k=20, heads_q=4, heads_k=4,
                  head_dim=8, with_values=False)
    wr.q = w.q
    wr.k = np.repeat(w.k, 2, axis=1)
    wr.v = np.repeat(w.v, 2, axis=1)
    Or, Lr = oracle.attention(wr)
    assert np.array_equal(O, Or) and np.array_equal(L, Lr)


def test_selected_rows_match_full_run():
    w = W.make("prefix_softcap", small=True)
    rng = np.random.default_rng(0)
    rows = np.stack([rng.integers(0, w.total_q, 50), rng.integers(0, w.heads_q, 50)], 1)
    O, L = oracle.attention(w)
    Os, Ls = oracle.attention(w, rows=rows)
    assert np.array_equal(Os, O[rows[:, 0], rows[:, 1]])
    assert np.array_equal(Ls, L[rows[:, 1], rows[:, 0]])


def test_fully_masked_rows(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "p1_design_rules.json")))
    mf = np.zeros((1, 3, 10), np.int32)
    mf[0, :, 5:] = [[0], [2], [6]]
    w = W.custom(mf, batch=1, seqlen_q=10, seqlen_k=8, heads_q=1, head_dim=8)
    O, L = oracle.attention(w)
    assert g["empty_row"]["LSE"] == "-inf"
    assert np.all(O[:5] == g["empty_row"]["O"]) and np.all(L[0, :5] == -np.inf)
    assert np.all(np.isfinite(L[0, 5:]))

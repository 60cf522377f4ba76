"""Helpers for the GPU tests: move a seeded workload to the device, run the HIP
path through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

import mask_planned_block_amd as mpb
import workloads as W

TOL = {W.DTYPE_FP32: (1e-4, 1e-4), W.DTYPE_BF16: (2e-2, 1e-2)}   # (O, LSE) max-abs


def torch_dtype(w):
    return torch.bfloat16 if w.dtype == W.DTYPE_BF16 else torch.float32


def device_inputs(w, device="cuda"):
    return W.to_device(w, device)


def problem(w, tile_q=0, tile_k=0):
    return mpb.make_problem(w.layout, w.dtype, w.batch, w.seqlen_q, w.seqlen_k, w.total_q,
                            w.total_k, w.heads_q, w.heads_k, w.head_dim, w.mask_heads, w.nfunc,
                            tile_q, tile_k)


def build_plan(w, d, tile_q=0, tile_k=0, stream=None, build_backward=False, time_stages=False,
               pack_gqa=None, defer_header=False):
    return mpb.mask_plan_build(problem(w, tile_q, tile_k), d["mask_func"], d["cu_q"], d["cu_k"],
                               stream=stream, build_backward=build_backward,
                               time_stages=time_stages, pack_gqa=pack_gqa,
                               defer_header=defer_header)


def run_attention(w, d, plan, **kw):
    o, lse = mpb.flex_attn_fwd(plan, d["q"], d["k"], d["v"], scale=w.scale,
                               softcap=w.softcap if w.softcap > 0 else None,
                               alibi_slopes=d["slopes"],
                               alibi_before_softcap=w.alibi_before_softcap, **kw)
    return o, lse


def flat_o(w, o):
    """O as [total_q, Hq, d] float64 numpy."""
    return o.float().reshape(w.total_q, w.heads_q, w.head_dim).cpu().numpy().astype(np.float64)


def compare_plan(gp, op, with_k2q=False):
    """Bit-exact comparison of a GPU plan export with the oracle's plan
    (header slots 3..6 are zero unless the plan holds the K2Q view)."""
    assert gp["header"][7] == 0
    assert list(gp["header"][:3]) == [int(x) for x in op.header[:3]], (gp["header"], op.header)
    if not with_k2q:
        assert all(int(x) == 0 for x in gp["header"][3:7])
    for key in ("cu_rows", "seqdesc", "p_off", "f_off", "p_idx", "f_idx"):
        a, b = np.asarray(gp[key]), np.asarray(getattr(op, key))
        assert a.shape == b.shape and np.array_equal(a, b), key
    assert gp["p_masks"].shape == op.p_masks.shape
    assert np.array_equal(gp["p_masks"], op.p_masks), "payload words differ"


def snake_section(x, num_sections=8):
    """Section of flat (sample, KV head) index x = b*Hk + hk: blocks of
    num_sections go 0..7 when even and 7..0 when odd."""
    lo = x % num_sections
    return num_sections - 1 - lo if (x // num_sections) % 2 else lo


def check_schedule(w, gp, tile_q, num_sections=8):
    """The forward schedule is a permutation of all (row, head) tasks with the
    right q_valid_rows; positive-cost tasks sit in their (batch, kv-head)
    section (snake order over the flat index b*Hk + hk) in descending cost,
    ties by flat mask row (head-major) and then head; zero-cost tasks last,
    in the same tie order."""
    wd, so = gp["work_desc"], gp["section_off"]
    cu_rows, sd = gp["cu_rows"], gp["seqdesc"]
    rows_total = int(cu_rows[-1])
    n = rows_total * w.heads_q
    assert wd.shape == (n, 4) and so[0] == 0 and so[-1] == n
    assert np.all(np.diff(so) >= 0)
    p_off, f_off = gp["p_off"], gp["f_off"]
    group = w.heads_q // w.heads_k

    def cost(b, h, i):
        hm = 0 if w.mask_heads == 1 else h
        flat = hm * rows_total + int(cu_rows[b]) + i
        return int(p_off[flat + 1] - p_off[flat] + f_off[flat + 1] - f_off[flat])

    seen = set()
    for s in range(num_sections + 1):
        prev = None
        for t in range(so[s], so[s + 1]):
            i, h, b, qv = (int(x) for x in wd[t])
            assert (b, h, i) not in seen
            seen.add((b, h, i))
            q_len = int(sd[b][2])
            assert qv == min(tile_q, q_len - i * tile_q)
            c = cost(b, h, i)
            tie = (b, i, h) if w.mask_heads == 1 else (h, b, i)
            if s < num_sections:
                assert c > 0 and snake_section(b * w.heads_k + h // group, num_sections) == s
                key = (-c,) + tie
            else:
                assert c == 0
                key = tie
            assert prev is None or key > prev, (s, prev, key)
            prev = key
    assert len(seen) == n


def check_launch_order(w, gp, tile_q, num_sections=8):
    """Launch records: a permutation of the schedule with the sections
    interleaved (slot = sum_s' min(r, n_s') + #{s' < s : n_s' > r} for the
    r-th task of section s; zero-cost tasks last in schedule order), each
    record carrying the task's geometry, CSR ranges and first K tile."""
    wd, so, rec = gp["work_desc"], gp["section_off"], gp["launch"]
    n = wd.shape[0]
    assert rec.shape == (n, 16)
    sizes = np.diff(so)
    rows_total = int(gp["cu_rows"][-1])
    want = np.full(n, -1, np.int64)
    for s in range(num_sections + 1):
        for r in range(int(sizes[s])):
            t = int(so[s]) + r
            if s < num_sections:
                slot = sum(min(r, int(sizes[x])) for x in range(num_sections)) + \
                    sum(1 for x in range(s) if sizes[x] > r)
            else:
                slot = int(so[num_sections]) + r
            assert want[slot] == -1
            want[slot] = t
    for slot in range(n):
        t = want[slot]
        m_block, h, b, qv = (int(x) for x in wd[t])
        R = rec[slot]
        assert list(R[:4]) == [m_block, h, b, qv]
        sd = gp["seqdesc"][b]
        assert list(R[4:8]) == [int(sd[0]), int(sd[1]), int(sd[2]), int(sd[3])]
        hm = 0 if w.mask_heads == 1 else h
        flat = hm * rows_total + int(sd[4]) + m_block
        pb, pe = int(gp["p_off"][flat]), int(gp["p_off"][flat + 1])
        fb, fe = int(gp["f_off"][flat]), int(gp["f_off"][flat + 1])
        assert list(R[8:12]) == [pb, pe - pb, fb, fe - fb]
        first = int(gp["p_idx"][pb]) if pe > pb else (int(gp["f_idx"][fb]) if fe > fb else -1)
        assert int(R[12]) == first
        assert int(R[13]) == hm and int(R[14]) == h // (w.heads_q // w.heads_k)
        assert 0 <= int(R[15]) <= num_sections


def compare_attention(w, o_ref, lse_ref, o_gpu, lse_gpu, what=""):
    """Max-abs comparison at the stated tolerance; empty rows must be exactly
    O = 0 and LSE = -inf on both sides."""
    tol_o, tol_l = TOL[w.dtype]
    empty = ~np.isfinite(lse_ref)
    assert np.array_equal(~np.isfinite(lse_gpu), empty), what + " non-finite LSE pattern differs"
    assert np.all(lse_gpu[empty] == -np.inf)
    if empty.any():
        # LSE is [Hq, T] (or [n]); O is [T, Hq, d] (or [n, d])
        empty_o = empty.T if empty.ndim == 2 else empty
        assert np.all(o_gpu[empty_o] == 0.0), what + " empty rows must be O = 0"
    fin = ~empty
    assert not np.isnan(o_gpu).any(), what + " NaN in O"
    do = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    dl = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert do <= tol_o, "%s max|dO| = %.3g > %.3g" % (what, do, tol_o)
    assert dl <= tol_l, "%s max|dLSE| = %.3g > %.3g" % (what, dl, tol_l)
    return do, dl


def sample_rows(w, n_random=1500, seed=0, tile_q=128):
    """(token, head) pairs: random ones plus the edges of every sample and of
    Q tiles (first/last rows, rows on both sides of a tile boundary)."""
    rng = np.random.default_rng(seed)
    rows = set()
    for _ in range(n_random):
        rows.add((int(rng.integers(0, w.total_q)), int(rng.integers(0, w.heads_q))))
    heads = sorted({0, w.heads_q - 1, w.heads_q // 2})
    for b in range(w.batch):
        qo, ql, _, _ = w.sample_bounds(b)
        cand = [0, 1, ql - 1, ql - 2, tile_q - 1, tile_q, ql // 2]
        for q in cand:
            if 0 <= q < ql:
                for h in heads:
                    rows.add((qo + q, h))
    return np.asarray(sorted(rows), dtype=np.int64)


def sample_krows(w, items, n_random=100, seed=0, tile_k=64):
    """(K token, KV head) pairs inside the given (sample, KV head) items:
    random keys plus the sample's edges, both sides of K-tile boundaries,
    the first tile's keys (a sink) and the middle key."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b, g in items:
        _, _, ko, kl = w.sample_bounds(b)
        if kl == 0:
            continue
        for _ in range(n_random):
            rows.add((ko + int(rng.integers(0, kl)), g))
        cand = [0, 1, 2, 31, 32, 63, kl - 1, kl - 2, kl // 2]
        for j in range(1, kl // tile_k + 1, max(1, kl // tile_k // 6)):
            cand += [j * tile_k - 1, j * tile_k]
        for k in cand:
            if 0 <= k < kl:
                rows.add((ko + k, g))
    return np.asarray(sorted(rows), dtype=np.int64)


def compare_k2q(gk, ok):
    """Bit-exact comparison of a GPU K2Q export with the oracle's K2Q view."""
    assert list(gk["header"][3:7]) == [int(x) for x in ok.header], (gk["header"], ok.header)
    for key in ("cu_krows", "p_off", "f_off", "p_idx", "f_idx"):
        a, b = np.asarray(gk[key]), np.asarray(getattr(ok, key))
        assert a.shape == b.shape and np.array_equal(a, b), key
    assert gk["p_masks"].shape == ok.p_masks.shape
    assert np.array_equal(gk["p_masks"], ok.p_masks), "K2Q payload words differ"


def check_k2q_order(gk, mask_heads):
    """The K2Q launch order: a permutation of the K rows with non-increasing
    cost (partial + full Q tiles summed over mask heads), ties by K row."""
    krows = int(gk["header"][4])
    order = np.asarray(gk["order"], np.int64)
    assert order.shape == (krows,) and np.array_equal(np.sort(order), np.arange(krows))
    po, fo = np.asarray(gk["p_off"], np.int64), np.asarray(gk["f_off"], np.int64)
    cost = np.zeros(krows, np.int64)
    for hm in range(mask_heads):
        sl = slice(hm * krows, (hm + 1) * krows + 1)
        cost += np.diff(po[sl]) + np.diff(fo[sl])
    c = cost[order]
    assert np.all(c[:-1] >= c[1:]), "order not by descending cost"
    ties = c[:-1] == c[1:]
    assert np.all(order[:-1][ties] < order[1:][ties]), "ties not by K row"

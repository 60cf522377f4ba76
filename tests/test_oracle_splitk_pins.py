"""Pins of the oracle's Split-K partial state and merge (CPU only).

The Tessera page's "Split-K" section (Figure 5) partitions one query tile's
K/V reduction: each part keeps its max, its sum of exponentials and its
partial output, and a merge rescales the parts to a common maximum, sums and
normalizes.  The oracle holds the partial state as (O normalized over the
part's keys, LSE of the part) and merges with
LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.

What pins it (none of these re-types the merge):
  * merging the parts of ANY partition of the K axis must reproduce the
    unsplit attention (itself pinned in test_oracle_pins.py) -- a dropped
    part, a wrong sign or a missing rescale breaks this;
  * a part's range restriction equals a dense masked softmax written here in
    numpy with the range folded into the mask;
  * closed forms of the merge: equal LSEs average the outputs and add ln(P);
    empty parts (LSE = -inf) change nothing; all-empty rows give O = 0,
    LSE = -inf; the merge is invariant under permuting the parts.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def _partition(rng, k_max, nparts):
    cuts = np.sort(rng.integers(0, k_max + 1, size=nparts - 1))
    edges = np.concatenate([[0], cuts, [k_max + 7]])
    return [(int(edges[i]), int(edges[i + 1])) for i in range(nparts)]


@pytest.mark.parametrize("name", ["tiny_causal", "window_sink", "varlen_doc", "block_sparse",
                                  "prefix_softcap"])
@pytest.mark.parametrize("nparts", [2, 5])
def test_merge_of_any_partition_is_the_attention(name, nparts):
    w = W.make(name, small=True)
    o_ref, l_ref = oracle.attention(w)
    rng = np.random.default_rng(nparts)
    parts = _partition(rng, w.seqlen_k, nparts)
    outs = [oracle.attention_part(w, a, b) for (a, b) in parts]
    n = w.total_q * w.heads_q
    o_parts = np.stack([o.reshape(n, w.head_dim) for o, _ in outs])
    # partial LSE is [Hq, total_q]; the merge rows follow O's (token, head) order
    l_parts = np.stack([l.T.reshape(n) for _, l in outs])
    o, l = oracle.merge(o_parts, l_parts)
    o = o.reshape(w.total_q, w.heads_q, w.head_dim)
    l = l.reshape(w.total_q, w.heads_q).T
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), fin)
    assert np.max(np.abs(l[fin] - l_ref[fin]), initial=0.0) < 1e-12
    assert np.max(np.abs(o - o_ref)) < 1e-12
    assert np.all(o[~fin.T] == 0.0)


def test_full_range_part_is_the_attention_and_empty_range_is_empty():
    w = W.make("window_sink", small=True)
    o_ref, l_ref = oracle.attention(w)
    o, l = oracle.attention_part(w, 0, 1 << 40)
    assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref)
    o, l = oracle.attention_part(w, 300, 300)
    assert np.all(o == 0.0) and np.all(l == -np.inf)


def test_range_restriction_matches_dense_masked_softmax():
    """Causal B=1 fixed-length case: keys in [k_lo, k_hi) AND k <= q, written as
    a dense numpy softmax (no interval code)."""
    w = W.make("tiny_causal", small=True)
    k_lo, k_hi = 40, 170
    o, l = oracle.attention_part(w, k_lo, k_hi)
    S = w.seqlen_q
    kk = np.arange(S)[None, :]
    qq = np.arange(S)[:, None]
    keep = (kk <= qq) & (kk >= k_lo) & (kk < k_hi)
    for h in range(w.heads_q):
        q = w.q[:, h, :].astype(np.float64)
        k = w.k[:, h, :].astype(np.float64)
        v = w.v[:, h, :].astype(np.float64)
        s = w.scale * (q @ k.T)
        s = np.where(keep, s, -np.inf)
        for r in range(S):
            if not keep[r].any():
                assert l[h, r] == -np.inf and np.all(o[r, h] == 0.0)
                continue
            m = s[r].max()
            e = np.exp(s[r] - m)
            assert abs(l[h, r] - (m + math.log(e.sum()))) < 1e-12
            assert np.max(np.abs(o[r, h] - (e @ v) / e.sum())) < 1e-12


def test_merge_closed_forms():
    rng = np.random.default_rng(3)
    P, n, d = 4, 6, 8
    o_parts = rng.standard_normal((P, n, d))
    # equal LSEs: the mean of the outputs, LSE + ln P
    lse = np.full((P, n), 1.25)
    o, l = oracle.merge(o_parts, lse)
    assert np.allclose(l, 1.25 + math.log(P), atol=1e-14, rtol=0)
    assert np.allclose(o, o_parts.mean(axis=0), atol=1e-14, rtol=0)
    # one part: identity
    o1, l1 = oracle.merge(o_parts[:1], lse[:1] + rng.standard_normal((1, n)))
    assert np.allclose(o1, o_parts[0], atol=0, rtol=0)
    # empty parts are ignored even if their O holds garbage
    lse2 = rng.standard_normal((P, n))
    lse2[1] = -np.inf
    junk = o_parts.copy()
    junk[1] = np.nan
    o2, l2 = oracle.merge(junk, lse2)
    keep = [0, 2, 3]
    o3, l3 = oracle.merge(o_parts[keep], lse2[keep])
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)
    # weights: part s gets exp(L_s) / sum exp(L)
    wts = np.exp(lse2[keep]) / np.exp(lse2[keep]).sum(axis=0)
    assert np.allclose(o3, np.einsum("pn,pnd->nd", wts, o_parts[keep]), atol=1e-13, rtol=0)
    # all parts empty: O = 0, LSE = -inf
    o4, l4 = oracle.merge(o_parts, np.full((P, n), -np.inf))
    assert np.all(o4 == 0.0) and np.all(l4 == -np.inf)
    # permutation invariance
    perm = [2, 0, 3, 1]
    o5, l5 = oracle.merge(o_parts[perm], lse2[perm])
    o6, l6 = oracle.merge(o_parts, lse2)
    assert np.allclose(o5, o6, atol=1e-14, rtol=0) and np.allclose(l5, l6, atol=1e-14, rtol=0)

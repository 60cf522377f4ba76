"""Seeded synthetic inputs for interval-mask flex attention.

This module only *draws inputs*: Q/K/V values, interval endpoints and
sequence splits.  It holds none of the method's arithmetic (no expansion of
endpoints, no tile classification, no attention).  Both the CPU oracle and
the GPU path are fed the same bytes from here.

Workloads (shapes and mask structure follow the five benchmark cases of this
project; the mask semantics follow "Flex Attention Mask Plan Design", §2
"Public Mask Representation": row q sees [0,F0) U [F1,F2) U ... with
sample-local K positions):

  tiny_causal      B=1, H=2, S=256, d=64, fp32, F0=q+1
  window_sink      B=2, H=16, S=2048, d=128, bf16, nfunc=3:
                   F0=min(64,q+1), F1=max(F0,q-255), F2=q+1
  varlen_doc       THD, 16384 tokens in 8 samples (each >=256), H=16, d=128,
                   bf16, F0=local_q+1
  block_sparse     B=1, H=24, S=8190, d=128, bf16, logical blocks 90x78,
                   each (head, q-block, kv-block) active w.p. 0.2, diagonal
                   kv-block == q-block always active; per row the union of
                   active kv-block runs becomes endpoints (F0=0), padded with
                   repeats of the last endpoint to nfunc = 2*maxRuns+1
  prefix_softcap   B=4, H=32, S=4096, d=128, bf16, F0=max(1024,q+1),
                   score = 30*tanh(s*scale/30) + slope_h*(k-q),
                   slope_h = 2^(-8(h+1)/H)

A sixth shape, for the Split-K forward (few tasks, long K lists):

  chunk_long_kv    B=1, Hq=32, Hk=8 (grouped K/V heads), Sq=512, Sk=32768,
                   d=128, bf16: the last 512 tokens of a 32768-token causal
                   sequence attend to the whole prefix, F0 = Sk - Sq + q + 1

Random draws use numpy's PCG64 generator seeded with ``seed``, in the order
structure, then Q, K, V.  bf16 cases draw fp32 N(0,1) values and round them to
bf16 (round to nearest, ties to even); the rounded values are kept as exact
float32 numbers so the oracle sees exactly what the GPU sees.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

LAYOUT_BSHD = 0
LAYOUT_THD = 1
DTYPE_BF16 = 0
DTYPE_FP32 = 1


@dataclasses.dataclass
class Workload:
    name: str
    layout: int
    dtype: int
    batch: int
    seqlen_q: int          # BSHD: Sq ; THD: max_seqlen_q
    seqlen_k: int          # BSHD: Sk ; THD: max_seqlen_k
    total_q: int
    total_k: int
    heads_q: int
    heads_k: int
    head_dim: int
    mask_heads: int
    nfunc: int
    mask_func: np.ndarray              # int32 [mask_heads, nfunc, total_q]
    cu_seqlens_q: Optional[np.ndarray]  # int32 [batch+1] (THD) or None
    cu_seqlens_k: Optional[np.ndarray]
    q: Optional[np.ndarray]            # float32 [total_q, heads_q, d] (bf16-exact for bf16)
    k: Optional[np.ndarray]            # float32 [total_k, heads_k, d]
    v: Optional[np.ndarray]
    scale: float
    softcap: float = 0.0               # 0 = off
    alibi_slopes: Optional[np.ndarray] = None  # float32 [heads_q] or None
    alibi_before_softcap: bool = False
    seed: int = 0
    extra: dict = dataclasses.field(default_factory=dict)

    def sample_bounds(self, b: int):
        """(q_offset, q_len, k_offset, k_len) of sample b (input bookkeeping)."""
        if self.layout == LAYOUT_BSHD:
            return b * self.seqlen_q, self.seqlen_q, b * self.seqlen_k, self.seqlen_k
        cq, ck = self.cu_seqlens_q, self.cu_seqlens_k
        return int(cq[b]), int(cq[b + 1] - cq[b]), int(ck[b]), int(ck[b + 1] - ck[b])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32.  Inputs here are finite normal draws."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _draw_qkv(rng, total_q, total_k, hq, hk, d, dtype, with_values=True):
    if not with_values:
        return None, None, None
    q = rng.standard_normal((total_q, hq, d), dtype=np.float32)
    k = rng.standard_normal((total_k, hk, d), dtype=np.float32)
    v = rng.standard_normal((total_k, hk, d), dtype=np.float32)
    if dtype == DTYPE_BF16:
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def grad_output(w: "Workload") -> np.ndarray:
    """Seeded incoming gradient dO [total_q, Hq, d] for a backward pass: N(0,1)
    from its own generator (seeded with (seed, 1), so the forward inputs are
    unchanged), bf16-rounded for bf16 workloads."""
    rng = np.random.default_rng([w.seed, 1])
    do = rng.standard_normal((w.total_q, w.heads_q, w.head_dim), dtype=np.float32)
    return round_to_bf16(do) if w.dtype == DTYPE_BF16 else do


def alibi_slopes(heads: int) -> np.ndarray:
    """slope_h = 2^(-8(h+1)/H) as float32."""
    h = np.arange(heads, dtype=np.float64)
    return np.exp2(-8.0 * (h + 1.0) / heads).astype(np.float32)


# ---------------------------------------------------------------- endpoints

def causal_endpoints(q_local: np.ndarray) -> np.ndarray:
    """nfunc=1 endpoints for a causal row: F0 = q+1."""
    return (q_local + 1)[None, :].astype(np.int32)


def window_sink_endpoints(q_local: np.ndarray, sink: int, window: int) -> np.ndarray:
    """nfunc=3: F0=min(sink,q+1), F1=max(F0,q-window+1), F2=q+1."""
    f0 = np.minimum(sink, q_local + 1)
    f1 = np.maximum(f0, q_local - (window - 1))
    f2 = q_local + 1
    return np.stack([f0, f1, f2]).astype(np.int32)


def prefix_lm_endpoints(q_local: np.ndarray, prefix: int, k_len: int) -> np.ndarray:
    """nfunc=1: F0 = max(prefix, q+1), limited to the sample's K length."""
    return np.minimum(np.maximum(prefix, q_local + 1), k_len)[None, :].astype(np.int32)


def block_sparse_endpoints(active: np.ndarray, block_q: int, block_k: int,
                           seqlen_q: int, seqlen_k: int):
    """Turn a logical block mask active[H, nqb, nkb] into endpoints.

    Per (head, q-block) the active kv-blocks are merged into maximal runs of
    consecutive blocks; run [j0, j1] becomes the interval
    [j0*block_k, min((j1+1)*block_k, seqlen_k)).  F0 = 0 (the leading
    interval is empty); rows are padded with repeats of their last endpoint to
    nfunc = 2*maxRuns + 1.  Returns (mask_func [H, nfunc, seqlen_q], nfunc).
    """
    H, nqb, nkb = active.shape
    runs = []   # runs[h][i] = list of (start, end) token intervals
    max_runs = 0
    for h in range(H):
        per_h = []
        for i in range(nqb):
            cols = np.flatnonzero(active[h, i])
            row_runs = []
            if cols.size:
                brk = np.flatnonzero(np.diff(cols) != 1)
                starts = np.concatenate([[cols[0]], cols[brk + 1]])
                ends = np.concatenate([cols[brk], [cols[-1]]])
                for s, e in zip(starts, ends):
                    row_runs.append((int(s) * block_k, min((int(e) + 1) * block_k, seqlen_k)))
            max_runs = max(max_runs, len(row_runs))
            per_h.append(row_runs)
        runs.append(per_h)
    nfunc = 2 * max_runs + 1
    mf = np.zeros((H, nfunc, seqlen_q), dtype=np.int32)
    for h in range(H):
        for i in range(nqb):
            r0, r1 = i * block_q, min((i + 1) * block_q, seqlen_q)
            ep = [0]
            for (a, b) in runs[h][i]:
                ep += [a, b]
            ep += [ep[-1]] * (nfunc - len(ep))
            mf[h, :, r0:r1] = np.asarray(ep, dtype=np.int32)[:, None]
    return mf, nfunc


def _tile_bsh(mf_one: np.ndarray, batch: int) -> np.ndarray:
    """Repeat a per-sample [nfunc, Sq] endpoint row set over B samples
    (batch-major flattening of Q rows)."""
    return np.tile(mf_one, (1, batch))


# ---------------------------------------------------------------- workloads

def tiny_causal(seed=0, batch=1, heads=2, seqlen=256, head_dim=64,
                dtype=DTYPE_FP32, with_values=True) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    ql = np.arange(seqlen, dtype=np.int64)
    mf = _tile_bsh(causal_endpoints(ql), batch)[None]
    total = batch * seqlen
    q, k, v = _draw_qkv(rng, total, total, heads, heads, head_dim, dtype, with_values)
    return Workload("tiny_causal", LAYOUT_BSHD, dtype, batch, seqlen, seqlen, total, total,
                    heads, heads, head_dim, 1, 1, np.ascontiguousarray(mf), None, None,
                    q, k, v, 1.0 / math.sqrt(head_dim), seed=seed)


def window_sink(seed=0, batch=2, heads=16, seqlen=2048, head_dim=128, sink=64, window=256,
                dtype=DTYPE_BF16, with_values=True, heads_k=None) -> Workload:
    heads_k = heads if heads_k is None else heads_k
    rng = np.random.Generator(np.random.PCG64(seed))
    ql = np.arange(seqlen, dtype=np.int64)
    mf = _tile_bsh(window_sink_endpoints(ql, sink, window), batch)[None]
    total = batch * seqlen
    q, k, v = _draw_qkv(rng, total, total, heads, heads_k, head_dim, dtype, with_values)
    return Workload("window_sink", LAYOUT_BSHD, dtype, batch, seqlen, seqlen, total, total,
                    heads, heads_k, head_dim, 1, 3, np.ascontiguousarray(mf), None, None,
                    q, k, v, 1.0 / math.sqrt(head_dim), seed=seed,
                    extra={"sink": sink, "window": window})


def varlen_lengths(rng, total: int, nseq: int, min_len: int) -> np.ndarray:
    """len_i = min_len + Multinomial(total - nseq*min_len, uniform over nseq)."""
    extra = rng.multinomial(total - nseq * min_len, [1.0 / nseq] * nseq)
    return (min_len + extra).astype(np.int64)


def varlen_doc(seed=0, total=16384, nseq=8, min_len=256, heads=16, head_dim=128,
               dtype=DTYPE_BF16, with_values=True, lengths=None, heads_k=None) -> Workload:
    heads_k = heads if heads_k is None else heads_k
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.asarray(lengths, dtype=np.int64) if lengths is not None else \
        varlen_lengths(rng, total, nseq, min_len)
    nseq = len(lens)
    total = int(lens.sum())
    cu = np.zeros(nseq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    mf = np.zeros((1, 1, total), dtype=np.int32)
    for b in range(nseq):
        ql = np.arange(int(lens[b]), dtype=np.int64)
        mf[0, :, cu[b]:cu[b + 1]] = causal_endpoints(ql)
    maxlen = int(lens.max()) if nseq else 0
    q, k, v = _draw_qkv(rng, total, total, heads, heads_k, head_dim, dtype, with_values)
    return Workload("varlen_doc", LAYOUT_THD, dtype, nseq, maxlen, maxlen, total, total,
                    heads, heads_k, head_dim, 1, 1, mf, cu, cu.copy(), q, k, v,
                    1.0 / math.sqrt(head_dim), seed=seed, extra={"lengths": lens.tolist()})


def block_sparse(seed=0, batch=1, heads=24, seqlen=8190, head_dim=128, block_q=90, block_k=78,
                 density=0.2, dtype=DTYPE_BF16, with_values=True) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    nqb = -(-seqlen // block_q)
    nkb = -(-seqlen // block_k)
    active = rng.random((heads, nqb, nkb)) < density
    for i in range(min(nqb, nkb)):
        active[:, i, i] = True
    mf_one, nfunc = block_sparse_endpoints(active, block_q, block_k, seqlen, seqlen)
    mf = np.ascontiguousarray(np.tile(mf_one, (1, 1, batch)))
    total = batch * seqlen
    q, k, v = _draw_qkv(rng, total, total, heads, heads, head_dim, dtype, with_values)
    return Workload("block_sparse", LAYOUT_BSHD, dtype, batch, seqlen, seqlen, total, total,
                    heads, heads, head_dim, heads, nfunc, mf, None, None, q, k, v,
                    1.0 / math.sqrt(head_dim), seed=seed,
                    extra={"block_q": block_q, "block_k": block_k, "density": density,
                           "active_fraction": float(active.mean())})


def prefix_softcap(seed=0, batch=4, heads=32, seqlen=4096, head_dim=128, prefix=1024,
                   softcap=30.0, dtype=DTYPE_BF16, with_values=True, heads_k=None) -> Workload:
    heads_k = heads if heads_k is None else heads_k
    rng = np.random.Generator(np.random.PCG64(seed))
    ql = np.arange(seqlen, dtype=np.int64)
    mf = _tile_bsh(prefix_lm_endpoints(ql, prefix, seqlen), batch)[None]
    total = batch * seqlen
    q, k, v = _draw_qkv(rng, total, total, heads, heads_k, head_dim, dtype, with_values)
    return Workload("prefix_softcap", LAYOUT_BSHD, dtype, batch, seqlen, seqlen, total, total,
                    heads, heads_k, head_dim, 1, 1, np.ascontiguousarray(mf), None, None,
                    q, k, v, 1.0 / math.sqrt(head_dim), softcap=softcap,
                    alibi_slopes=alibi_slopes(heads), seed=seed, extra={"prefix": prefix})


def chunk_long_kv(seed=0, batch=1, heads_q=32, heads_k=8, seqlen_q=512, seqlen_k=32768,
                  head_dim=128, dtype=DTYPE_BF16, with_values=True) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    ql = np.arange(seqlen_q, dtype=np.int64)
    mf = _tile_bsh(causal_endpoints(ql + (seqlen_k - seqlen_q)), batch)[None]
    total_q, total_k = batch * seqlen_q, batch * seqlen_k
    q, k, v = _draw_qkv(rng, total_q, total_k, heads_q, heads_k, head_dim, dtype, with_values)
    return Workload("chunk_long_kv", LAYOUT_BSHD, dtype, batch, seqlen_q, seqlen_k, total_q,
                    total_k, heads_q, heads_k, head_dim, 1, 1, np.ascontiguousarray(mf), None,
                    None, q, k, v, 1.0 / math.sqrt(head_dim), seed=seed)


FULL_CONFIGS = {
    "tiny_causal": tiny_causal,
    "window_sink": window_sink,
    "varlen_doc": varlen_doc,
    "block_sparse": block_sparse,
    "prefix_softcap": prefix_softcap,
}

# Reduced shapes of the same structure that the oracle finishes in seconds while
# still spanning several tiles and ragged tails.
SMALL_CONFIGS = {
    "tiny_causal": lambda seed=0, **kw: tiny_causal(seed=seed, **kw),
    "window_sink": lambda seed=0, **kw: window_sink(seed=seed, batch=2, heads=2, seqlen=700,
                                                    sink=64, window=256, **kw),
    "varlen_doc": lambda seed=0, **kw: varlen_doc(seed=seed, total=1500, nseq=5, min_len=100,
                                                  heads=2, **kw),
    "block_sparse": lambda seed=0, **kw: block_sparse(seed=seed, heads=3, seqlen=700, **kw),
    "prefix_softcap": lambda seed=0, **kw: prefix_softcap(seed=seed, batch=2, heads=4,
                                                          seqlen=600, prefix=150, **kw),
}


# Shapes outside the five benchmark cases (Split-K: few tasks, long K lists).
EXTRA_FULL = {"chunk_long_kv": chunk_long_kv}
EXTRA_SMALL = {
    "chunk_long_kv": lambda seed=0, **kw: chunk_long_kv(seed=seed, batch=2, heads_q=4, heads_k=2,
                                                        seqlen_q=200, seqlen_k=3000, **kw),
}


def make(name: str, seed: int = 0, small: bool = False, **kw) -> Workload:
    table = dict(SMALL_CONFIGS, **EXTRA_SMALL) if small else dict(FULL_CONFIGS, **EXTRA_FULL)
    return table[name](seed=seed, **kw)


def custom(mask_func, layout=LAYOUT_BSHD, batch=1, seqlen_q=None, seqlen_k=None,
           cu_seqlens_q=None, cu_seqlens_k=None, heads_q=1, heads_k=None, head_dim=64,
           dtype=DTYPE_FP32, seed=0, softcap=0.0, alibi=None, alibi_before_softcap=False,
           scale=None, with_values=True, name="custom") -> Workload:
    """Build a workload from explicit endpoints (tests and edge cases)."""
    mf = np.ascontiguousarray(np.asarray(mask_func, dtype=np.int32))
    if mf.ndim == 2:
        mf = mf[None]
    heads_k = heads_q if heads_k is None else heads_k
    if layout == LAYOUT_BSHD:
        total_q = batch * seqlen_q
        total_k = batch * seqlen_k
        cq = ck = None
    else:
        cq = np.asarray(cu_seqlens_q, dtype=np.int32)
        ck = np.asarray(cu_seqlens_k, dtype=np.int32)
        batch = len(cq) - 1
        total_q, total_k = int(cq[-1]), int(ck[-1])
        if seqlen_q is None:
            seqlen_q = int(np.max(np.diff(cq))) if batch else 0
        if seqlen_k is None:
            seqlen_k = int(np.max(np.diff(ck))) if batch else 0
    rng = np.random.Generator(np.random.PCG64(seed))
    q, k, v = _draw_qkv(rng, total_q, total_k, heads_q, heads_k, head_dim, dtype, with_values)
    slopes = alibi_slopes(heads_q) if alibi is True else alibi
    return Workload(name, layout, dtype, batch, seqlen_q, seqlen_k, total_q, total_k, heads_q,
                    heads_k, head_dim, mf.shape[0], mf.shape[1], mf, cq, ck, q, k, v,
                    scale if scale is not None else 1.0 / math.sqrt(head_dim), softcap=softcap,
                    alibi_slopes=slopes, alibi_before_softcap=alibi_before_softcap, seed=seed)


def to_device(w: Workload, device="cuda") -> dict:
    """Copy a workload's input arrays into torch device tensors (exact: bf16
    values are bf16-representable).  BSHD tensors are [B, S, H, d], THD
    [T, H, d]."""
    import torch

    dt = torch.bfloat16 if w.dtype == DTYPE_BF16 else torch.float32

    def qkv(x, total):
        t = torch.from_numpy(x).to(dt)
        if w.layout == LAYOUT_BSHD:
            t = t.reshape(w.batch, total // w.batch, x.shape[1], x.shape[2])
        return t.contiguous().to(device)

    d = {
        "mask_func": torch.from_numpy(np.ascontiguousarray(w.mask_func)).to(device),
        "cu_q": None if w.cu_seqlens_q is None else torch.from_numpy(w.cu_seqlens_q).to(device),
        "cu_k": None if w.cu_seqlens_k is None else torch.from_numpy(w.cu_seqlens_k).to(device),
        "slopes": None if w.alibi_slopes is None else torch.from_numpy(w.alibi_slopes).to(device),
    }
    if w.q is not None:
        d["q"] = qkv(w.q, w.total_q)
        d["k"] = qkv(w.k, w.total_k)
        d["v"] = qkv(w.v, w.total_k)
    return d

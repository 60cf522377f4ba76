"""CPU oracle for interval-mask flex attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library
(``mask_planned_block_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain loops, double precision); this
module only marshals numpy arrays through ctypes.  See ``oracle.c`` for the
passage each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# MPB_ORACLE_LIB selects another build of the same source (the sanitizer
# test loads an AddressSanitizer/UBSan build through it)
_LIB_PATH = os.environ.get("MPB_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

ERR_SEQLENS = 1
ERR_RANGE = 2
ERR_ORDER = 4

CLASS_EMPTY = 0
CLASS_PARTIAL = 1
CLASS_FULL = 2


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layout", "batch", "seqlen_q", "seqlen_k", "total_q", "total_k", "heads_q", "heads_k",
        "head_dim", "mask_heads", "nfunc", "tile_q", "tile_k")]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER(_Problem)
        vp = ctypes.c_void_p
        lib.orc_validate.argtypes = [P, vp, vp, vp]
        lib.orc_validate.restype = ctypes.c_uint32
        lib.orc_expand_row.argtypes = [vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int64, vp]
        lib.orc_expand_row.restype = None
        lib.orc_plan_build.argtypes = [P, vp, vp, vp, ctypes.c_int]
        lib.orc_plan_build.restype = vp
        lib.orc_plan_sizes.argtypes = [vp, vp, vp, vp]
        lib.orc_plan_export.argtypes = [vp, P, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.orc_plan_free.argtypes = [vp]
        lib.orc_k2q_build.argtypes = [P, vp, vp, vp, ctypes.c_int]
        lib.orc_k2q_build.restype = vp
        lib.orc_k2q_sizes.argtypes = [vp, vp]
        lib.orc_k2q_export.argtypes = [vp, P, vp, vp, vp, vp, vp, vp]
        lib.orc_k2q_free.argtypes = [vp]
        lib.orc_attention.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_double, ctypes.c_int,
                                      ctypes.c_double, ctypes.c_int, vp, ctypes.c_int,
                                      ctypes.c_int64, vp, vp, vp, ctypes.c_int]
        lib.orc_attention.restype = None
        lib.orc_attention_part.argtypes = [P, vp, vp, vp, vp, vp, vp, ctypes.c_double,
                                           ctypes.c_int, ctypes.c_double, ctypes.c_int, vp,
                                           ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int64, vp, vp, vp, ctypes.c_int]
        lib.orc_attention_part.restype = None
        lib.orc_merge.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, vp, vp, vp, vp]
        lib.orc_merge.restype = None
        lib.orc_attention_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_double,
                                          ctypes.c_int, ctypes.c_double, ctypes.c_int, vp,
                                          ctypes.c_int, vp, vp, vp, ctypes.c_int]
        lib.orc_attention_bwd.restype = None
        lib.orc_attention_bwd_dq_rows.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, ctypes.c_double,
                                                  ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                                  vp, ctypes.c_int, ctypes.c_int64, vp, vp,
                                                  ctypes.c_int]
        lib.orc_attention_bwd_dq_rows.restype = None
        lib.orc_attention_bwd_dkdv_rows.argtypes = [P, vp, vp, vp, vp, vp, vp, vp,
                                                    ctypes.c_double, ctypes.c_int,
                                                    ctypes.c_double, ctypes.c_int, vp,
                                                    ctypes.c_int, ctypes.c_int64, vp, vp, vp,
                                                    ctypes.c_int]
        lib.orc_attention_bwd_dkdv_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _problem(w, tile_q=64, tile_k=64) -> _Problem:
    return _Problem(w.layout, w.batch, w.seqlen_q, w.seqlen_k, w.total_q, w.total_k, w.heads_q,
                    w.heads_k, w.head_dim, w.mask_heads, w.nfunc, tile_q, tile_k)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def validate(w) -> int:
    """OR of ERR_* bits for the workload's endpoints and prefixes."""
    p = _problem(w)
    mf, cq, ck = _i32(w.mask_func), _i32(w.cu_seqlens_q), _i32(w.cu_seqlens_k)
    return int(_load().orc_validate(ctypes.byref(p), _ptr(mf), _ptr(cq), _ptr(ck)))


def expand_row(endpoints, k_len: int) -> np.ndarray:
    """Dense boolean visibility of one row with the given endpoints."""
    F = np.ascontiguousarray(np.asarray(endpoints, dtype=np.int32))
    out = np.zeros(max(k_len, 1), dtype=np.uint8)
    _load().orc_expand_row(_ptr(F), 1, len(F), k_len, _ptr(out))
    return out[:k_len].astype(bool)


class Plan:
    """Host copy of the oracle's plan (all arrays numpy)."""

    def __init__(self, header, rows_total, nk_max, tile_q, tile_k, cu_rows=None, seqdesc=None,
                 p_off=None, p_idx=None, p_masks=None, f_off=None, f_idx=None, cls=None):
        self.header = header
        self.rows_total = rows_total
        self.nk_max = nk_max
        self.tile_q, self.tile_k = tile_q, tile_k
        self.cu_rows, self.seqdesc = cu_rows, seqdesc
        self.p_off, self.p_idx, self.p_masks = p_off, p_idx, p_masks
        self.f_off, self.f_idx, self.cls = f_off, f_idx, cls

    @property
    def err(self) -> int:
        return int(self.header[7])


def build_plan(w, tile_q: int, tile_k: int, nthreads: Optional[int] = None) -> Plan:
    """Brute-force plan: validation, expansion, classification, packing, CSR."""
    lib = _load()
    p = _problem(w, tile_q, tile_k)
    mf, cq, ck = _i32(w.mask_func), _i32(w.cu_seqlens_q), _i32(w.cu_seqlens_k)
    h = lib.orc_plan_build(ctypes.byref(p), _ptr(mf), _ptr(cq), _ptr(ck),
                           nthreads or default_threads())
    if not h:
        raise MemoryError("oracle plan allocation failed")
    try:
        header = np.zeros(8, dtype=np.int64)
        rows = ctypes.c_int32()
        nk = ctypes.c_int32()
        lib.orc_plan_sizes(h, _ptr(header), ctypes.byref(rows), ctypes.byref(nk))
        if header[7]:
            return Plan(header, 0, 0, tile_q, tile_k)
        R, nkm = rows.value, nk.value
        items = w.mask_heads * R
        words = tile_k // 32
        cu_rows = np.zeros(w.batch + 1, np.int32)
        seqdesc = np.zeros((w.batch, 8), np.int32)
        p_off = np.zeros(items + 1, np.int32)
        f_off = np.zeros(items + 1, np.int32)
        p_idx = np.zeros(max(int(header[1]), 1), np.int32)
        f_idx = np.zeros(max(int(header[2]), 1), np.int32)
        p_masks = np.zeros(max(int(header[1]) * tile_q * words, 1), np.uint32)
        cls = np.zeros(max(items * nkm, 1), np.uint8)
        lib.orc_plan_export(h, ctypes.byref(p), _ptr(cu_rows), _ptr(seqdesc), _ptr(p_off),
                            _ptr(p_idx), _ptr(p_masks), _ptr(f_off), _ptr(f_idx), _ptr(cls))
        pn, fn = int(header[1]), int(header[2])
        return Plan(header, R, nkm, tile_q, tile_k, cu_rows, seqdesc, p_off, p_idx[:pn],
                    p_masks[:pn * tile_q * words].reshape(pn, tile_q, words), f_off, f_idx[:fn],
                    cls[:items * nkm].reshape(w.mask_heads, R, nkm))
    finally:
        lib.orc_plan_free(h)


class K2Q:
    """Host copy of the oracle's backward K2Q view (all arrays numpy).

    header = (Q rows, K rows, partial nnz, full nnz); K rows flattened
    head-major; p_masks [pnnz][tile_k][tile_q/32] (K-major predicate)."""

    def __init__(self, header, tile_q, tile_k, cu_krows, p_off, p_idx, p_masks, f_off, f_idx):
        self.header = header
        self.tile_q, self.tile_k = tile_q, tile_k
        self.cu_krows = cu_krows
        self.p_off, self.p_idx, self.p_masks = p_off, p_idx, p_masks
        self.f_off, self.f_idx = f_off, f_idx


def build_k2q(w, tile_q: int, tile_k: int, nthreads: Optional[int] = None) -> Optional[K2Q]:
    """Brute-force K2Q view ("Flex Attention Mask Plan Design" §4.4, §4.7);
    None when the workload fails validation."""
    lib = _load()
    p = _problem(w, tile_q, tile_k)
    mf, cq, ck = _i32(w.mask_func), _i32(w.cu_seqlens_q), _i32(w.cu_seqlens_k)
    h = lib.orc_k2q_build(ctypes.byref(p), _ptr(mf), _ptr(cq), _ptr(ck),
                          nthreads or default_threads())
    if not h:
        return None
    try:
        header = np.zeros(4, dtype=np.int64)
        lib.orc_k2q_sizes(h, _ptr(header))
        kitems = w.mask_heads * int(header[1])
        pn, fn = int(header[2]), int(header[3])
        wq = tile_q // 32
        cu_krows = np.zeros(w.batch + 1, np.int32)
        p_off = np.zeros(kitems + 1, np.int32)
        f_off = np.zeros(kitems + 1, np.int32)
        p_idx = np.zeros(max(pn, 1), np.int32)
        f_idx = np.zeros(max(fn, 1), np.int32)
        p_masks = np.zeros(max(pn * tile_k * wq, 1), np.uint32)
        lib.orc_k2q_export(h, ctypes.byref(p), _ptr(cu_krows), _ptr(p_off), _ptr(p_idx),
                           _ptr(p_masks), _ptr(f_off), _ptr(f_idx))
        return K2Q(header, tile_q, tile_k, cu_krows, p_off, p_idx[:pn],
                   p_masks[:pn * tile_k * wq].reshape(pn, tile_k, wq), f_off, f_idx[:fn])
    finally:
        lib.orc_k2q_free(h)


def attention(w, rows: Optional[np.ndarray] = None, nthreads: Optional[int] = None):
    """fp64 masked softmax attention with the workload's score_mod.

    rows=None: every (token, head); returns O [total_q, Hq, d] and
    LSE [Hq, total_q].  rows = int array [n, 2] of (token, head): returns O [n, d]
    and LSE [n].
    """
    return _attention(w, None, rows, nthreads)


def attention_part(w, k_lo: int, k_hi: int, rows: Optional[np.ndarray] = None,
                   nthreads: Optional[int] = None):
    """Split-K partial state: the attention of attention() with every row's
    visible keys cut to the sample-local range [k_lo, k_hi) (O normalized over
    those keys, their LSE; O = 0, LSE = -inf where none is left).  Same
    return layouts as attention()."""
    return _attention(w, (int(k_lo), int(k_hi)), rows, nthreads)


def _attention(w, krange, rows, nthreads):
    lib = _load()
    p = _problem(w)
    mf, cq, ck = _i32(w.mask_func), _i32(w.cu_seqlens_q), _i32(w.cu_seqlens_k)
    q = np.ascontiguousarray(w.q, dtype=np.float32)
    k = np.ascontiguousarray(w.k, dtype=np.float32)
    v = np.ascontiguousarray(w.v, dtype=np.float32)
    slopes = None if w.alibi_slopes is None else np.ascontiguousarray(w.alibi_slopes, np.float32)
    if rows is None:
        o = np.zeros((w.total_q, w.heads_q, w.head_dim), np.float64)
        lse = np.zeros((w.heads_q, w.total_q), np.float64)
        n, rp = 0, None
    else:
        rp = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
        n = rp.shape[0]
        o = np.zeros((n, w.head_dim), np.float64)
        lse = np.zeros(n, np.float64)
    common = (ctypes.byref(p), _ptr(mf), _ptr(cq), _ptr(ck), _ptr(q), _ptr(k), _ptr(v),
              float(w.scale), int(w.softcap > 0), float(w.softcap), int(slopes is not None),
              _ptr(slopes), int(bool(w.alibi_before_softcap)))
    tail = (n, _ptr(rp), _ptr(o), _ptr(lse), nthreads or default_threads())
    if krange is None:
        lib.orc_attention(*common, *tail)
    else:
        lib.orc_attention_part(*common, krange[0], krange[1], *tail)
    return o, lse


def merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge of Split-K partial states (orc_merge): o_parts [P, n, d] (each
    normalized over its keys), lse_parts [P, n] -> (O [n, d], LSE [n])."""
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    P, n, d = o_parts.shape
    assert lse_parts.shape == (P, n)
    o = np.zeros((n, d), np.float64)
    lse = np.zeros(n, np.float64)
    _load().orc_merge(P, n, d, _ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse))
    return o, lse


def attention_bwd(w, dout: np.ndarray, nthreads: Optional[int] = None):
    """fp64 gradients (dQ, dK, dV) of the workload's attention output for the
    incoming gradient dout [total_q, Hq, d] (the chain rule of FlexAttention
    Eq. 1 with the score_mod's derivative; see orc_attention_bwd).  Returns
    dQ [total_q, Hq, d], dK and dV [total_k, Hk, d]."""
    lib = _load()
    p = _problem(w)
    mf, cq, ck = _i32(w.mask_func), _i32(w.cu_seqlens_q), _i32(w.cu_seqlens_k)
    q = np.ascontiguousarray(w.q, dtype=np.float32)
    k = np.ascontiguousarray(w.k, dtype=np.float32)
    v = np.ascontiguousarray(w.v, dtype=np.float32)
    do = np.ascontiguousarray(dout, dtype=np.float32)
    assert do.shape == q.shape
    slopes = None if w.alibi_slopes is None else np.ascontiguousarray(w.alibi_slopes, np.float32)
    dq = np.zeros((w.total_q, w.heads_q, w.head_dim), np.float64)
    dk = np.zeros((w.total_k, w.heads_k, w.head_dim), np.float64)
    dv = np.zeros((w.total_k, w.heads_k, w.head_dim), np.float64)
    lib.orc_attention_bwd(ctypes.byref(p), _ptr(mf), _ptr(cq), _ptr(ck), _ptr(q), _ptr(k),
                          _ptr(v), _ptr(do), float(w.scale), int(w.softcap > 0),
                          float(w.softcap), int(slopes is not None), _ptr(slopes),
                          int(bool(w.alibi_before_softcap)), _ptr(dq), _ptr(dk), _ptr(dv),
                          nthreads or default_threads())
    return dq, dk, dv


def attention_bwd_dq_rows(w, dout: np.ndarray, rows: np.ndarray,
                          nthreads: Optional[int] = None) -> np.ndarray:
    """dQ [n, d] of the selected (token, head) rows (same chain rule as
    attention_bwd, one row at a time)."""
    lib = _load()
    p = _problem(w)
    mf, cq, ck = _i32(w.mask_func), _i32(w.cu_seqlens_q), _i32(w.cu_seqlens_k)
    q = np.ascontiguousarray(w.q, dtype=np.float32)
    k = np.ascontiguousarray(w.k, dtype=np.float32)
    v = np.ascontiguousarray(w.v, dtype=np.float32)
    do = np.ascontiguousarray(dout, dtype=np.float32)
    rp = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    slopes = None if w.alibi_slopes is None else np.ascontiguousarray(w.alibi_slopes, np.float32)
    dq = np.zeros((rp.shape[0], w.head_dim), np.float64)
    lib.orc_attention_bwd_dq_rows(ctypes.byref(p), _ptr(mf), _ptr(cq), _ptr(ck), _ptr(q),
                                  _ptr(k), _ptr(v), _ptr(do), float(w.scale),
                                  int(w.softcap > 0), float(w.softcap), int(slopes is not None),
                                  _ptr(slopes), int(bool(w.alibi_before_softcap)),
                                  rp.shape[0], _ptr(rp), _ptr(dq), nthreads or default_threads())
    return dq


def attention_bwd_dkdv_rows(w, dout: np.ndarray, rows: np.ndarray,
                            nthreads: Optional[int] = None):
    """dK and dV [n, d] of the selected (K token, KV head) rows (same chain
    rule as attention_bwd; each Q row that sees the key is recomputed from
    that row alone).  The cost grows with the (sample, KV head) pairs the
    rows fall in, not with their number."""
    lib = _load()
    p = _problem(w)
    mf, cq, ck = _i32(w.mask_func), _i32(w.cu_seqlens_q), _i32(w.cu_seqlens_k)
    q = np.ascontiguousarray(w.q, dtype=np.float32)
    k = np.ascontiguousarray(w.k, dtype=np.float32)
    v = np.ascontiguousarray(w.v, dtype=np.float32)
    do = np.ascontiguousarray(dout, dtype=np.float32)
    rp = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    slopes = None if w.alibi_slopes is None else np.ascontiguousarray(w.alibi_slopes, np.float32)
    n = rp.shape[0]
    dk = np.zeros((max(n, 1), w.head_dim), np.float64)
    dv = np.zeros((max(n, 1), w.head_dim), np.float64)
    rc = lib.orc_attention_bwd_dkdv_rows(ctypes.byref(p), _ptr(mf), _ptr(cq), _ptr(ck), _ptr(q),
                                         _ptr(k), _ptr(v), _ptr(do), float(w.scale),
                                         int(w.softcap > 0), float(w.softcap),
                                         int(slopes is not None), _ptr(slopes),
                                         int(bool(w.alibi_before_softcap)), n, _ptr(rp),
                                         _ptr(dk), _ptr(dv), nthreads or default_threads())
    if rc != 0:
        raise ValueError("a selected K token lies outside every sample")
    return dk[:n], dv[:n]

"""Python binding of libmpb: interval-mask flex attention on MI355X (gfx950).

Argument marshalling only.  Every step of the path -- plan building and the
attention forward -- runs in the HIP kernels of ``libmpb.so`` behind the C ABI
of ``include/mpb.h``; torch tensors provide device memory and streams.  There
is no CPU fallback: importing this package fails if the library is missing.

    plan = mask_plan_build(problem, mask_func, cu_seqlens_q, cu_seqlens_k)
    o, lse = flex_attn_fwd(plan, q, k, v, scale=..., softcap=..., alibi_slopes=...)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

__all__ = [
    "LAYOUT_BSHD", "LAYOUT_THD", "DTYPE_BF16", "DTYPE_FP32", "MPBError", "Problem", "MaskPlan",
    "make_problem", "mask_plan_build", "mask_plan_destroy", "mask_plan_info", "mask_plan_export",
    "flex_attn_fwd", "flex_attn_fwd_workspace_size", "flex_attn_fwd_num_splits",
    "flex_attn_fwd_splitk_workspace_size", "flex_attn_fwd_merge", "flex_attn_fwd_paged",
    "flex_attn_fwd_splitk_noalloc",
    "flex_attn_fwd_paged_workspace_size", "flex_attn_bwd",
    "flex_attn_bwd_workspace_size", "library_path", "TASK_REC_FIELDS",
]

LAYOUT_BSHD = 0
LAYOUT_THD = 1
DTYPE_BF16 = 0
DTYPE_FP32 = 1
BUILD_EXACT, BUILD_IN_PLACE, BUILD_SINGLE_PASS, BUILD_SINGLE_PASS_DEFERRED = 0, 1, 2, 3   # PlanInfo.build_mode
NUM_QUEUES = 9
TASK_REC_INTS = 16
TASK_REC_FIELDS = ("m_block", "head", "batch", "q_valid_rows", "q_offset", "k_offset", "q_len",
                   "k_len", "partial_begin", "partial_count", "full_begin", "full_count",
                   "first_k_tile", "mask_head", "kv_head", "section")

STATUS = {0: "MPB_OK", 1: "MPB_ERR_INVALID_ARGUMENT", 2: "MPB_ERR_ENDPOINT_RANGE",
          3: "MPB_ERR_ENDPOINT_ORDER", 4: "MPB_ERR_SEQLENS", 5: "MPB_ERR_SIGNATURE_MISMATCH",
          6: "MPB_ERR_WORKSPACE", 7: "MPB_ERR_UNSUPPORTED", 8: "MPB_ERR_OUT_OF_MEMORY",
          9: "MPB_ERR_DEVICE"}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmpb.so")


class MPBError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, "MPB_ERR_%d" % status)
        super().__init__("%s: %s" % (self.name, detail))


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layout", "dtype", "batch", "seqlen_q", "seqlen_k", "total_q", "total_k", "heads_q",
        "heads_k", "head_dim", "mask_heads", "nfunc", "tile_q", "tile_k")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class Signature(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "arch", "direction", "kernel_family", "tile_q", "tile_k", "head_dim", "dtype",
        "payload_layout", "scheduler", "pack_gqa")]


class PlanInfo(ctypes.Structure):
    _fields_ = [("header", ctypes.c_int64 * 8), ("rows_total", ctypes.c_int32),
                ("nk_max", ctypes.c_int32), ("words_per_row", ctypes.c_int32),
                ("num_tasks", ctypes.c_int32), ("num_sections", ctypes.c_int32),
                ("device", ctypes.c_int32), ("problem", Problem), ("signature", Signature),
                ("device_bytes", ctypes.c_int64), ("build_mode", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class BuildOptions(ctypes.Structure):
    _fields_ = [("build_backward", ctypes.c_int32), ("time_stages", ctypes.c_int32),
                ("pack_gqa", ctypes.c_int32), ("defer_header", ctypes.c_int32)]


class ScoreMod(ctypes.Structure):
    _fields_ = [("softcap_enabled", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("alibi_enabled", ctypes.c_int32), ("alibi_slopes", ctypes.c_void_p),
                ("alibi_before_softcap", ctypes.c_int32)]


def _load():
    if not os.path.exists(library_path):
        raise ImportError("libmpb.so is not built (%s); run __graft_entry__.build() or "
                          "python mask_planned_block_amd/build.py" % library_path)
    lib = ctypes.CDLL(library_path)
    vp, P = ctypes.c_void_p, ctypes.POINTER
    lib.mask_plan_build.argtypes = [P(Problem), vp, vp, vp, vp, P(vp)]
    lib.mask_plan_build_ex.argtypes = [P(Problem), P(BuildOptions), vp, vp, vp, vp, P(vp)]
    lib.mask_plan_export_k2q.argtypes = [vp] + [vp] * 6
    lib.mask_plan_stage_times.argtypes = [vp, vp]
    lib.mask_plan_export_k2q_order.argtypes = [vp, vp]
    lib.mask_plan_destroy.argtypes = [vp]
    lib.mask_plan_info.argtypes = [vp, P(PlanInfo)]
    lib.mask_plan_export.argtypes = [vp] + [vp] * 9
    lib.mask_plan_export_launch_order.argtypes = [vp, vp]
    lib.flex_attn_fwd_workspace_size.argtypes = [vp]
    lib.flex_attn_fwd_workspace_size.restype = ctypes.c_size_t
    fwd_args = [vp, P(Problem), vp, vp, vp, vp, vp, ctypes.c_float, P(ScoreMod), vp,
                ctypes.c_size_t, vp]
    lib.flex_attn_fwd.argtypes = fwd_args
    lib.flex_attn_fwd_ablation.argtypes = fwd_args + [ctypes.c_int32]
    lib.flex_attn_fwd_num_splits.argtypes = [vp]
    lib.flex_attn_fwd_num_splits.restype = ctypes.c_int32
    lib.flex_attn_fwd_splitk_workspace_size.argtypes = [vp, ctypes.c_int32]
    lib.flex_attn_fwd_splitk_workspace_size.restype = ctypes.c_size_t
    lib.flex_attn_fwd_splitk.argtypes = fwd_args[:9] + [ctypes.c_int32] + fwd_args[9:]
    lib.flex_attn_fwd_splitk_noalloc.argtypes = fwd_args[:9] + [ctypes.c_int32, vp]
    lib.flex_attn_fwd_merge.argtypes = [ctypes.c_int32] * 5 + [vp] * 5
    lib.flex_attn_fwd_paged_workspace_size.argtypes = [vp, ctypes.c_int32]
    lib.flex_attn_fwd_paged_workspace_size.restype = ctypes.c_size_t
    lib.flex_attn_fwd_paged.argtypes = [vp, P(Problem), vp, vp, vp, vp] + [ctypes.c_int32] * 3 + \
        [vp, vp, ctypes.c_float, P(ScoreMod), ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_size_t,
         vp]
    lib.flex_attn_bwd_workspace_size.argtypes = [vp]
    lib.flex_attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.flex_attn_bwd.argtypes = [vp, P(Problem)] + [vp] * 9 + [ctypes.c_float, P(ScoreMod), vp,
                                                              ctypes.c_size_t, vp]
    lib.flex_attn_bwd_ablation.argtypes = lib.flex_attn_bwd.argtypes + [ctypes.c_int32]
    lib.mpb_status_string.restype = ctypes.c_char_p
    lib.mpb_status_string.argtypes = [ctypes.c_int]
    lib.mpb_last_error_detail.restype = ctypes.c_char_p
    lib.mpb_version.restype = ctypes.c_int32
    for name in ("mask_plan_build", "mask_plan_build_ex", "mask_plan_destroy", "mask_plan_info",
                 "mask_plan_export", "mask_plan_export_k2q", "mask_plan_stage_times", "mask_plan_export_k2q_order",
                 "mask_plan_export_launch_order",
                 "flex_attn_fwd", "flex_attn_fwd_ablation", "flex_attn_fwd_splitk",
                 "flex_attn_fwd_splitk_noalloc",
                 "flex_attn_fwd_merge", "flex_attn_fwd_paged", "flex_attn_bwd",
                 "flex_attn_bwd_ablation"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


_lib = _load()


def _check(status: int):
    if status != 0:
        raise MPBError(status, _lib.mpb_last_error_detail().decode())


def _stream_handle(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dev_ptr(t: Optional[torch.Tensor], what: str, dtype=None):
    if t is None:
        return None
    if not (t.is_cuda and t.is_contiguous()) or (dtype is not None and t.dtype != dtype):
        raise ValueError("%s must be a contiguous device tensor%s (got %s, %s, contiguous=%s)"
                         % (what, "" if dtype is None else " of " + str(dtype), t.device,
                            t.dtype, t.is_contiguous()))
    return t.data_ptr()


def _require_shape(t: Optional[torch.Tensor], what: str, shape):
    """Caller-supplied outputs and per-head arrays must have the size the
    kernels write or read: the library only sees bare pointers, so an
    undersized tensor would become an out-of-bounds device access."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (what, tuple(shape), tuple(t.shape)))


def _check_slopes(alibi_slopes: Optional[torch.Tensor], heads_q: int):
    if alibi_slopes is not None and alibi_slopes.numel() < heads_q:
        raise ValueError("alibi_slopes needs one value per Q head (%d), got %d"
                         % (heads_q, alibi_slopes.numel()))


ABLATE_FULL_AS_PARTIAL = 1
ABLATE_NO_SKIP = 2


def make_problem(layout, dtype, batch, seqlen_q, seqlen_k, total_q, total_k, heads_q, heads_k,
                 head_dim, mask_heads, nfunc, tile_q=0, tile_k=0) -> Problem:
    return Problem(layout, dtype, batch, seqlen_q, seqlen_k, total_q, total_k, heads_q, heads_k,
                   head_dim, mask_heads, nfunc, tile_q, tile_k)


class MaskPlan:
    """Owner of an opaque mpb_plan handle (immutable device plan)."""

    def __init__(self, handle: int, stream_handle: int, problem: Problem):
        self._h = ctypes.c_void_p(handle)
        self._stream = stream_handle
        self._bound = Problem.from_buffer_copy(problem)   # geometry the plan was built for
        self._info = None
        self._ws = None

    @property
    def handle(self):
        return self._h

    @property
    def info(self) -> "PlanInfo":
        if self._info is None:
            self._info = mask_plan_info(self)
        return self._info

    @property
    def problem(self) -> Problem:
        """The plan binding, with the physical tile resolved."""
        return self.info.problem

    @property
    def workspace_bytes(self) -> int:
        if self._ws is None:
            self._ws = int(_lib.flex_attn_fwd_workspace_size(self._h))
        return self._ws

    def header(self):
        return list(self.info.header)

    def export(self):
        return mask_plan_export(self)

    def export_k2q(self):
        return mask_plan_export_k2q(self)

    def stage_times(self):
        return mask_plan_stage_times(self)

    def close(self):
        if self._h and self._h.value:
            _lib.mask_plan_destroy(self._h)
            self._h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mask_plan_build(problem: Problem, mask_func: torch.Tensor,
                    cu_seqlens_q: Optional[torch.Tensor] = None,
                    cu_seqlens_k: Optional[torch.Tensor] = None, stream=None,
                    build_backward: bool = False, time_stages: bool = False,
                    pack_gqa: Optional[bool] = None, defer_header: bool = False) -> MaskPlan:
    """Builds a MaskPlan on the GPU (one header read-back; see include/mpb.h);
    build_backward adds the K2Q view, time_stages records HIP events around the
    planner launches, pack_gqa forces PackGQA on (True) or off (False), None
    leaves it to the library, defer_header returns without the header
    read-back (the first call that needs the header reads it and reports the
    build's errors) (all through mask_plan_build_ex)."""
    mf = _dev_ptr(mask_func, "mask_func", torch.int32)
    cq = _dev_ptr(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    ck = _dev_ptr(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    s = _stream_handle(stream)
    out = ctypes.c_void_p()
    pack = 0 if pack_gqa is None else (2 if pack_gqa else 1)
    if build_backward or time_stages or pack or defer_header:
        opt = BuildOptions(int(build_backward), int(time_stages), pack, int(defer_header))
        _check(_lib.mask_plan_build_ex(ctypes.byref(problem), ctypes.byref(opt), mf, cq, ck, s,
                                       ctypes.byref(out)))
    else:
        _check(_lib.mask_plan_build(ctypes.byref(problem), mf, cq, ck, s, ctypes.byref(out)))
    return MaskPlan(out.value, s, problem)


def mask_plan_destroy(plan: MaskPlan):
    plan.close()


def mask_plan_info(plan: MaskPlan) -> PlanInfo:
    info = PlanInfo()
    _check(_lib.mask_plan_info(plan.handle, ctypes.byref(info)))
    return info


def mask_plan_export(plan: MaskPlan) -> dict:
    """Host copies of every plan array (numpy)."""
    info = plan.info
    p = info.problem
    n_off = p.mask_heads * info.rows_total + 1
    pnnz, fnnz = int(info.header[1]), int(info.header[2])
    W = p.tile_k // 32
    tq = p.tile_q // info.signature.pack_gqa   # payload word rows per partial tile
    a = {
        "cu_rows": np.zeros(p.batch + 1, np.int32),
        "seqdesc": np.zeros((p.batch, 8), np.int32),
        "p_off": np.zeros(n_off, np.int32),
        "p_idx": np.zeros(max(pnnz, 1), np.int32),
        "p_masks": np.zeros(max(pnnz * tq * W, 1), np.uint32),
        "f_off": np.zeros(n_off, np.int32),
        "f_idx": np.zeros(max(fnnz, 1), np.int32),
        "work_desc": np.zeros((max(info.num_tasks, 1), 4), np.int32),
        "section_off": np.zeros(NUM_QUEUES + 1, np.int32),
    }
    ptrs = [ctypes.c_void_p(a[k].ctypes.data) for k in
            ("cu_rows", "seqdesc", "p_off", "p_idx", "p_masks", "f_off", "f_idx", "work_desc",
             "section_off")]
    _check(_lib.mask_plan_export(plan.handle, *ptrs))
    a["p_idx"] = a["p_idx"][:pnnz]
    a["f_idx"] = a["f_idx"][:fnnz]
    a["p_masks"] = a["p_masks"][:pnnz * tq * W].reshape(pnnz, tq, W)
    a["work_desc"] = a["work_desc"][:info.num_tasks]
    a["header"] = np.asarray(list(info.header), np.int64)
    rec = np.zeros((max(info.num_tasks, 1), TASK_REC_INTS), np.int32)
    _check(_lib.mask_plan_export_launch_order(plan.handle, ctypes.c_void_p(rec.ctypes.data)))
    a["launch"] = rec[:info.num_tasks]
    return a


def mask_plan_export_k2q(plan: MaskPlan) -> dict:
    """Host copies of the backward K2Q view (numpy); header slots 3..6 are
    (Q rows, K rows, partial nnz, full nnz)."""
    info = plan.info
    p = info.problem
    krows, pn, fn = int(info.header[4]), int(info.header[5]), int(info.header[6])
    n_off = p.mask_heads * krows + 1
    wq = p.tile_q // 32
    a = {
        "cu_krows": np.zeros(p.batch + 1, np.int32),
        "p_off": np.zeros(n_off, np.int32),
        "p_idx": np.zeros(max(pn, 1), np.int32),
        "p_masks": np.zeros(max(pn * p.tile_k * wq, 1), np.uint32),
        "f_off": np.zeros(n_off, np.int32),
        "f_idx": np.zeros(max(fn, 1), np.int32),
    }
    ptrs = [ctypes.c_void_p(a[k].ctypes.data) for k in
            ("cu_krows", "p_off", "p_idx", "p_masks", "f_off", "f_idx")]
    _check(_lib.mask_plan_export_k2q(plan.handle, *ptrs))
    a["p_idx"] = a["p_idx"][:pn]
    a["f_idx"] = a["f_idx"][:fn]
    a["p_masks"] = a["p_masks"][:pn * p.tile_k * wq].reshape(pn, p.tile_k, wq)
    a["header"] = np.asarray(list(info.header), np.int64)
    order = np.zeros(max(krows, 1), np.int32)
    _check(_lib.mask_plan_export_k2q_order(plan.handle, ctypes.c_void_p(order.ctypes.data)))
    a["order"] = order[:krows]
    return a


STAGE_NAMES = ("geometry", "classify", "schedule", "materialize", "k2q_count",
               "k2q_materialize", "span")


def mask_plan_stage_times(plan: MaskPlan) -> dict:
    """GPU microseconds of each planner stage of a build made with
    time_stages=True (-1 for a stage that did not run on its own)."""
    us = (ctypes.c_float * len(STAGE_NAMES))()
    _check(_lib.mask_plan_stage_times(plan.handle, ctypes.cast(us, ctypes.c_void_p)))
    return {n: float(v) for n, v in zip(STAGE_NAMES, us)}


def flex_attn_fwd_workspace_size(plan: MaskPlan) -> int:
    return int(_lib.flex_attn_fwd_workspace_size(plan.handle))


_CALL_PROBLEMS = {}


def _call_problem(plan: MaskPlan, q: torch.Tensor, k: torch.Tensor) -> Problem:
    """Geometry of the call as the tensors show it (checked against the plan
    binding by the library).  Problems are reused across calls and plans with
    the same binding, shapes and dtype (the library only reads them)."""
    key = (bytes(plan._bound), q.shape, k.shape, q.dtype)
    prob = _CALL_PROBLEMS.get(key)
    if prob is None:
        if len(_CALL_PROBLEMS) >= 64:
            _CALL_PROBLEMS.clear()
        prob = _CALL_PROBLEMS[key] = _make_call_problem(plan, q, k)
    return prob


def _make_call_problem(plan: MaskPlan, q: torch.Tensor, k: torch.Tensor) -> Problem:
    p = plan._bound
    dt = DTYPE_BF16 if q.dtype == torch.bfloat16 else (DTYPE_FP32 if q.dtype == torch.float32
                                                     else -1)
    if p.layout == LAYOUT_BSHD:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("BSHD q/k/v must be 4-D [B, S, H, D]")
        B, Sq, Hq, D = q.shape
        _, Sk, Hk, _ = k.shape
        return Problem(LAYOUT_BSHD, dt, B, Sq, Sk, B * Sq, B * Sk, Hq, Hk, D, p.mask_heads,
                       p.nfunc, 0, 0)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("THD q/k/v must be 3-D [T, H, D]")
    Tq, Hq, D = q.shape
    Tk, Hk, _ = k.shape
    return Problem(LAYOUT_THD, dt, p.batch, p.seqlen_q, p.seqlen_k, Tq, Tk, Hq, Hk, D,
                   p.mask_heads, p.nfunc, 0, 0)


def flex_attn_fwd_num_splits(plan: MaskPlan) -> int:
    """The library's Split-K part count for this plan (1 = no split)."""
    return int(_lib.flex_attn_fwd_num_splits(plan.handle))


def flex_attn_fwd_splitk_workspace_size(plan: MaskPlan, num_splits: int = 0) -> int:
    return int(_lib.flex_attn_fwd_splitk_workspace_size(plan.handle, int(num_splits)))


def flex_attn_fwd(plan: MaskPlan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  scale: Optional[float] = None, softcap: Optional[float] = None,
                  alibi_slopes: Optional[torch.Tensor] = None, alibi_before_softcap=False,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  force_partial: bool = False, num_splits: Optional[int] = None,
                  no_skip: bool = False):
    """Block-sparse attention forward over a plan.  Returns (O, LSE[Hq, total_q]).

    num_splits=None runs flex_attn_fwd; an int runs flex_attn_fwd_splitk with
    that many parts (0 = the library's choice).  force_partial / no_skip run
    flex_attn_fwd_ablation (identical results through slower paths).
    Allocates O/LSE/workspace with torch when not given (device memory
    only)."""
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    flags = (ABLATE_FULL_AS_PARTIAL if force_partial else 0) | (ABLATE_NO_SKIP if no_skip else 0)
    if flags and num_splits is not None:
        raise ValueError("the ablation flags and num_splits are separate entry points")
    prob = _call_problem(plan, q, k)
    _require_shape(out, "out", q.shape)
    _require_shape(lse, "lse", (q.shape[-2], prob.total_q))
    _check_slopes(alibi_slopes, q.shape[-2])
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[-2], prob.total_q), dtype=torch.float32, device=q.device)
    if workspace is None:   # a given workspace is checked by the library
        need = plan.workspace_bytes if num_splits is None else \
            flex_attn_fwd_splitk_workspace_size(plan, num_splits)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    mod = None
    if softcap or alibi_slopes is not None:
        mod = ScoreMod(1 if softcap else 0, float(softcap or 0.0),
                       1 if alibi_slopes is not None else 0,
                       _dev_ptr(alibi_slopes, "alibi_slopes", torch.float32),
                       1 if alibi_before_softcap else 0)
    sc = float(scale) if scale is not None else 1.0 / float(q.shape[-1]) ** 0.5
    head = (plan.handle, ctypes.byref(prob), _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype),
            _dev_ptr(v, "v", q.dtype), _dev_ptr(out, "out", q.dtype),
            _dev_ptr(lse, "lse", torch.float32), sc,
            ctypes.byref(mod) if mod is not None else None)
    tail = (_dev_ptr(workspace, "workspace"),
            0 if workspace is None else workspace.numel() * workspace.element_size(),
            _stream_handle(stream))
    if num_splits is not None:
        _check(_lib.flex_attn_fwd_splitk(*head, int(num_splits), *tail))
    elif flags:
        _check(_lib.flex_attn_fwd_ablation(*head, *tail, flags))
    else:
        _check(_lib.flex_attn_fwd(*head, *tail))
    return out, lse


def flex_attn_fwd_splitk_noalloc(plan: MaskPlan, q: torch.Tensor, k: torch.Tensor,
                                 v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                                 scale: Optional[float] = None, softcap: Optional[float] = None,
                                 alibi_slopes: Optional[torch.Tensor] = None,
                                 alibi_before_softcap=False, num_splits: int = 0, stream=None):
    """Split-K forward whose partial states live in the library's static
    scratch (see include/mpb.h): nothing is allocated, so out and lse must be
    given.  Calls that overlap on one GPU share the scratch and race."""
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    prob = _call_problem(plan, q, k)
    _require_shape(out, "out", q.shape)
    _require_shape(lse, "lse", (q.shape[-2], prob.total_q))
    _check_slopes(alibi_slopes, q.shape[-2])
    mod = None
    if softcap or alibi_slopes is not None:
        mod = ScoreMod(1 if softcap else 0, float(softcap or 0.0),
                       1 if alibi_slopes is not None else 0,
                       _dev_ptr(alibi_slopes, "alibi_slopes", torch.float32),
                       1 if alibi_before_softcap else 0)
    sc = float(scale) if scale is not None else 1.0 / float(q.shape[-1]) ** 0.5
    _check(_lib.flex_attn_fwd_splitk_noalloc(
        plan.handle, ctypes.byref(prob), _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype),
        _dev_ptr(v, "v", q.dtype), _dev_ptr(out, "out", q.dtype),
        _dev_ptr(lse, "lse", torch.float32), sc, ctypes.byref(mod) if mod is not None else None,
        int(num_splits), _stream_handle(stream)))
    return out, lse


def flex_attn_fwd_paged_workspace_size(plan: MaskPlan, num_splits: int = 1) -> int:
    return int(_lib.flex_attn_fwd_paged_workspace_size(plan.handle, int(num_splits)))


def flex_attn_fwd_paged(plan: MaskPlan, q: torch.Tensor, k_pages: torch.Tensor,
                        v_pages: torch.Tensor, page_table: torch.Tensor, page_size: int,
                        scale: Optional[float] = None, softcap: Optional[float] = None,
                        alibi_slopes: Optional[torch.Tensor] = None, alibi_before_softcap=False,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, stream=None,
                        num_splits: int = 1, remap: bool = True):
    """Forward with K/V in page pools (see include/mpb.h, flex_attn_fwd_paged).
    remap=False reuses the remapped tile lists an earlier call left in the
    same workspace (same plan, page table and page size).

    k_pages/v_pages: [num_pages, page_size, Hk, D] (or [num_pages*page_size,
    Hk, D]); page_table: int32 [batch, pages_per_seq].  Returns (O, LSE)."""
    p = plan._bound
    if k_pages.shape != v_pages.shape or k_pages.dtype != q.dtype:
        raise ValueError("k_pages and v_pages must match each other and q's dtype")
    if page_table.dim() != 2 or page_table.shape[0] != p.batch:
        raise ValueError("page_table must be [batch, pages_per_seq]")
    Hk, D = k_pages.shape[-2], k_pages.shape[-1]
    rows = k_pages.numel() // (Hk * D)
    if rows % page_size:
        raise ValueError("pool rows are not a multiple of page_size")
    dt = DTYPE_BF16 if q.dtype == torch.bfloat16 else (DTYPE_FP32 if q.dtype == torch.float32
                                                     else -1)
    if p.layout == LAYOUT_BSHD:
        B, Sq, Hq, Dq = q.shape
        prob = Problem(LAYOUT_BSHD, dt, B, Sq, p.seqlen_k, B * Sq, p.total_k, Hq, Hk, Dq,
                       p.mask_heads, p.nfunc, 0, 0)
    else:
        Tq, Hq, Dq = q.shape
        prob = Problem(LAYOUT_THD, dt, p.batch, p.seqlen_q, p.seqlen_k, Tq, p.total_k, Hq, Hk,
                       Dq, p.mask_heads, p.nfunc, 0, 0)
    _require_shape(out, "out", q.shape)
    _require_shape(lse, "lse", (q.shape[-2], prob.total_q))
    _check_slopes(alibi_slopes, q.shape[-2])
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[-2], prob.total_q), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(flex_attn_fwd_paged_workspace_size(plan, num_splits), 256),
                                dtype=torch.uint8, device=q.device)
    mod = None
    if softcap or alibi_slopes is not None:
        mod = ScoreMod(1 if softcap else 0, float(softcap or 0.0),
                       1 if alibi_slopes is not None else 0,
                       _dev_ptr(alibi_slopes, "alibi_slopes", torch.float32),
                       1 if alibi_before_softcap else 0)
    sc = float(scale) if scale is not None else 1.0 / float(q.shape[-1]) ** 0.5
    _check(_lib.flex_attn_fwd_paged(
        plan.handle, ctypes.byref(prob), _dev_ptr(q, "q"), _dev_ptr(k_pages, "k_pages", q.dtype),
        _dev_ptr(v_pages, "v_pages", q.dtype), _dev_ptr(page_table, "page_table", torch.int32),
        int(page_size), int(page_table.shape[1]), rows // page_size,
        _dev_ptr(out, "out", q.dtype), _dev_ptr(lse, "lse", torch.float32), sc,
        ctypes.byref(mod) if mod is not None else None, int(num_splits), 1 if remap else 0,
        _dev_ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream_handle(stream)))
    return out, lse


def flex_attn_fwd_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        out_dtype=torch.bfloat16, stream=None):
    """Merges partial attention states (see include/mpb.h, flex_attn_fwd_merge).

    o_parts: fp32 [P, total_q, Hq, D] (each part normalized over its keys);
    lse_parts: fp32 [P, Hq, total_q].  Returns (O [total_q, Hq, D] in
    out_dtype, LSE [Hq, total_q])."""
    if o_parts.dim() != 4 or lse_parts.dim() != 3:
        raise ValueError("o_parts must be [P, T, H, D] and lse_parts [P, H, T]")
    P, T, H, D = o_parts.shape
    if tuple(lse_parts.shape) != (P, H, T):
        raise ValueError("lse_parts must be [P, H, T] = %s" % ((P, H, T),))
    _require_shape(out, "out", (T, H, D))
    _require_shape(lse, "lse", (H, T))
    if out is None:
        out = torch.empty((T, H, D), dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty((H, T), dtype=torch.float32, device=o_parts.device)
    dt = DTYPE_BF16 if out.dtype == torch.bfloat16 else (DTYPE_FP32 if out.dtype == torch.float32
                                                        else -1)
    _check(_lib.flex_attn_fwd_merge(P, T, H, D, dt, _dev_ptr(o_parts, "o_parts", torch.float32),
                                    _dev_ptr(lse_parts, "lse_parts", torch.float32),
                                    _dev_ptr(out, "out"), _dev_ptr(lse, "lse", torch.float32),
                                    _stream_handle(stream)))
    return out, lse


def flex_attn_bwd_workspace_size(plan: MaskPlan) -> int:
    return int(_lib.flex_attn_bwd_workspace_size(plan.handle))


def flex_attn_bwd(plan: MaskPlan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  o: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                  scale: Optional[float] = None, softcap: Optional[float] = None,
                  alibi_slopes: Optional[torch.Tensor] = None, alibi_before_softcap=False,
                  dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                  dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None, no_skip: bool = False):
    """Backward of flex_attn_fwd over a plan built with build_backward=True:
    returns (dQ, dK, dV) for the incoming gradient dout (see include/mpb.h).
    no_skip runs flex_attn_bwd_ablation (identical results, no zero-weight
    skips).

    Allocates the outputs and the workspace with torch when not given."""
    if k.shape != v.shape or dout.shape != q.shape or o.shape != q.shape:
        raise ValueError("k/v, and q/o/dout must have matching shapes")
    prob = _call_problem(plan, q, k)
    _require_shape(dq, "dq", q.shape)
    _require_shape(dk, "dk", k.shape)
    _require_shape(dv, "dv", v.shape)
    _require_shape(lse, "lse", (q.shape[-2], prob.total_q))
    _check_slopes(alibi_slopes, q.shape[-2])
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(flex_attn_bwd_workspace_size(plan), dtype=torch.uint8,
                                device=q.device)
    mod = None
    if softcap or alibi_slopes is not None:
        mod = ScoreMod(1 if softcap else 0, float(softcap or 0.0),
                       1 if alibi_slopes is not None else 0,
                       _dev_ptr(alibi_slopes, "alibi_slopes", torch.float32),
                       1 if alibi_before_softcap else 0)
    sc = float(scale) if scale is not None else 1.0 / float(q.shape[-1]) ** 0.5
    args = (plan.handle, ctypes.byref(prob), _dev_ptr(q, "q"), _dev_ptr(k, "k", q.dtype),
            _dev_ptr(v, "v", q.dtype), _dev_ptr(o, "o", q.dtype),
            _dev_ptr(lse, "lse", torch.float32), _dev_ptr(dout, "dout", q.dtype),
            _dev_ptr(dq, "dq", q.dtype), _dev_ptr(dk, "dk", q.dtype), _dev_ptr(dv, "dv", q.dtype),
            sc, ctypes.byref(mod) if mod is not None else None, _dev_ptr(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream_handle(stream))
    if no_skip:
        _check(_lib.flex_attn_bwd_ablation(*args, ABLATE_NO_SKIP))
    else:
        _check(_lib.flex_attn_bwd(*args))
    return dq, dk, dv

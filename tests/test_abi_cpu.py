"""C-ABI checks that need no GPU.

The library must load and export every function include/mpb.h declares, and
every host-decidable refusal must happen before any device call (so these run
on a machine without a GPU).  Loaded with ctypes directly; no compute call is
made.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mpb.h")
LIB = os.path.join(ROOT, "mask_planned_block_amd", "libmpb.so")
PROBE_HEADER = os.path.join(ROOT, "include", "mpb_probe.h")
PROBE_LIB = os.path.join(ROOT, "mask_planned_block_amd", "libmpb_probe.so")
# every header under include/ and the library that must export what it declares
HEADER_LIBS = {HEADER: LIB, PROBE_HEADER: PROBE_LIB}


def _ensure_built():
    if not (os.path.exists(LIB) and os.path.exists(PROBE_LIB)):
        subprocess.check_call(["python", os.path.join(ROOT, "mask_planned_block_amd", "build.py")])


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if not n.startswith("__")))


def exported_symbols(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True,
                         text=True).stdout
    return set(line.split()[-1] for line in out.splitlines() if line.strip())


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    fns = declared_functions()
    for name in ("mask_plan_build", "flex_attn_fwd", "mask_plan_destroy", "mask_plan_info",
                 "mask_plan_export", "flex_attn_fwd_workspace_size", "mpb_status_string",
                 "mpb_last_error_detail", "mask_plan_build_ex", "mask_plan_export_k2q",
                 "mask_plan_stage_times", "flex_attn_fwd_splitk", "flex_attn_fwd_merge",
                 "flex_attn_fwd_num_splits", "flex_attn_fwd_splitk_workspace_size"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    _ensure_built()
    headers = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                     if f.endswith(".h"))
    assert set(headers) == set(HEADER_LIBS), headers
    for header, lib_path in HEADER_LIBS.items():
        handle = ctypes.CDLL(lib_path)
        missing = [n for n in declared_functions(header) if not hasattr(handle, n)]
        assert not missing, (header, missing)
        exported = exported_symbols(lib_path)
        for n in declared_functions(header):
            assert n in exported, (header, n)


def test_probe_is_outside_the_attention_library():
    """The MFMA throughput probe is a measurement helper: it lives in its own
    library and header, and libmpb.so does not export it."""
    _ensure_built()
    assert "mpb_mfma_probe" in declared_functions(PROBE_HEADER)
    assert "mpb_mfma_probe" not in declared_functions(HEADER)
    assert "mpb_mfma_probe" not in exported_symbols(LIB)


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layout", "dtype", "batch", "seqlen_q", "seqlen_k", "total_q", "total_k", "heads_q",
        "heads_k", "head_dim", "mask_heads", "nfunc", "tile_q", "tile_k")]


def _good(**kw):
    base = dict(layout=0, dtype=0, batch=2, seqlen_q=256, seqlen_k=256, total_q=512, total_k=512,
                heads_q=4, heads_k=4, head_dim=128, mask_heads=1, nfunc=1, tile_q=0, tile_k=0)
    base.update(kw)
    return Problem(**base)


def _build(lib, prob, mask_ptr=1, cu_q=None, cu_k=None):
    lib.mask_plan_build.restype = ctypes.c_int
    lib.mask_plan_build.argtypes = [ctypes.POINTER(Problem)] + [ctypes.c_void_p] * 4 + \
        [ctypes.POINTER(ctypes.c_void_p)]
    out = ctypes.c_void_p(12345)
    st = lib.mask_plan_build(ctypes.byref(prob) if prob is not None else None,
                             ctypes.c_void_p(mask_ptr) if mask_ptr else None,
                             ctypes.c_void_p(cu_q) if cu_q else None,
                             ctypes.c_void_p(cu_k) if cu_k else None, None, ctypes.byref(out))
    return st, out.value


INVALID, UNSUPPORTED = 1, 7


@pytest.mark.parametrize("kw,status", [
    (dict(layout=2), INVALID), (dict(dtype=5), INVALID), (dict(batch=0), INVALID),
    (dict(total_q=511), INVALID), (dict(total_k=100), INVALID), (dict(heads_q=0), INVALID),
    (dict(heads_q=6, heads_k=4), INVALID), (dict(mask_heads=2), INVALID),
    (dict(nfunc=2), INVALID), (dict(nfunc=0), INVALID), (dict(nfunc=4097), UNSUPPORTED),
    (dict(head_dim=96), UNSUPPORTED), (dict(tile_q=48), UNSUPPORTED),
    (dict(tile_k=48), UNSUPPORTED), (dict(tile_q=256, tile_k=256), UNSUPPORTED),
    (dict(seqlen_q=-1), INVALID),
    (dict(seqlen_k=8192 * 64, total_k=2 * 8192 * 64), UNSUPPORTED),   # > 8191 K tiles
])
def test_host_refusals_before_any_launch(lib, kw, status):
    st, out = _build(lib, _good(**kw))
    assert st == status
    assert out is None  # *out is NULL on failure
    lib.mpb_last_error_detail.restype = ctypes.c_char_p
    assert lib.mpb_last_error_detail()  # names the violated rule


def test_null_arguments(lib):
    st, out = _build(lib, None)
    assert st == INVALID and out is None
    st, out = _build(lib, _good(), mask_ptr=0)
    assert st == INVALID
    st, out = _build(lib, _good(layout=1, total_q=300, total_k=300))  # THD without prefixes
    assert st == INVALID


def test_fwd_refuses_null_plan_and_workspace_size(lib):
    lib.flex_attn_fwd.restype = ctypes.c_int
    lib.flex_attn_fwd.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_float] + \
        [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    st = lib.flex_attn_fwd(None, None, None, None, None, None, None, 1.0, None, None, 0, None)
    assert st == INVALID
    lib.mpb_status_string.restype = ctypes.c_char_p
    assert lib.mpb_status_string(5) == b"MPB_ERR_SIGNATURE_MISMATCH"
    lib.mask_plan_destroy.restype = ctypes.c_int
    assert lib.mask_plan_destroy(None) == 0


class BuildOptions(ctypes.Structure):
    _fields_ = [("build_backward", ctypes.c_int32), ("time_stages", ctypes.c_int32),
                ("pack_gqa", ctypes.c_int32), ("defer_header", ctypes.c_int32)]


def test_build_options_and_k2q_export_refusals(lib):
    lib.mask_plan_build_ex.restype = ctypes.c_int
    lib.mask_plan_build_ex.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(BuildOptions)] + \
        [ctypes.c_void_p] * 4 + [ctypes.POINTER(ctypes.c_void_p)]
    out = ctypes.c_void_p(12345)
    prob = _good()
    for opt in (BuildOptions(2, 0), BuildOptions(0, -1), BuildOptions(0, 0, 3),
                BuildOptions(0, 0, -1), BuildOptions(0, 0, 0, 2)):
        out = ctypes.c_void_p(12345)
        st = lib.mask_plan_build_ex(ctypes.byref(prob), ctypes.byref(opt),
                                    ctypes.c_void_p(1), None, None, None, ctypes.byref(out))
        assert st == INVALID and out.value is None
    # options are checked with the problem: a bad problem still names its own rule
    bad = _good(head_dim=96)
    st = lib.mask_plan_build_ex(ctypes.byref(bad), ctypes.byref(BuildOptions(1)),
                                ctypes.c_void_p(1), None, None, None, ctypes.byref(out))
    assert st == UNSUPPORTED and out.value is None
    lib.mask_plan_export_k2q.restype = ctypes.c_int
    lib.mask_plan_export_k2q.argtypes = [ctypes.c_void_p] * 7
    assert lib.mask_plan_export_k2q(None, None, None, None, None, None, None) == INVALID
    lib.mask_plan_stage_times.restype = ctypes.c_int
    lib.mask_plan_stage_times.argtypes = [ctypes.c_void_p] * 2
    assert lib.mask_plan_stage_times(None, None) == INVALID


@pytest.mark.parametrize("kw,bwd", [
    (dict(), 0),                                     # heads_q == heads_k: nothing to pack
    (dict(heads_q=8, heads_k=2, mask_heads=8), 0),   # per-head masks differ inside a group
    (dict(heads_q=6, heads_k=2), 0),                 # group of 3: not a power of two
    (dict(heads_q=32, heads_k=2, tile_q=128), 0),    # 128 / 16 = 8 tokens per plan row
    (dict(heads_q=8, heads_k=2), 1),                 # no backward view over packed tiles
])
def test_pack_gqa_refusals(lib, kw, bwd):
    """PackGQA forced on (pack_gqa = 2) where it cannot run is refused on the
    host, before any launch, with the rule named."""
    lib.mask_plan_build_ex.restype = ctypes.c_int
    lib.mask_plan_build_ex.argtypes = [ctypes.POINTER(Problem), ctypes.POINTER(BuildOptions)] + \
        [ctypes.c_void_p] * 4 + [ctypes.POINTER(ctypes.c_void_p)]
    prob = _good(tile_k=64, **kw)
    out = ctypes.c_void_p(12345)
    st = lib.mask_plan_build_ex(ctypes.byref(prob), ctypes.byref(BuildOptions(bwd, 0, 2)),
                                ctypes.c_void_p(1), None, None, None, ctypes.byref(out))
    assert st == UNSUPPORTED and out.value is None
    lib.mpb_last_error_detail.restype = ctypes.c_char_p
    assert b"PackGQA" in lib.mpb_last_error_detail()


def test_splitk_and_merge_host_refusals(lib):
    """Split-K and merge refusals are decided on the host, before any device
    call; a merge of zero rows is a no-op."""
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.flex_attn_fwd_splitk.restype = ctypes.c_int
    lib.flex_attn_fwd_splitk.argtypes = [vp] * 7 + [ctypes.c_float, vp, i32, vp, ctypes.c_size_t,
                                                    vp]
    assert lib.flex_attn_fwd_splitk(None, None, None, None, None, None, None, 1.0, None, 2, None,
                                    0, None) == INVALID
    lib.flex_attn_fwd_num_splits.restype = i32
    lib.flex_attn_fwd_num_splits.argtypes = [vp]
    assert lib.flex_attn_fwd_num_splits(None) == 1
    lib.flex_attn_fwd_splitk_workspace_size.restype = ctypes.c_size_t
    lib.flex_attn_fwd_splitk_workspace_size.argtypes = [vp, i32]
    assert lib.flex_attn_fwd_splitk_workspace_size(None, 4) == 0
    lib.flex_attn_fwd_merge.restype = ctypes.c_int
    lib.flex_attn_fwd_merge.argtypes = [i32] * 5 + [vp] * 5
    p = ctypes.c_void_p(256)
    assert lib.flex_attn_fwd_merge(0, 4, 2, 128, 0, p, p, p, p, None) == INVALID   # no parts
    assert lib.flex_attn_fwd_merge(2, -1, 2, 128, 0, p, p, p, p, None) == INVALID
    assert lib.flex_attn_fwd_merge(2, 4, 2, 96, 0, p, p, p, p, None) == UNSUPPORTED
    assert lib.flex_attn_fwd_merge(2, 4, 2, 128, 7, p, p, p, p, None) == INVALID   # dtype
    assert lib.flex_attn_fwd_merge(2, 4, 2, 128, 0, None, p, p, p, None) == INVALID
    assert lib.flex_attn_fwd_merge(2, 4, 2, 128, 0, ctypes.c_void_p(264), p, p, p,
                                   None) == INVALID                              # alignment
    assert lib.flex_attn_fwd_merge(2, 0, 2, 128, 0, None, None, None, None, None) == 0

"""Host logic of the Python binding (no GPU): the call geometry it hands the
library.  The binding describes each call by a Problem built from the tensor
shapes and reuses it across calls and plans with the same binding, shapes and
dtype; a different shape, dtype or binding must give a different Problem."""
import torch

import mask_planned_block_amd as mpb


class _Plan:
    """Stands in for a MaskPlan: the binding reads only its bound geometry."""

    def __init__(self, **kw):
        args = dict(layout=mpb.LAYOUT_BSHD, dtype=mpb.DTYPE_BF16, batch=2, seqlen_q=2048,
                    seqlen_k=2048, total_q=4096, total_k=4096, heads_q=16, heads_k=16,
                    head_dim=128, mask_heads=1, nfunc=3, tile_q=0, tile_k=0)
        args.update(kw)
        self._bound = mpb.make_problem(**args)


def _fields(p):
    return tuple(getattr(p, f) for f, _ in mpb.Problem._fields_)


def test_call_problem_follows_the_tensors():
    plan = _Plan()
    q = torch.empty(2, 2048, 16, 128, dtype=torch.bfloat16)
    k = torch.empty(2, 1500, 4, 128, dtype=torch.bfloat16)
    p = mpb._call_problem(plan, q, k)
    assert _fields(p) == (mpb.LAYOUT_BSHD, mpb.DTYPE_BF16, 2, 2048, 1500, 4096, 3000, 16, 4, 128,
                          1, 3, 0, 0)
    thd = _Plan(layout=mpb.LAYOUT_THD, batch=3, seqlen_q=900, seqlen_k=800)
    p = mpb._call_problem(thd, torch.empty(1000, 8, 64, dtype=torch.float32),
                          torch.empty(700, 2, 64, dtype=torch.float32))
    assert _fields(p) == (mpb.LAYOUT_THD, mpb.DTYPE_FP32, 3, 900, 800, 1000, 700, 8, 2, 64, 1, 3,
                          0, 0)


def test_call_problem_reuse_is_keyed_on_binding_shape_and_dtype():
    q = torch.empty(2, 2048, 16, 128, dtype=torch.bfloat16)
    a, b = _Plan(), _Plan()
    p1 = mpb._call_problem(a, q, q)
    assert mpb._call_problem(b, q, q) is p1             # same binding and tensors: reused
    assert mpb._call_problem(a, q.float(), q.float()) is not p1
    assert mpb._call_problem(_Plan(nfunc=5), q, q).nfunc == 5
    q2 = torch.empty(2, 1024, 16, 128, dtype=torch.bfloat16)
    assert mpb._call_problem(a, q2, q2).seqlen_q == 1024
    assert _fields(mpb._call_problem(a, q, q)) == _fields(p1)


def test_call_problem_cache_is_bounded():
    q = torch.empty(1, 8, 1, 64, dtype=torch.bfloat16)
    for s in range(1, 200):
        k = torch.empty(1, s, 1, 64, dtype=torch.bfloat16)
        assert mpb._call_problem(_Plan(), q, k).seqlen_k == s
    assert len(mpb._CALL_PROBLEMS) <= 64


def test_outputs_and_slopes_are_size_checked_before_any_call():
    """The library sees bare pointers, so the binding refuses an output or a
    slope array whose size differs from what the kernels write or read
    (ValueError before any library call; CPU tensors never reach it)."""
    import pytest
    plan = _Plan(heads_q=4, heads_k=4, batch=1, seqlen_q=64, seqlen_k=64, total_q=64,
                 total_k=64)
    q = torch.empty(1, 64, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        mpb.flex_attn_fwd(plan, q, q, q, out=torch.empty(1, 63, 4, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="lse"):
        mpb.flex_attn_fwd(plan, q, q, q, lse=torch.empty(4, 63))
    with pytest.raises(ValueError, match="alibi_slopes"):
        mpb.flex_attn_fwd(plan, q, q, q, alibi_slopes=torch.empty(3))
    lse = torch.empty(4, 64)
    with pytest.raises(ValueError, match="dq"):
        mpb.flex_attn_bwd(plan, q, q, q, q, lse, q, dq=torch.empty(1, 64, 4, 64))
    with pytest.raises(ValueError, match="dk"):
        mpb.flex_attn_bwd(plan, q, q, q, q, lse, q, dk=torch.empty(2, 64, 4, 128))
    with pytest.raises(ValueError, match="lse"):
        mpb.flex_attn_bwd(plan, q, q, q, q, torch.empty(64, 4), q)
    parts = torch.empty(2, 64, 4, 128)
    with pytest.raises(ValueError, match="lse"):
        mpb.flex_attn_fwd_merge(parts, torch.empty(2, 4, 64), lse=torch.empty(4, 65))

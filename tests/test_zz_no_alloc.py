"""tsa_forward_fused_noalloc through the C ABI (GPU): the entry point for callers that
cannot allocate, whose scratch is a static device array of the library.

It must give tsa_forward_fused's results bit for bit (budgets, index sets, outputs),
call after call on the same GPU, although the scratch keeps the previous call's
contents: a larger problem, then a smaller one, then the larger one again.
"""
import ctypes

import numpy as np
import pytest
import torch

from tests.parity import say, to_dev
from token_sparse_attention_proxy_amd import _lib, inputs
from token_sparse_attention_proxy_amd import tsa as T

pytestmark = pytest.mark.gpu

CASES = [
    inputs.small_workload("bf16", B=2, Hq=8, Hkv=2, L=3000, d=128, w=64, tau=0.05, seed_base=9600),
    inputs.small_workload("bf16", B=1, Hq=4, Hkv=1, L=1000, d=128, w=32, tau=0.2, seed_base=9610),
    inputs.small_workload("bf16", B=2, Hq=8, Hkv=2, L=3000, d=128, w=64, tau=0.05, seed_base=9600),
]


def _noalloc(prob, q, k, v):
    lib = _lib.load()
    o = torch.full_like(q, float("nan"))
    budget = torch.full(prob.budget_shape, -7, dtype=torch.int32, device=q.device)
    idx = torch.full((prob.B, prob.Hq, prob.L), -7, dtype=torch.int32, device=q.device)
    p = prob.c()
    st = torch.cuda.current_stream(q.device).cuda_stream
    _lib.check(lib.tsa_forward_fused_noalloc(ctypes.byref(p), q.data_ptr(), k.data_ptr(),
                                             v.data_ptr(), o.data_ptr(), budget.data_ptr(),
                                             idx.data_ptr(), st), "tsa_forward_fused_noalloc")
    return o, budget, idx


def test_noalloc_equals_fused_call_after_call():
    for n, wl in enumerate(CASES):
        say(f"case noalloc call {n}: {wl.name}")
        q, k, v = inputs.make_qkv(wl)
        qd, kd, vd = to_dev(q, wl.dtype), to_dev(k, wl.dtype), to_dev(v, wl.dtype)
        prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, float(wl.taus[0]), wl.dtype)
        o, budget, idx = _noalloc(prob, qd, kd, vd)
        o_ref, b_ref, i_ref = T.tsa_forward_fused(prob, qd, kd, vd)
        torch.cuda.synchronize()
        say(f"  budget {budget.cpu().tolist()} (workspace path {b_ref.cpu().tolist()})")
        assert torch.equal(budget, b_ref)
        assert torch.equal(idx, i_ref)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))


def test_noalloc_per_head_budgets():
    wl = CASES[1]
    say("case noalloc per-head budgets")
    q, k, v = inputs.make_qkv(wl)
    qd, kd, vd = to_dev(q, wl.dtype), to_dev(k, wl.dtype), to_dev(v, wl.dtype)
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, 0.2, wl.dtype, T.TSA_FLAG_PER_HEAD_BUDGET)
    o, budget, idx = _noalloc(prob, qd, kd, vd)
    o_ref, b_ref, i_ref = T.tsa_forward_fused(prob, qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(budget, b_ref) and torch.equal(idx, i_ref)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))


def test_noalloc_rejects_oversized_problem():
    """A problem whose scratch exceeds the static array is refused before anything runs."""
    lib = _lib.load()
    p = T.Problem(1, 64, 8, 1 << 21, 128, 64, 0.05, "bf16")
    need = T.fused_workspace_bytes(p)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    st = lib.tsa_forward_fused_noalloc(ctypes.byref(p.c()), fake, fake, fake, fake, fake, fake,
                                       None)
    assert st == _lib.TSA_ERR_UNSUPPORTED
    assert "scratch" in lib.tsa_last_error().decode()
    # the largest workload of the bench fits
    big = T.Problem(2, 28, 4, 65536, 128, 128, 0.1, "bf16", T.TSA_FLAG_PER_HEAD_BUDGET)
    assert T.fused_workspace_bytes(big) <= _lib.NOALLOC_SCRATCH_BYTES
    say(f"  scratch {need} > {_lib.NOALLOC_SCRATCH_BYTES} refused")

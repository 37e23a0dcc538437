"""The alternative readings (TSA_FLAG_* bits) on the GPU against the fp64 oracle.

  NONCAUSAL_PROXY  every proxy row sees all L keys;
  PER_HEAD_BUDGET  one coverage cut per head (ragged budgets [B,Hq]);
  KEEP_WINDOW      the w proxy positions are never pruned.

Each step is compared as in the main reading: scores within the score
tolerance, budgets and sets bit-exact (near-ties reported), outputs within
the output tolerance; the fused path equals the step-by-step path bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import tsa_oracle as O
from tests.parity import (assert_outputs_close, assert_scores_close, compare_forward, say, to_dev,
                          to_np)
from token_sparse_attention_proxy_amd import inputs
from token_sparse_attention_proxy_amd import tsa as T

pytestmark = pytest.mark.gpu

NC, PH, KW = T.TSA_FLAG_NONCAUSAL_PROXY, T.TSA_FLAG_PER_HEAD_BUDGET, T.TSA_FLAG_KEEP_WINDOW
ALL_FLAG_SETS = [NC, PH, KW, NC | PH, NC | KW, PH | KW, NC | PH | KW]


def _name(flags):
    return "+".join(n for n, f in (("noncausal", NC), ("perhead", PH), ("keep", KW)) if flags & f)


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


# --------------------------------------------------------------------------- S1
SCORE_CASES = [
    inputs.small_workload("bf16", B=1, Hq=8, Hkv=2, L=1000, d=128, w=64, seed_base=9500),
    inputs.small_workload("bf16", B=2, Hq=4, Hkv=4, L=513, d=64, w=33, seed_base=9510),
    inputs.small_workload("bf16", B=1, Hq=6, Hkv=2, L=300, d=128, w=300, seed_base=9520),
    inputs.small_workload("f32", B=1, Hq=4, Hkv=2, L=257, d=128, w=20, seed_base=9530),
    inputs.small_workload("f32", B=1, Hq=2, Hkv=1, L=700, d=64, w=16, seed_base=9540),
]


@pytest.mark.parametrize("wl", SCORE_CASES, ids=[w.name for w in SCORE_CASES])
def test_score_noncausal(wl):
    say(f"case score noncausal {wl.name}")
    q, k, _ = inputs.make_qkv(wl)
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, 0.05, wl.dtype, NC)
    s = to_np(T.tsa_score(prob, to_dev(q, wl.dtype), to_dev(k, wl.dtype)))
    ref = O.proxy_scores(q, k, wl.w, causal=False)
    assert_scores_close(s, ref, f" noncausal {wl.name}")
    assert np.allclose(s.sum(-1), 1.0, atol=1e-5)


# --------------------------------------------------------------------------- S2
BUDGET_CASES = [
    # (B, Hq, L, w, seed, ties, zero_frac, alpha)
    (1, 8, 1000, 64, 1, False, 0.0, 1.0),
    (2, 32, 8192, 64, 2, False, 0.0, 0.3),
    (2, 4, 777, 100, 3, True, 0.0, 1.0),
    (1, 3, 5000, 1, 4, False, 0.5, 0.2),
    (3, 2, 64, 64, 6, True, 0.3, 1.0),
    (1, 28, 4096, 16, 7, False, 0.0, 5.0),
]


@pytest.mark.parametrize("flags", [PH, KW, PH | KW], ids=_name)
@pytest.mark.parametrize("case", BUDGET_CASES, ids=[str(c) for c in BUDGET_CASES])
def test_budget_readings(case, flags):
    B, Hq, L, w, seed, ties, zf, alpha = case
    say(f"case budget {_name(flags)} {case}")
    s = inputs.make_scores(B, Hq, L, seed=seed, ties=ties, zero_frac=zf, alpha=alpha)
    sd = to_dev(s, "f32")
    keep = w if flags & KW else 0
    for tau in (0.0, 1e-4, 0.01, 0.05, 0.1, 0.3, 0.5, 0.9, 0.999):
        prob = T.Problem(B, Hq, Hq, L, 128, w, tau, "bf16", flags)
        got = to_np(T.tsa_budget(prob, sd))
        want = O.coverage_budget(s.astype(np.float64), tau, per_head=bool(flags & PH), keep=keep)
        assert got.shape == want.shape
        assert np.array_equal(got, want), (tau, got, want)


# --------------------------------------------------------------------------- S3
@pytest.mark.parametrize("keep", [0, 1, 37, 300])
def test_select_ragged_budgets_and_window(keep):
    """Per-head budgets [B,Hq] (ragged) and a kept window."""
    B, H, L = 2, 6, 1025
    say(f"case select per-head keep={keep}")
    s = inputs.make_scores(B, H, L, seed=40 + keep, ties=True, zero_frac=0.1)
    rng = np.random.default_rng(keep)
    budget = rng.integers(max(keep, 1), L + 1, size=(B, H)).astype(np.int32)
    budget[0, 0], budget[1, -1] = max(keep, 1), L
    flags = PH | (KW if keep else 0)
    prob = T.Problem(B, H, H, L, 128, max(keep, 1), 0.05, "bf16", flags)
    idx, rank = T.tsa_select(prob, to_dev(s, "f32"), torch.from_numpy(budget).cuda())
    ridx, rrank = O.select_heads(s.astype(np.float64), budget, keep=keep)
    assert np.array_equal(to_np(idx), ridx)
    assert np.array_equal(to_np(rank), rrank)


# --------------------------------------------------------------------------- S4-S6 with ragged budgets
@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_ragged_gather_attention_scatter(dt, d):
    B, Hq, Hkv, L = 2, 8, 2, 900
    say(f"case ragged steps {dt} d={d}")
    q = inputs.make_dense((B, Hq, L, d), 61, dt)
    k = inputs.make_dense((B, Hkv, L, d), 62, dt, scale=1.5)
    v = inputs.make_dense((B, Hkv, L, d), 63, dt)
    rng = np.random.default_rng(64)
    budget = rng.integers(1, L + 1, size=(B, Hq)).astype(np.int32)
    budget[0, 0], budget[0, 1], budget[1, 7] = 1, L, 257
    s = inputs.make_scores(B, Hq, L, seed=65)
    idx_np, rank_np = O.select_heads(s.astype(np.float64), budget)
    prob = T.Problem(B, Hq, Hkv, L, d, 1, 0.05, dt, PH)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    bd = torch.from_numpy(budget).cuda()
    idd, rkd = torch.from_numpy(idx_np).cuda(), torch.from_numpy(rank_np).cuda()
    qc, kc, vc = T.tsa_gather(prob, qd, kd, vd, idd, bd)
    qc_r, kc_r, vc_r = O.gather(q, k, v, idx_np, budget)
    for b in range(B):
        for h in range(Hq):
            K = int(budget[b, h])
            for got, want in ((qc, qc_r), (kc, kc_r), (vc, vc_r)):
                assert np.array_equal(to_np(got[b, h, :K]), want[b, h, :K])
    oc = T.tsa_attention(prob, qc, kc, vc, bd, 1)
    o = T.tsa_scatter(prob, oc, rkd)
    o_idx = torch.full_like(qd, float("nan"))
    T.tsa_zero_unselected(prob, rkd, o_idx)
    T.tsa_attention_indexed(prob, qd, kd, vd, idd, bd, o_idx)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(o_idx))
    ref = O.scatter(O.attention_heads(qc_r, kc_r, vc_r, budget), idx_np, budget)
    assert_outputs_close(to_np(o), ref, dt, what=f" ragged {dt} d={d}")


# --------------------------------------------------------------------------- whole op
SMALL = [
    inputs.small_workload("bf16", B=1, Hq=8, Hkv=2, L=1000, d=128, w=64, tau=0.05, seed_base=9600),
    inputs.small_workload("bf16", B=2, Hq=6, Hkv=2, L=700, d=128, w=32, tau=0.2, plant_frac=0.02,
                          plant_amp=5.0, seed_base=9610),
    inputs.small_workload("bf16", B=1, Hq=4, Hkv=1, L=2048, d=64, w=64, tau=0.3, zipf_s=1.1,
                          plant="none", seed_base=9620),
    inputs.small_workload("f32", B=1, Hq=4, Hkv=2, L=600, d=64, w=16, tau=0.1, seed_base=9630),
]


@pytest.mark.parametrize("flags", ALL_FLAG_SETS, ids=_name)
@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_forward_readings_small(wl, flags):
    tau = wl.taus[0]
    say(f"case forward {_name(flags)} {wl.name} tau={tau}")
    q, k, v = inputs.make_qkv(wl)
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, float(tau), wl.dtype, flags)
    qd, kd, vd = to_dev(q, wl.dtype), to_dev(k, wl.dtype), to_dev(v, wl.dtype)
    o, budget, idx = T.tsa_forward(prob, qd, kd, vd)
    o2 = torch.full_like(qd, float("nan"))
    o2, budget2, idx2 = T.tsa_forward_fused(prob, qd, kd, vd, o2)
    torch.cuda.synchronize()
    assert torch.equal(budget, budget2) and torch.equal(idx, idx2)
    assert torch.equal(_bits(o), _bits(o2))
    ref = O.forward(q, k, v, wl.w, tau, causal=not flags & NC, per_head=bool(flags & PH),
                    keep_window=bool(flags & KW))
    assert_scores_close(to_np(T.tsa_score(prob, qd, kd)), ref["s"], f" {_name(flags)}")
    compare_forward(ref, to_np(o), to_np(budget), to_np(idx), q, k, v, tau, wl.dtype,
                    per_head=bool(flags & PH), keep=wl.w if flags & KW else 0)


@pytest.mark.parametrize("flags", [NC, PH, KW, NC | PH | KW], ids=_name)
def test_forward_readings_full_size(flags):
    """The 32K Zipf workload at full size, in the launch configuration the bench
    times: scores, budgets and sets in full, outputs on sampled rows."""
    wl = inputs.WORKLOADS["llama8b_bf16_L32k_zipf"]
    tau = wl.taus[1]
    say(f"case forward full {_name(flags)} {wl.name} tau={tau}: generating inputs")
    q, k, v = inputs.make_qkv(wl)
    qd, kd, vd = to_dev(q, wl.dtype), to_dev(k, wl.dtype), to_dev(v, wl.dtype)
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, float(tau), wl.dtype, flags)
    o, budget, idx = T.tsa_forward_fused(prob, qd, kd, vd)
    s_gpu = to_np(T.tsa_score(prob, qd, kd))
    torch.cuda.synchronize()
    say("  oracle")
    causal, per_head, keep = not flags & NC, bool(flags & PH), wl.w if flags & KW else 0
    s_ref = O.proxy_scores(q, k, wl.w, causal=causal)
    assert_scores_close(s_gpu, s_ref, f" full {_name(flags)}")
    b_ref = O.coverage_budget(s_ref, tau, per_head=per_head, keep=keep)
    idx_ref, _ = O.select_heads(s_ref, b_ref, keep=keep)
    bud = to_np(budget)
    say(f"  budget K/L: mean {np.mean(bud) / wl.L:.4f} min {np.min(bud) / wl.L:.4f} "
        f"max {np.max(bud) / wl.L:.4f}")
    compare_forward({"s": s_ref, "budget": b_ref, "idx": idx_ref}, to_np(o), bud, to_np(idx),
                    q, k, v, tau, wl.dtype, sample_rows=4, seed=11, per_head=per_head, keep=keep)
    del o, budget, idx, qd, kd, vd
    torch.cuda.empty_cache()

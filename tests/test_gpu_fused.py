"""The fused path (GPU): tsa_attention_indexed and tsa_forward_fused.

The fused kernel reads Q, K, V through the index set and writes O rows to
their sequence positions, so it must equal gather -> attention -> scatter
bit for bit (the MFMA order is the same), and through that the oracle.
Both comparisons are made: bitwise against the step-by-step entry points,
and element-wise against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

from oracle import tsa_oracle as O
from tests.parity import assert_outputs_close, check_rows_written, compare_forward, say, to_dev, to_np
from tests.test_gpu_forward import FULL, SMALL
from token_sparse_attention_proxy_amd import inputs
from token_sparse_attention_proxy_amd import tsa as T

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


INDEXED_CASES = [
    # dtype, B, Hq, Hkv, L, d, budgets
    ("bf16", 1, 8, 2, 1000, 128, [613]),
    ("bf16", 2, 4, 4, 777, 128, [777, 300]),
    ("bf16", 1, 4, 1, 1500, 64, [1337]),
    ("bf16", 2, 6, 2, 600, 64, [1, 65]),
    ("bf16", 1, 3, 3, 129, 128, [128]),
    ("bf16", 1, 2, 2, 400, 128, [130]),         # 3 key tiles: a pair and a lone last tile
    ("bf16", 1, 4, 2, 900, 128, [449]),         # 8 tiles, the last holding one row
    ("f32", 1, 4, 2, 1000, 64, [900]),
    ("f32", 2, 4, 4, 300, 128, [33, 300]),
]


@pytest.mark.parametrize("case", INDEXED_CASES, ids=[str(c) for c in INDEXED_CASES])
def test_attention_indexed_equals_steps_and_oracle(case):
    dt, B, Hq, Hkv, L, d, budgets = case
    say(f"case attention_indexed {case}")
    q = inputs.make_dense((B, Hq, L, d), 41, dt)
    k = inputs.make_dense((B, Hkv, L, d), 42, dt, scale=1.5)
    v = inputs.make_dense((B, Hkv, L, d), 43, dt)
    budget = np.array(budgets, np.int32)
    idx, rank = inputs.make_indices(B, Hq, L, budget, seed=44)
    prob = T.Problem(B, Hq, Hkv, L, d, 1, 0.05, dt)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    bd = torch.from_numpy(budget).cuda()
    idd, rkd = torch.from_numpy(idx).cuda(), torch.from_numpy(rank).cuda()
    # canary: unselected rows must be left as they were
    o = torch.full((B, Hq, L, d), float("nan"), dtype=qd.dtype, device="cuda")
    T.tsa_attention_indexed(prob, qd, kd, vd, idd, bd, o)
    qc, kc, vc = T.tsa_gather(prob, qd, kd, vd, idd, bd)
    oc = T.tsa_attention(prob, qc, kc, vc, bd, 1)
    o_steps = T.tsa_scatter(prob, oc, rkd)
    torch.cuda.synchronize()
    sel = torch.from_numpy(rank >= 0).cuda()
    assert torch.equal(_bits(o)[sel], _bits(o_steps)[sel])
    assert torch.isnan(o[~sel].float()).all()
    # the oracle on the compact tensors, scattered back
    qc_r, kc_r, vc_r = O.gather(q, k, v, idx, budget)
    ref = O.scatter(O.attention_heads(qc_r, kc_r, vc_r, budget), idx, budget)
    got = to_np(o)
    got[~(rank >= 0)] = 0.0
    assert_outputs_close(got, ref, dt, what=f" indexed {case}")


@pytest.mark.parametrize("case", INDEXED_CASES, ids=[str(c) for c in INDEXED_CASES])
def test_attention_qo_indexed_equals_steps(case):
    """Compact K and V, Q read and O written through the index set (the whole op's attention):
    the same bits as gather -> attention -> scatter on the selected rows, and the K/V-only
    gather writes the same compact K and V as the full one."""
    dt, B, Hq, Hkv, L, d, budgets = case
    say(f"case attention_qo_indexed {case}")
    q = inputs.make_dense((B, Hq, L, d), 51, dt)
    k = inputs.make_dense((B, Hkv, L, d), 52, dt, scale=1.5)
    v = inputs.make_dense((B, Hkv, L, d), 53, dt)
    budget = np.array(budgets, np.int32)
    idx, rank = inputs.make_indices(B, Hq, L, budget, seed=54)
    prob = T.Problem(B, Hq, Hkv, L, d, 1, 0.05, dt)
    qd, kd, vd = to_dev(q, dt), to_dev(k, dt), to_dev(v, dt)
    bd = torch.from_numpy(budget).cuda()
    idd, rkd = torch.from_numpy(idx).cuda(), torch.from_numpy(rank).cuda()
    qc, kc, vc = T.tsa_gather(prob, qd, kd, vd, idd, bd)
    oc = T.tsa_attention(prob, qc, kc, vc, bd, 1)
    o_steps = T.tsa_scatter(prob, oc, rkd)
    _, kc2, vc2 = T.tsa_gather(prob, qd, kd, vd, idd, bd, with_q=False)
    o = torch.full((B, Hq, L, d), float("nan"), dtype=qd.dtype, device="cuda")
    T.tsa_attention_qo_indexed(prob, qd, kc2, vc2, idd, bd, o)
    torch.cuda.synchronize()
    for b in range(B):
        n = int(budget[b])
        assert torch.equal(_bits(kc2[b, :, :n]), _bits(kc[b, :, :n]))
        assert torch.equal(_bits(vc2[b, :, :n]), _bits(vc[b, :, :n]))
    sel = torch.from_numpy(rank >= 0).cuda()
    assert torch.equal(_bits(o)[sel], _bits(o_steps)[sel])
    assert torch.isnan(o[~sel].float()).all()


@pytest.mark.parametrize("late_key", [700, 130])
def test_attention_indexed_recompute_path(late_key):
    """Identity index set on inputs that force the exact-max recompute: the
    second walk over the keys must re-publish the index ring and give the
    dense kernel's result bit for bit."""
    say(f"case attention_indexed recompute late key {late_key}")
    B, H, L, d = 1, 2, 900, 128
    rng = np.random.default_rng(77)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    q[:, :, late_key:] += 10.0 * u
    k[:, :, late_key] += 60.0 * u
    prob = T.Problem(B, H, H, L, d, 1, 0.05, "bf16")
    qd, kd, vd = (to_dev(x.astype(np.float32), "bf16") for x in (q, k, v))
    idx = torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, H, 1).contiguous()
    bd = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o = torch.zeros_like(qd)
    T.tsa_attention_indexed(prob, qd, kd, vd, idx, bd, o)
    dense = T.tsa_attention(prob, qd, kd, vd, None, 1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(dense))


@pytest.mark.parametrize("late_key", [700, 130])
def test_attention_qo_recompute_path(late_key):
    """The whole op's attention (compact K and V, Q read and O written through the index set)
    on inputs that force the exact-max recompute, with the identity index set: the dense
    kernel's result bit for bit."""
    say(f"case attention_qo_indexed recompute late key {late_key}")
    B, H, L, d = 1, 2, 900, 128
    rng = np.random.default_rng(78)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    q[:, :, late_key:] += 10.0 * u
    k[:, :, late_key] += 60.0 * u
    prob = T.Problem(B, H, H, L, d, 1, 0.05, "bf16")
    qd, kd, vd = (to_dev(x.astype(np.float32), "bf16") for x in (q, k, v))
    idx = torch.arange(L, dtype=torch.int32, device="cuda").repeat(B, H, 1).contiguous()
    bd = torch.full((B,), L, dtype=torch.int32, device="cuda")
    o = torch.full_like(qd, float("nan"))
    T.tsa_attention_qo_indexed(prob, qd, kd, vd, idx, bd, o)
    dense = T.tsa_attention(prob, qd, kd, vd, None, 1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(dense))
    # and the oracle, which the recompute must still match
    qr, kr, vr = (to_np(x) for x in (qd, kd, vd))
    for h in range(H):
        ref = O.causal_attention(qr[0, h], kr[0, h], vr[0, h])
        assert_outputs_close(to_np(o)[0, h], ref, "bf16", what=f" qo recompute h={h}")


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_forward_fused_small(wl):
    tau = wl.taus[0]
    say(f"case forward_fused {wl.name} tau={tau}")
    q, k, v = inputs.make_qkv(wl)
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, float(tau), wl.dtype)
    qd, kd, vd = to_dev(q, wl.dtype), to_dev(k, wl.dtype), to_dev(v, wl.dtype)
    # stale output contents must not leak: unselected rows are zeroed by the call
    o = torch.full_like(qd, float("nan"))
    o, budget, idx = T.tsa_forward_fused(prob, qd, kd, vd, o)
    o2, budget2, idx2 = T.tsa_forward(prob, qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(budget, budget2) and torch.equal(idx, idx2)
    assert torch.equal(_bits(o), _bits(o2))
    ref = O.forward(q, k, v, wl.w, tau)
    compare_forward(ref, to_np(o), to_np(budget), to_np(idx), q, k, v, tau, wl.dtype)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "forward"])
def test_forward_tau0_equals_dense(fused):
    """tau = 0 keeps every token: both whole-op paths give the dense kernel's bits."""
    wl = inputs.small_workload("bf16", B=1, Hq=8, Hkv=2, L=1000, d=128, w=64, seed_base=9200)
    say(f"case tau=0 vs dense, fused={fused}")
    q, k, v = inputs.make_qkv(wl)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    prob = T.Problem(1, 8, 2, 1000, 128, 64, 0.0, "bf16")
    o, budget, _ = (T.tsa_forward_fused if fused else T.tsa_forward)(prob, qd, kd, vd)
    dense = T.tsa_attention(prob, qd, kd, vd, None, 4)
    torch.cuda.synchronize()
    assert int(budget[0]) == 1000
    assert torch.equal(_bits(o), _bits(dense))


@pytest.mark.parametrize("name", FULL)
def test_forward_fused_full_size(name):
    """Full sizes, the launch configuration the bench times: the fused call
    equals the step-by-step call bit for bit, and sampled rows match the
    oracle (index sets and budgets are checked in full)."""
    wl = inputs.WORKLOADS[name]
    say(f"case forward_fused full {name}: generating inputs")
    q, k, v = inputs.make_qkv(wl)
    qd, kd, vd = to_dev(q, wl.dtype), to_dev(k, wl.dtype), to_dev(v, wl.dtype)
    tau = wl.taus[0]
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, float(tau), wl.dtype)
    # NaN before the call: a workgroup that never writes its rows cannot pass
    o = torch.full((wl.B, wl.Hq, wl.L, wl.d), float("nan"), dtype=qd.dtype, device=qd.device)
    o, budget, idx = T.tsa_forward_fused(prob, qd, kd, vd, o)
    o2, budget2, idx2 = T.tsa_forward(prob, qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(budget, budget2) and torch.equal(idx, idx2)
    assert torch.equal(_bits(o), _bits(o2))
    del o2, budget2, idx2
    check_rows_written(o, idx, budget)
    say("  oracle scores")
    s_ref = O.proxy_scores(q, k, wl.w)
    b_ref = O.coverage_budget(s_ref, tau)
    idx_ref, _ = O.select_heads(s_ref, b_ref)
    ref = {"s": s_ref, "budget": b_ref, "idx": idx_ref}
    sample = 0 if wl.L <= 1024 else 6
    if sample == 0:
        qc, kc, vc = O.gather(q, k, v, idx_ref, b_ref)
        ref["o"] = O.scatter(O.attention_heads(qc, kc, vc, b_ref), idx_ref, b_ref)
    compare_forward(ref, to_np(o), to_np(budget), to_np(idx), q, k, v, tau, wl.dtype,
                    sample_rows=sample, seed=7)
    del o, budget, idx, qd, kd, vd
    torch.cuda.empty_cache()


def test_fused_steps_compose_to_forward_fused():
    """score -> budget -> select -> zero_unselected -> attention_indexed, called
    one by one, give tsa_forward_fused's result bit for bit."""
    wl = SMALL[1]
    say("case fused steps == forward_fused")
    q, k, v = inputs.make_qkv(wl)
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, 0.2, wl.dtype)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o, budget, idx = T.tsa_forward_fused(prob, qd, kd, vd)
    s = T.tsa_score(prob, qd, kd)
    bud = T.tsa_budget(prob, s)
    idx2, rank = T.tsa_select(prob, s, bud)
    o2 = torch.full_like(qd, float("nan"))
    T.tsa_zero_unselected(prob, rank, o2)
    T.tsa_attention_indexed(prob, qd, kd, vd, idx2, bud, o2)
    torch.cuda.synchronize()
    assert torch.equal(budget, bud) and torch.equal(idx, idx2)
    assert torch.equal(_bits(o), _bits(o2))

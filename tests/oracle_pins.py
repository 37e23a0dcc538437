"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes an oracle module ``O`` (the real one, or a copy with a
planted mistake in ``tests/test_oracle_mutants.py``) and raises
AssertionError when the module disagrees with:

* the hand-derived worked example in ``tests/golden/worked_example_L3.json``;
* closed forms (identical keys, Q = 0, constant V, a single key);
* library routines (``torch.softmax``, ``torch.nn.functional.scaled_dot_product_attention``
  in float64 on the CPU, ``itertools`` enumeration);
* brute force over all subsets on tiny inputs;
* invariants (mass conservation, zero rows, linearity in V, monotonicity in tau).
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _frac(x: str) -> float:
    return float(Fraction(x))


# --------------------------------------------------------------------------- worked example
def load_worked_example():
    with open(os.path.join(GOLDEN, "worked_example_L3.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], dtype=np.float64).reshape(1, 1, 3, 1)
    k = np.log(np.array(ex["k_log"], dtype=np.float64)).reshape(1, 1, 3, 1)
    v = np.array(ex["v"], dtype=np.float64).reshape(1, 1, 3, 1)
    return ex, q, k, v


def pin_worked_example(O):
    ex, q, k, v = load_worked_example()
    s = O.proxy_scores(q, k, ex["w"])
    want = np.array([_frac(x) for x in ex["scores"]])
    assert np.allclose(s[0, 0], want, rtol=0, atol=1e-14), (s, want)
    exact_s = want.reshape(1, 1, 3)
    for case in ex["cases"]:
        kb = O.coverage_budget(exact_s, case["tau"])
        assert int(kb[0]) == case["budget"], (case, kb)
        idx, rank = O.select_heads(exact_s, kb)
        assert list(idx[0, 0, :kb[0]]) == case["idx"], (case, idx)
        out = O.forward(q, k, v, ex["w"], case["tau"])
        assert int(out["budget"][0]) == case["budget"]
        want_o = np.array([_frac(x) for x in case["o"]])
        assert np.allclose(out["o"][0, 0, :, 0], want_o, rtol=0, atol=1e-13), (case, out["o"])


# --------------------------------------------------------------------------- step 1: scores
def pin_scores_mass(O):
    r = _rng(11)
    for (B, Hq, Hkv, L, d, w) in [(2, 4, 2, 37, 8, 5), (1, 3, 1, 20, 4, 20), (1, 2, 2, 9, 16, 1)]:
        q = r.standard_normal((B, Hq, L, d)) * 2
        k = r.standard_normal((B, Hkv, L, d)) * 2
        s = O.proxy_scores(q, k, w)
        assert s.shape == (B, Hq, L)
        assert np.all(s >= 0)
        assert np.allclose(s.sum(-1), 1.0, rtol=0, atol=1e-12), s.sum(-1)


def pin_scores_identical_keys(O):
    """All keys equal: each proxy row r is uniform over its r+1 visible keys."""
    r = _rng(12)
    for (L, w, d) in [(40, 8, 4), (12, 12, 2), (30, 1, 3)]:
        k = np.tile(r.standard_normal(d), (L, 1)).reshape(1, 1, L, d)
        q = r.standard_normal((1, 1, L, d)) * 3
        s = O.proxy_scores(q, k, w)[0, 0]
        want = np.array([sum(Fraction(1, rr + 1) for rr in range(max(j, L - w), L)) / w
                         for j in range(L)], dtype=np.float64)
        assert np.allclose(s, want, rtol=0, atol=1e-13), (s, want)


def pin_scores_w1_softmax(O):
    """w = 1: importance is one softmax row of the last query over all keys (library)."""
    r = _rng(13)
    B, Hq, Hkv, L, d = 1, 4, 2, 25, 8
    q = r.standard_normal((B, Hq, L, d))
    k = r.standard_normal((B, Hkv, L, d))
    s = O.proxy_scores(q, k, 1)
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    logits = torch.einsum("bhd,bhld->bhl", torch.from_numpy(q[:, :, -1]), kt) / math.sqrt(d)
    want = torch.softmax(logits, dim=-1).numpy()
    assert np.allclose(s, want, rtol=0, atol=1e-14)


def pin_scores_proxy_window(O):
    """Only the last w query rows matter: changing earlier queries leaves s unchanged,
    changing a proxy query changes it; a planted key shows up in its own column."""
    r = _rng(14)
    B, Hq, Hkv, L, d, w = 1, 2, 1, 30, 8, 6
    q = r.standard_normal((B, Hq, L, d))
    k = r.standard_normal((B, Hkv, L, d))
    s0 = O.proxy_scores(q, k, w)
    q2 = q.copy()
    q2[:, :, : L - w] = r.standard_normal((B, Hq, L - w, d))
    assert np.array_equal(O.proxy_scores(q2, k, w), s0)
    q3 = q.copy()
    q3[:, :, L - w] += 1.0
    assert not np.allclose(O.proxy_scores(q3, k, w), s0)
    # a key aligned with every proxy query becomes the most important token
    k4 = k.copy()
    k4[0, 0, 7] = 6.0 * q[0, :, L - w:].sum(axis=(0, 1)) / np.linalg.norm(q[0, :, L - w:].sum(axis=(0, 1)))
    s4 = O.proxy_scores(q, k4, w)
    assert int(np.argmax(s4[0, 0])) == 7 and int(np.argmax(s4[0, 1])) == 7


# --------------------------------------------------------------------------- step 2: budget
def _dyadic_scores(r, B, H, L, zero_frac=0.2):
    """Rows of multiples of 2^-10 summing to <= 1 (exact in every reading)."""
    x = r.integers(0, 64, size=(B, H, L)).astype(np.float64)
    x[r.random((B, H, L)) < zero_frac] = 0.0
    x[..., 0] += 1.0
    return x / 1024.0


def _bruteforce_budget(s_b, tau):
    """P = max{p in [0, L-1] : min over p-subsets of the head-mean mass <= tau}."""
    H, L = s_b.shape
    mean = [sum(Fraction(float(s_b[h, j])) for h in range(H)) / H for j in range(L)]
    t = Fraction(float(np.float32(tau)))
    if t == 0:
        return L
    best_p = 0
    for p in range(L):
        cp = min(sum((mean[j] for j in sub), Fraction(0)) for sub in itertools.combinations(range(L), p))
        if cp <= t:
            best_p = p
    return L - best_p


def pin_budget_bruteforce(O):
    r = _rng(21)
    for trial in range(12):
        B, H, L = 2, int(r.integers(1, 4)), int(r.integers(2, 9))
        s = _dyadic_scores(r, B, H, L)
        # tau grid: random values plus values hit exactly by some partial sum
        taus = [0.0, 0.01, 0.3, 0.999]
        m = s[0].mean(axis=0)
        srt = np.sort(m)
        taus += [float(srt[:p].sum()) for p in range(1, L)]
        for tau in taus:
            if not (0.0 <= float(np.float32(tau)) < 1.0):
                continue
            kb = O.coverage_budget(s, tau)
            for b in range(B):
                want = _bruteforce_budget(s[b], tau)
                assert int(kb[b]) == want, (trial, b, tau, kb, want)


def pin_budget_invariants(O):
    r = _rng(22)
    s = r.gamma(0.5, size=(2, 3, 200))
    s = s / s.sum(-1, keepdims=True)
    L = s.shape[-1]
    assert list(O.coverage_budget(s, 0.0)) == [L, L]
    prev = None
    for tau in np.linspace(0.0, 0.99, 23):
        kb = O.coverage_budget(s, tau)
        assert np.all((kb >= 1) & (kb <= L))
        if prev is not None:
            assert np.all(kb <= prev), (tau, kb, prev)
        prev = kb
    # C(P) <= tau < C(P+1) on the head-mean masses (float64 check, tau away from ties)
    tau = 0.37
    kb = O.coverage_budget(s, tau)
    for b in range(2):
        m = np.sort(s[b].mean(axis=0))
        P = L - int(kb[b])
        assert m[:P].sum() <= tau + 1e-12 and m[:P + 1].sum() > tau - 1e-12


# --------------------------------------------------------------------------- step 3: select
def _bruteforce_select(s_row, K):
    L = len(s_row)
    hits = []
    for sub in itertools.combinations(range(L), K):
        ss = set(sub)
        ok = all((s_row[i] > s_row[j]) or (s_row[i] == s_row[j] and i < j)
                 for i in ss for j in range(L) if j not in ss)
        if ok:
            hits.append(list(sub))
    assert len(hits) == 1
    return hits[0]


def pin_select_bruteforce(O):
    r = _rng(31)
    for trial in range(10):
        L = int(r.integers(1, 10))
        s_row = r.integers(0, 4, size=L).astype(np.float64) / 8.0   # many exact ties
        for K in range(1, L + 1):
            got = list(O.select_topk(s_row, K))
            assert got == _bruteforce_select(s_row, K), (s_row, K, got)


def pin_select_invariants(O):
    r = _rng(32)
    s = r.random((2, 3, 50))
    s[:, :, 10:20] = 0.25           # exact ties
    budget = np.array([17, 50], dtype=np.int32)
    idx, rank = O.select_heads(s, budget)
    for b in range(2):
        K = int(budget[b])
        for h in range(3):
            sel = idx[b, h, :K]
            assert np.all(np.diff(sel) > 0)
            assert np.all(idx[b, h, K:] == -1)
            assert np.array_equal(rank[b, h, sel], np.arange(K))
            assert np.sum(rank[b, h] >= 0) == K
            # nested: the top-(K-1) set is inside the top-K set
            small = set(O.select_topk(s[b, h], max(K - 1, 1)))
            assert small <= set(sel)


# --------------------------------------------------------------------------- step 5: attention
def pin_attention_sdpa(O):
    r = _rng(41)
    for (n, d) in [(1, 4), (7, 8), (300, 16), (513, 32)]:
        qc, kc, vc = (r.standard_normal((n, d)) for _ in range(3))
        got = O.causal_attention(qc, kc, vc)
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qc)[None], torch.from_numpy(kc)[None], torch.from_numpy(vc)[None],
            is_causal=True)[0].numpy()
        assert np.allclose(got, want, rtol=0, atol=1e-12), np.abs(got - want).max()
        rows = np.array([0, n - 1, n // 2])
        assert np.allclose(O.causal_attention(qc, kc, vc, rows=rows), want[rows], rtol=0, atol=1e-12)


def pin_attention_closed_forms(O):
    r = _rng(42)
    n, d = 40, 8
    kc, vc = r.standard_normal((n, d)), r.standard_normal((n, d))
    # Q = 0: uniform weights -> running mean of V
    got = O.causal_attention(np.zeros((n, d)), kc, vc)
    want = np.cumsum(vc, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.allclose(got, want, rtol=0, atol=1e-13)
    # constant V rows -> every output is that row
    row = r.standard_normal(d)
    got = O.causal_attention(r.standard_normal((n, d)), kc, np.tile(row, (n, 1)))
    assert np.allclose(got, np.tile(row, (n, 1)), rtol=0, atol=1e-13)
    # a single key: output is V_0
    got = O.causal_attention(r.standard_normal((1, d)), kc[:1], vc[:1])
    assert np.allclose(got, vc[:1], rtol=0, atol=0)


# --------------------------------------------------------------------------- whole op
def _sdpa_dense(q, k, v):
    Hq, Hkv = q.shape[1], k.shape[1]
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kt, vt, is_causal=True).numpy()


def pin_forward_tau0_dense(O):
    r = _rng(51)
    B, Hq, Hkv, L, d, w = 2, 6, 2, 33, 16, 5
    q, k, v = (r.standard_normal(sh) for sh in [(B, Hq, L, d), (B, Hkv, L, d), (B, Hkv, L, d)])
    out = O.forward(q, k, v, w, 0.0)
    assert list(out["budget"]) == [L] * B
    assert np.allclose(out["o"], _sdpa_dense(q, k, v), rtol=0, atol=1e-12)
    assert np.allclose(O.dense_causal_attention(q, k, v), _sdpa_dense(q, k, v), rtol=0, atol=1e-12)


def pin_forward_zero_rows_and_linearity(O):
    r = _rng(52)
    B, Hq, Hkv, L, d, w = 1, 4, 2, 64, 8, 8
    q, k, v = (r.standard_normal(sh) for sh in [(B, Hq, L, d), (B, Hkv, L, d), (B, Hkv, L, d)])
    k[0, 0, :5] += 4.0 * q[0, 0, -1] / np.linalg.norm(q[0, 0, -1])
    out = O.forward(q, k, v, w, 0.2)
    K = int(out["budget"][0])
    assert 1 <= K < L
    for h in range(Hq):
        sel = out["idx"][0, h, :K]
        mask = np.ones(L, bool)
        mask[sel] = False
        assert np.all(out["o"][0, h, mask] == 0.0)
        g = h // (Hq // Hkv)
        comp = O.causal_attention(q[0, h, sel], k[0, g, sel], v[0, g, sel])
        assert np.allclose(out["o"][0, h, sel], comp, rtol=0, atol=1e-13)
        # the selected set is this head's own top-K of its own scores
        assert list(sel) == sorted(np.lexsort((np.arange(L), -out["s"][0, h]))[:K])
    out2 = O.forward(q, k, 2.5 * v, w, 0.2)
    assert np.array_equal(out2["idx"], out["idx"])
    assert np.allclose(out2["o"], 2.5 * out["o"], rtol=1e-13, atol=1e-13)


def _bruteforce_forward(q, k, v, w, tau):
    """Tiny-input pipeline built from library routines and enumeration."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    s = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            for rr in range(L - w, L):
                x = (kt[b, h // G, : rr + 1] @ qt[b, h, rr]) / math.sqrt(d)
                s[b, h, : rr + 1] += torch.softmax(x, 0).numpy() / w
    o = np.zeros((B, Hq, L, d))
    budget = []
    for b in range(B):
        K = _bruteforce_budget(s[b], tau)
        budget.append(K)
        for h in range(Hq):
            sel = _bruteforce_select(list(s[b, h]), K)
            ot = torch.nn.functional.scaled_dot_product_attention(
                qt[b, h, sel][None], kt[b, h // G, sel][None], vt[b, h // G, sel][None],
                is_causal=True)[0].numpy()
            o[b, h, sel] = ot
    return s, budget, o


def pin_forward_bruteforce(O):
    r = _rng(53)
    for trial in range(6):
        B, Hkv, G = 1, int(r.integers(1, 3)), int(r.integers(1, 3))
        Hq, L, d = Hkv * G, int(r.integers(3, 8)), 2
        w = int(r.integers(1, L + 1))
        q, k, v = (r.standard_normal(sh) * 1.5 for sh in [(B, Hq, L, d), (B, Hkv, L, d), (B, Hkv, L, d)])
        for tau in (0.0, 0.15, 0.4):
            s_bf, kb_bf, o_bf = _bruteforce_forward(q, k, v, w, tau)
            out = O.forward(q, k, v, w, tau)
            assert np.allclose(out["s"], s_bf, rtol=0, atol=1e-13)
            assert list(out["budget"]) == kb_bf, (trial, tau, out["budget"], kb_bf)
            assert np.allclose(out["o"], o_bf, rtol=0, atol=1e-12), (trial, tau)


# --------------------------------------------------------------------------- alternative readings
def pin_worked_example_alternatives(O):
    ex, q, k, v = load_worked_example()
    alt = ex["alternatives"]
    s = O.proxy_scores(q, k, ex["w"], causal=False)
    want = np.array([_frac(x) for x in alt["noncausal_scores"]])
    assert np.allclose(s[0, 0], want, rtol=0, atol=1e-14), (s, want)
    for case in alt["noncausal_cases"]:
        out = O.forward(q, k, v, ex["w"], case["tau"], causal=False)
        assert int(out["budget"][0]) == case["budget"], (case, out["budget"])
        assert list(out["idx"][0, 0, :case["budget"]]) == case["idx"]
        want_o = np.array([_frac(x) for x in case["o"]])
        assert np.allclose(out["o"][0, 0, :, 0], want_o, rtol=0, atol=1e-13), (case, out["o"])
    for case in alt["keep_window_cases"]:
        out = O.forward(q, k, v, ex["w"], case["tau"], keep_window=True)
        assert int(out["budget"][0]) == case["budget"], (case, out["budget"])
        assert list(out["idx"][0, 0, :case["budget"]]) == case["idx"]
        want_o = np.array([_frac(x) for x in case["o"]])
        assert np.allclose(out["o"][0, 0, :, 0], want_o, rtol=0, atol=1e-13), (case, out["o"])
    # one head: the per-head budget is the global budget
    for case in ex["cases"]:
        out = O.forward(q, k, v, ex["w"], case["tau"], per_head=True)
        assert out["budget"].shape == (1, 1) and int(out["budget"][0, 0]) == case["budget"]


def pin_scores_noncausal(O):
    """Every proxy row sees all L keys: identical keys give s_j = 1/L exactly; otherwise
    s is the mean over the proxy rows of one library softmax over all keys."""
    r = _rng(15)
    for (L, w, d) in [(40, 8, 4), (12, 12, 2), (30, 1, 3)]:
        k = np.tile(r.standard_normal(d), (L, 1)).reshape(1, 1, L, d)
        q = r.standard_normal((1, 1, L, d)) * 3
        s = O.proxy_scores(q, k, w, causal=False)[0, 0]
        assert np.allclose(s, 1.0 / L, rtol=0, atol=1e-14), s
    B, Hq, Hkv, L, d, w = 2, 4, 2, 23, 8, 5
    q = r.standard_normal((B, Hq, L, d))
    k = r.standard_normal((B, Hkv, L, d))
    s = O.proxy_scores(q, k, w, causal=False)
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    logits = torch.matmul(torch.from_numpy(q[:, :, L - w:]), kt.transpose(-1, -2).contiguous()) / math.sqrt(d)
    want = torch.softmax(logits, dim=-1).mean(dim=2).numpy()
    assert np.allclose(s, want, rtol=0, atol=1e-14)
    # the causal reading differs (rows before the last see fewer keys) unless w = 1
    assert not np.allclose(s, O.proxy_scores(q, k, w))
    assert np.allclose(O.proxy_scores(q, k, 1, causal=False), O.proxy_scores(q, k, 1), rtol=0, atol=1e-15)


def _bruteforce_cut(masses, t, pmax):
    """max{p in [0, pmax] : min over p-subsets of the summed masses <= t} (exact fractions)."""
    n = len(masses)
    best = 0
    for p in range(min(pmax, n) + 1):
        cp = min(sum((masses[j] for j in sub), Fraction(0)) for sub in itertools.combinations(range(n), p))
        if cp <= t:
            best = p
    return best


def pin_budget_per_head_bruteforce(O):
    r = _rng(23)
    for trial in range(10):
        B, H, L = 2, int(r.integers(1, 4)), int(r.integers(2, 9))
        s = _dyadic_scores(r, B, H, L)
        taus = [0.0, 0.01, 0.3, 0.999] + [float(np.sort(s[0, 0])[:p].sum()) for p in range(1, L)]
        for tau in taus:
            if not (0.0 <= float(np.float32(tau)) < 1.0):
                continue
            t = Fraction(float(np.float32(tau)))
            kb = O.coverage_budget(s, tau, per_head=True)
            assert kb.shape == (B, H)
            for b in range(B):
                for h in range(H):
                    m = [Fraction(float(x)) for x in s[b, h]]
                    want = L if t == 0 else L - _bruteforce_cut(m, t, L - 1)
                    assert int(kb[b, h]) == want, (trial, b, h, tau, kb, want)
            if H == 1:    # one head: the per-head cut is the global cut
                assert np.array_equal(kb[:, 0], O.coverage_budget(s, tau))


def pin_budget_keep_window_bruteforce(O):
    r = _rng(24)
    for trial in range(10):
        B, H, L = 1, int(r.integers(1, 4)), int(r.integers(2, 9))
        keep = int(r.integers(1, L + 1))
        s = _dyadic_scores(r, B, H, L)
        for tau in [0.0, 0.05, 0.2, 0.5, 0.9]:
            t = Fraction(float(np.float32(tau)))
            mean = [sum(Fraction(float(s[0, h, j])) for h in range(H)) / H for j in range(L)]
            want = L if t == 0 else L - _bruteforce_cut(mean[:L - keep], t, L - keep)
            kb = O.coverage_budget(s, tau, keep=keep)
            assert int(kb[0]) == want, (trial, keep, tau, kb, want)
            assert int(kb[0]) >= keep
            kh = O.coverage_budget(s, tau, per_head=True, keep=keep)
            for h in range(H):
                m = [Fraction(float(x)) for x in s[0, h]]
                wh = L if t == 0 else L - _bruteforce_cut(m[:L - keep], t, L - keep)
                assert int(kh[0, h]) == wh, (trial, keep, tau, h, kh, wh)


def pin_select_keep_window(O):
    """With a kept window the set is the window plus the brute-force top of the rest."""
    r = _rng(33)
    for trial in range(8):
        L = int(r.integers(2, 10))
        keep = int(r.integers(1, L + 1))
        s = (r.integers(0, 4, size=(1, 2, L)).astype(np.float64) / 8.0)
        for K in range(keep, L + 1):
            budget = np.full((1, 2), K, dtype=np.int32)           # per-head shape
            idx, rank = O.select_heads(s, budget, keep=keep)
            for h in range(2):
                top = _bruteforce_select(list(s[0, h, :L - keep]), K - keep) if K > keep else []
                want = sorted(top) + list(range(L - keep, L))
                assert list(idx[0, h, :K]) == want, (trial, keep, K, h, idx[0, h])
                assert np.all(idx[0, h, K:] == -1)
                assert np.array_equal(rank[0, h, idx[0, h, :K]], np.arange(K))


def _bruteforce_forward_alt(q, k, v, w, tau, causal, per_head, keep_window):
    """Tiny-input pipeline for the alternative readings from library routines and enumeration."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    keep = w if keep_window else 0
    t = Fraction(float(np.float32(tau)))
    s = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            for rr in range(L - w, L):
                hi = L if not causal else rr + 1
                x = (kt[b, h // G, :hi] @ qt[b, h, rr]) / math.sqrt(d)
                s[b, h, :hi] += torch.softmax(x, 0).numpy() / w
    o = np.zeros((B, Hq, L, d))
    budgets = np.zeros((B, Hq), dtype=np.int64)
    for b in range(B):
        mean = [sum(Fraction(float(s[b, h, j])) for h in range(Hq)) / Hq for j in range(L)]
        pmax = min(L - keep, L - 1)
        Kg = L if t == 0 else L - _bruteforce_cut(mean[:L - keep], t, pmax)
        for h in range(Hq):
            if per_head:
                m = [Fraction(float(x)) for x in s[b, h]]
                K = L if t == 0 else L - _bruteforce_cut(m[:L - keep], t, pmax)
            else:
                K = Kg
            budgets[b, h] = K
            top = _bruteforce_select(list(s[b, h, :L - keep]), K - keep) if K > keep else []
            sel = sorted(top) + list(range(L - keep, L))
            ot = torch.nn.functional.scaled_dot_product_attention(
                qt[b, h, sel][None], kt[b, h // G, sel][None], vt[b, h // G, sel][None],
                is_causal=True)[0].numpy()
            o[b, h, sel] = ot
    return s, budgets, o


def pin_forward_alternatives_bruteforce(O):
    r = _rng(54)
    for trial in range(8):
        B, Hkv, G = 1, int(r.integers(1, 3)), int(r.integers(1, 3))
        Hq, L, d = Hkv * G, int(r.integers(3, 8)), 2
        w = int(r.integers(1, L + 1))
        q, k, v = (r.standard_normal(sh) * 1.5 for sh in [(B, Hq, L, d), (B, Hkv, L, d), (B, Hkv, L, d)])
        causal, per_head, keep_window = bool(trial & 1), bool(trial & 2), bool(trial & 4)
        for tau in (0.0, 0.15, 0.4):
            s_bf, kb_bf, o_bf = _bruteforce_forward_alt(q, k, v, w, tau, causal, per_head, keep_window)
            out = O.forward(q, k, v, w, tau, causal=causal, per_head=per_head, keep_window=keep_window)
            assert np.allclose(out["s"], s_bf, rtol=0, atol=1e-13)
            got_b = out["budget"] if per_head else np.repeat(out["budget"][:, None], Hq, axis=1)
            assert np.array_equal(got_b, kb_bf), (trial, tau, out["budget"], kb_bf)
            assert np.allclose(out["o"], o_bf, rtol=0, atol=1e-12), (trial, tau)


# --------------------------------------------------------------------------- block-sparse composition
def pin_block_sparse_closed_forms(O):
    """Q = 0 gives uniform weights: row i's output is the mean of V over exactly the
    keys it may see, which pins the mask rule (block indices, orientation, the
    always-visible diagonal block) independently of the softmax."""
    r = _rng(44)
    Bk = O.BLOCK
    n, d = 3 * Bk, 4
    kc, vc = r.standard_normal((n, d)), r.standard_normal((n, d))
    qz = np.zeros((n, d))
    bm = np.zeros((3, 3), bool)
    bm[2, 0] = True                                  # block 2 also sees block 0; nothing else
    got = O.block_sparse_attention(qz, kc, vc, bm)
    for i in range(n):
        ib = i // Bk
        keys = list(range(ib * Bk, i + 1))
        if ib == 2:
            keys = list(range(0, Bk)) + keys
        assert np.allclose(got[i], vc[keys].mean(axis=0), rtol=0, atol=1e-13), i
    # all-false: every block attends only within itself = per-block causal attention (library)
    qc = r.standard_normal((n + 17, d))
    kc2, vc2 = r.standard_normal((n + 17, d)), r.standard_normal((n + 17, d))
    got = O.block_sparse_attention(qc, kc2, vc2, np.zeros((4, 4), bool))
    for b0 in range(0, n + 17, Bk):
        sl = slice(b0, min(b0 + Bk, n + 17))
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qc[sl])[None], torch.from_numpy(kc2[sl])[None],
            torch.from_numpy(vc2[sl])[None], is_causal=True)[0].numpy()
        assert np.allclose(got[sl], want, rtol=0, atol=1e-12)
    # all-true: plain causal attention (library)
    got = O.block_sparse_attention(qc, kc2, vc2, np.ones((4, 4), bool))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qc)[None], torch.from_numpy(kc2)[None], torch.from_numpy(vc2)[None],
        is_causal=True)[0].numpy()
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    rows = np.array([0, 70, n + 16])
    assert np.allclose(O.block_sparse_attention(qc, kc2, vc2, np.ones((4, 4), bool), rows=rows),
                       want[rows], rtol=0, atol=1e-12)


def pin_block_mask_bits(O):
    """Word w of row qb holds key blocks 32w .. 32w+31, bit kb % 32 (least significant first)."""
    words = np.array([[0b101, 0], [1 << 31, 1], [0, 0]], dtype=np.uint32)   # nb = 35: 2 words per row
    m = O.unpack_block_mask(words, 35)
    assert m.shape == (3, 35)
    assert list(np.nonzero(m[0])[0]) == [0, 2]
    assert list(np.nonzero(m[1])[0]) == [31, 32]
    assert not m[2].any()


ALL_PINS = [
    pin_worked_example,
    pin_scores_mass,
    pin_scores_identical_keys,
    pin_scores_w1_softmax,
    pin_scores_proxy_window,
    pin_budget_bruteforce,
    pin_budget_invariants,
    pin_select_bruteforce,
    pin_select_invariants,
    pin_attention_sdpa,
    pin_attention_closed_forms,
    pin_forward_tau0_dense,
    pin_forward_zero_rows_and_linearity,
    pin_forward_bruteforce,
    pin_worked_example_alternatives,
    pin_scores_noncausal,
    pin_budget_per_head_bruteforce,
    pin_budget_keep_window_bruteforce,
    pin_select_keep_window,
    pin_forward_alternatives_bruteforce,
    pin_block_sparse_closed_forms,
    pin_block_mask_bits,
]

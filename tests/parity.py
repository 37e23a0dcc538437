"""Helpers for comparing the HIP path with the fp64 oracle (test infrastructure).

Comparison rules:
  * budgets, index sets, rank maps, gathered and scattered rows: bit-exact;
  * scores: |s_gpu - s_ref| <= 1e-5 * s_ref + 1e-12 elementwise;
  * outputs, bf16: per (b, h) over the rows that are produced,
    max|O_gpu - O_ref| <= 2e-2 * max|O_ref|; f32: max-abs 1e-4;
  * end to end, a budget or set difference is accepted only as a near-tie:
    - set: every token in S_gpu xor S_ref has an oracle score within
      1e-6 * theta of theta, the oracle's K-th largest score of that head;
    - budget: |C_ref(p) - tau| <= 1e-6 * tau for every p between the two cuts.
    Near-ties are counted and reported, never silently accepted.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import tsa_oracle as O

BF16_REL = 2e-2
F32_ABS = 1e-4
SCORE_REL = 1e-5
SCORE_ABS = 1e-12
NEAR_TIE = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)
    return t.to("cuda").contiguous()


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def assert_scores_close(s_gpu: np.ndarray, s_ref: np.ndarray, what=""):
    err = np.abs(s_gpu - s_ref)
    bad = err > SCORE_REL * s_ref + SCORE_ABS
    rel = np.max(err / np.maximum(s_ref, 1e-30))
    say(f"[scores{what}] max rel err {rel:.3e}, bad {int(bad.sum())}")
    assert not bad.any(), f"score mismatch at {np.argwhere(bad)[:5]}"
    return rel


def assert_outputs_close(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, rows=None, what="",
                         quiet=False):
    """o_*: [B,H,n,d] (or [n,d] per head); compare per head."""
    if o_gpu.ndim == 2:
        o_gpu, o_ref = o_gpu[None, None], o_ref[None, None]
    worst = 0.0
    for b in range(o_gpu.shape[0]):
        for h in range(o_gpu.shape[1]):
            g, r = o_gpu[b, h], o_ref[b, h]
            if rows is not None:
                g, r = g[rows[b][h]], r[rows[b][h]]
            if g.size == 0:
                continue
            err = np.max(np.abs(g - r))
            if dtype == "bf16":
                scale = max(np.max(np.abs(r)), 1e-30)
                worst = max(worst, err / scale)
                assert err <= BF16_REL * scale, f"{what} b={b} h={h}: err {err:.3e} > {BF16_REL}*{scale:.3e}"
            else:
                worst = max(worst, err)
                assert err <= F32_ABS, f"{what} b={b} h={h}: max-abs err {err:.3e}"
    if not quiet:
        say(f"[outputs{what}] worst {'rel' if dtype == 'bf16' else 'abs'} err {worst:.3e}")
    return worst


def set_near_tie(s_ref_row: np.ndarray, sel_gpu, sel_ref, K: int) -> bool:
    """K: the number of tokens chosen by score among ``s_ref_row`` (the candidates)."""
    if K <= 0:
        return set(map(int, sel_gpu)) == set(map(int, sel_ref))
    theta = np.sort(s_ref_row)[::-1][K - 1]
    diff = set(map(int, sel_gpu)) ^ set(map(int, sel_ref))
    return all(abs(s_ref_row[j] - theta) <= NEAR_TIE * theta for j in diff)


def budget_near_tie(s_ref_b: np.ndarray, tau: float, K_gpu: int, K_ref: int, keep: int = 0) -> bool:
    """s_ref_b: the [H, L] scores of one budget row (all heads of a sequence, or one head)."""
    Hq, L = s_ref_b.shape
    sig = O.head_sum_masses(s_ref_b[None])[0][:L - keep]
    c = O.pruned_mass_curve(sig)
    scale = float(Hq) * float(2 ** O.SCORE_FRAC_BITS)
    p_lo, p_hi = sorted((L - K_gpu, L - K_ref))
    return all(abs(c[p] / scale - tau) <= NEAR_TIE * tau for p in range(p_lo, p_hi + 2)
               if p < len(c))


def _oracle_set(s_row: np.ndarray, K: int, keep: int) -> np.ndarray:
    L = s_row.shape[0]
    top = O.select_topk(s_row[:L - keep], K - keep) if K > keep else np.zeros(0, np.int32)
    return np.concatenate([top, np.arange(L - keep, L)]).astype(np.int32)


def compare_forward(ref: dict, o_gpu: np.ndarray, budget_gpu: np.ndarray, idx_gpu: np.ndarray,
                    q, k, v, tau: float, dtype: str, sample_rows: int = 0, seed: int = 0,
                    per_head: bool = False, keep: int = 0, block_heads=(), block_rows: int = 256):
    """End-to-end comparison.  ``ref`` is the oracle's forward() dict (with "o"
    present unless sample_rows > 0, in which case outputs are recomputed for
    sampled rows only).  per_head / keep: the alternative readings (budgets
    [B,Hq]; the last ``keep`` positions always kept).  block_heads: (b, h)
    pairs for which, on top of the sampled rows, one random compact row of
    every block of ``block_rows`` rows (one attention workgroup) is checked.
    Returns a report dict with near-tie counts."""
    B, Hq, L = idx_gpu.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    rep = {"budget_near_ties": 0, "set_near_ties": 0, "heads": B * Hq, "worst_err": 0.0}
    rng = np.random.default_rng(seed)
    for b in range(B):
        if not per_head:
            Kg, Kr = int(budget_gpu[b]), int(ref["budget"][b])
            if Kg != Kr:
                assert budget_near_tie(ref["s"][b], tau, Kg, Kr, keep), \
                    f"budget mismatch b={b}: {Kg} vs {Kr}"
                rep["budget_near_ties"] += 1
        for h in range(Hq):
            if per_head:
                Kg, Kr = int(budget_gpu[b, h]), int(ref["budget"][b, h])
                if Kg != Kr:
                    assert budget_near_tie(ref["s"][b, h][None], tau, Kg, Kr, keep), \
                        f"budget mismatch b={b} h={h}: {Kg} vs {Kr}"
                    rep["budget_near_ties"] += 1
            assert Kg >= keep
            g = h // G
            sel_g = idx_gpu[b, h, :Kg]
            assert np.all(np.diff(sel_g) > 0) and np.all(idx_gpu[b, h, Kg:] == -1)
            assert np.array_equal(sel_g[Kg - keep:], np.arange(L - keep, L))
            sel_r = ref["idx"][b, h, :Kr]
            same = Kg == Kr and np.array_equal(sel_g, sel_r)
            if not same:
                # the GPU set must be the oracle's set of size Kg up to near-ties
                top_r = _oracle_set(ref["s"][b, h], Kg, keep)
                if not np.array_equal(sel_g, top_r):
                    assert set_near_tie(ref["s"][b, h, :L - keep], sel_g, top_r, Kg - keep), \
                        f"set mismatch b={b} h={h}"
                rep["set_near_ties"] += 1
            # unselected rows are exactly +0.0
            mask = np.ones(L, bool)
            mask[sel_g] = False
            assert np.all(o_gpu[b, h, mask] == 0.0)
            if sample_rows:
                rows = np.unique(np.concatenate([[0, Kg - 1], rng.integers(0, Kg, sample_rows)]))
                if (b, h) in block_heads:
                    starts = np.arange(0, Kg, block_rows)
                    ends = np.minimum(starts + block_rows, Kg)
                    rows = np.unique(np.concatenate([rows, rng.integers(starts, ends)]))
                    rep["block_rows_checked"] = rep.get("block_rows_checked", 0) + len(starts)
            else:
                rows = np.arange(Kg)
            if same and not sample_rows:
                want = ref["o"][b, h, sel_g[rows]]
            else:
                # outputs of the GPU's (valid) set, recomputed for the chosen rows
                want = O.causal_attention(q[b, h, sel_g], k[b, g, sel_g], v[b, g, sel_g], rows=rows)
            got = o_gpu[b, h, sel_g[rows]]
            err = assert_outputs_close(got[None, None], want[None, None], dtype, what=f" b={b} h={h}",
                                       quiet=True)
            rep["worst_err"] = max(rep["worst_err"], err)
    say(f"[forward] near-ties: budget {rep['budget_near_ties']}, sets {rep['set_near_ties']} "
        f"of {rep['heads']} heads; worst output err {rep['worst_err']:.3e}"
        + (f"; {rep['block_rows_checked']} per-block rows" if "block_rows_checked" in rep else ""))
    return rep


def check_rows_written(o: torch.Tensor, idx: torch.Tensor, budget: torch.Tensor, per_head=False):
    """On the device, for an output that was filled with NaN before the call: every selected
    row is finite (some workgroup wrote it) and every unselected row holds +0.0 bits."""
    B, Hq, L, _ = o.shape
    pos = torch.arange(L, device=o.device)
    kb = budget.view(B, Hq if per_head else 1).expand(B, Hq).to(torch.int64)
    valid = pos[None, None, :] < kb[..., None]
    # entries past the budget go to a sentinel column L, dropped afterwards
    src = torch.where(valid, idx.to(torch.int64), torch.full_like(idx, L, dtype=torch.int64))
    sel = torch.zeros((B, Hq, L + 1), dtype=torch.bool, device=o.device)
    sel.scatter_(2, src, torch.ones_like(valid))
    sel = sel[..., :L]
    bits = o.view(torch.int16 if o.dtype == torch.bfloat16 else torch.int32)
    n_bad_sel = int((~torch.isfinite(o.float()).all(dim=-1) & sel).sum())
    n_bad_zero = int(((bits != 0).any(dim=-1) & ~sel).sum())
    say(f"[rows written] {int(sel.sum())} selected rows finite: {n_bad_sel == 0}; "
        f"{int((~sel).sum())} unselected rows +0.0: {n_bad_zero == 0}")
    assert n_bad_sel == 0, f"{n_bad_sel} selected rows were not written"
    assert n_bad_zero == 0, f"{n_bad_zero} unselected rows are not +0.0"

"""Planted mistakes in copies of the oracle must each fail at least one pin.

This shows the pins are strong enough: a dropped term, a wrong sign, an
off-by-one mask, a wrong head map or tie rule in the oracle would not go
unnoticed.  Every mutant lives in a private copy of the module on the CPU.
"""
import importlib.util
import math
import os

import numpy as np
import pytest

from tests.oracle_pins import ALL_PINS

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "tsa_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("tsa_oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _scores_variant(mask="causal", divide_w=True, scale=True, head_map="div", window="last"):
    def proxy_scores(q, k, w, causal=True):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        B, Hq, L, d = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        rows = np.arange(L - w, L) if window == "last" else np.arange(w)
        cols = np.arange(L)
        if not causal:
            vis = np.ones((len(rows), L), bool)
        elif mask == "causal":
            vis = cols[None, :] <= rows[:, None]
        elif mask == "strict":
            vis = (cols[None, :] < rows[:, None]) | (cols[None, :] == 0)
        else:
            vis = np.ones((len(rows), L), bool)
        s = np.zeros((B, Hq, L))
        for b in range(B):
            for h in range(Hq):
                g = h // G if head_map == "div" else h % Hkv
                x = q[b, h, rows] @ k[b, g].T
                if scale:
                    x = x / math.sqrt(d)
                x = np.where(vis, x, -np.inf)
                p = np.exp(x - x.max(1, keepdims=True))
                p /= p.sum(1, keepdims=True)
                s[b, h] = p.sum(0) / (w if divide_w else 1)
        return s
    return proxy_scores


def m_no_causal(O):
    O.proxy_scores = _scores_variant(mask="none")


def m_strict_causal(O):
    O.proxy_scores = _scores_variant(mask="strict")


def m_no_divide_w(O):
    O.proxy_scores = _scores_variant(divide_w=False)


def m_no_scale(O):
    O.proxy_scores = _scores_variant(scale=False)


def m_head_mod(O):
    O.proxy_scores = _scores_variant(head_map="mod")


def m_first_rows(O):
    O.proxy_scores = _scores_variant(window="first")


def m_budget_strict(O):
    orig_thr = O.tau_threshold
    O.tau_threshold = lambda tau, Hq: orig_thr(tau, Hq) - 1     # C(p) < tau instead of <=


def m_budget_prune_crossing(O):
    orig = O.coverage_budget

    def cb(s, tau, **kw):
        kb = orig(s, tau, **kw)
        return np.maximum(kb - (1 if float(np.float32(tau)) > 0 else 0), 1).astype(np.int32)
    O.coverage_budget = cb


def m_budget_descending(O):
    def curve(sig):
        srt = sorted((int(x) for x in sig), reverse=True)
        c = [0]
        for x in srt:
            c.append(c[-1] + x)
        return c
    O.pruned_mass_curve = curve


def m_budget_max_head(O):
    def hs(s):
        qm = O.quantised_masses(s)
        return qm.astype(object).max(axis=1) * qm.shape[1]
    O.head_sum_masses = hs


def m_budget_no_tau0(O):
    orig = O.coverage_budget

    def cb(s, tau, **kw):
        s = np.asarray(s, np.float64)
        if float(np.float32(tau)) == 0.0 and not kw.get("per_head") and not kw.get("keep"):
            sig = O.head_sum_masses(s)
            out = []
            for b in range(s.shape[0]):
                c = O.pruned_mass_curve(sig[b])
                p = max(pp for pp in range(s.shape[2]) if c[pp] <= 0)
                out.append(s.shape[2] - p)
            return np.array(out, dtype=np.int32)
        return orig(s, tau, **kw)
    O.coverage_budget = cb


def m_select_high_index_ties(O):
    def sel(s_row, K):
        s_row = np.asarray(s_row, np.float64)
        L = s_row.shape[0]
        order = np.lexsort((-np.arange(L), -s_row))
        return np.sort(order[:K]).astype(np.int32)
    O.select_topk = sel


def m_select_unsorted(O):
    def sel(s_row, K):
        s_row = np.asarray(s_row, np.float64)
        L = s_row.shape[0]
        return np.lexsort((np.arange(L), -s_row))[:K].astype(np.int32)
    O.select_topk = sel


def m_select_ascending_scores(O):
    def sel(s_row, K):
        s_row = np.asarray(s_row, np.float64)
        L = s_row.shape[0]
        return np.sort(np.lexsort((np.arange(L), s_row))[:K]).astype(np.int32)
    O.select_topk = sel


def _attn_variant(kind):
    def causal_attention(qc, kc, vc, rows=None, block=256):
        qc, kc, vc = (np.asarray(x, np.float64) for x in (qc, kc, vc))
        n, d = qc.shape
        rows = np.arange(n) if rows is None else np.asarray(rows)
        x = qc[rows] @ kc.T / math.sqrt(d)
        j = np.arange(n)[None, :]
        i = rows[:, None]
        if kind == "nomask":
            vis = np.ones_like(x, bool)
        elif kind == "strict":
            vis = (j < i) | (j == 0)
        else:
            vis = j <= i
        x = np.where(vis, x, -np.inf)
        p = np.exp(x - x.max(1, keepdims=True))
        return (p @ vc) / p.sum(1, keepdims=True)
    return causal_attention


def m_attn_nomask(O):
    O.causal_attention = _attn_variant("nomask")


def m_attn_strict(O):
    O.causal_attention = _attn_variant("strict")


def m_gather_wrong_kv(O):
    def gather(q, k, v, idx, budget):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        B, Hq, L, d = q.shape
        Hkv = k.shape[1]
        qc, kc, vc = (np.zeros((B, Hq, L, d)) for _ in range(3))
        for b in range(B):
            K = int(budget[b])
            for h in range(Hq):
                g = h % Hkv
                sel = idx[b, h, :K]
                qc[b, h, :K], kc[b, h, :K], vc[b, h, :K] = q[b, h, sel], k[b, g, sel], v[b, g, sel]
        return qc, kc, vc
    O.gather = gather


def m_scatter_compact(O):
    def scatter(oc, idx, budget):
        oc = np.asarray(oc, np.float64)
        o = np.zeros_like(oc)
        for b in range(oc.shape[0]):
            K = int(budget[b])
            o[b, :, :K] = oc[b, :, :K]
        return o
    O.scatter = scatter


def m_noncausal_ignored(O):
    orig = O.proxy_scores
    O.proxy_scores = lambda q, k, w, causal=True: orig(q, k, w)


def m_per_head_head_count_threshold(O):
    orig_thr = O.tau_threshold
    orig_cb = O.coverage_budget

    def cb(s, tau, per_head=False, keep=0):
        if not per_head:
            return orig_cb(s, tau, per_head=per_head, keep=keep)
        H = np.asarray(s).shape[1]
        O.tau_threshold = lambda t, Hq: orig_thr(t, H)       # threshold of the head sum
        try:
            return orig_cb(s, tau, per_head=True, keep=keep)
        finally:
            O.tau_threshold = orig_thr
    O.coverage_budget = cb


def m_keep_ignored_in_budget(O):
    orig = O.coverage_budget
    O.coverage_budget = lambda s, tau, per_head=False, keep=0: orig(s, tau, per_head=per_head, keep=0)


def m_keep_window_at_start(O):
    def select_heads(s, budget, keep=0):
        s = np.asarray(s, np.float64)
        B, H, L = s.shape
        idx = np.full((B, H, L), -1, dtype=np.int32)
        rank = np.full((B, H, L), -1, dtype=np.int32)
        for b in range(B):
            for h in range(H):
                K = O.head_budget(budget, b, h)
                rest = O.select_topk(s[b, h, keep:], K - keep) + keep
                sel = np.sort(np.concatenate([np.arange(keep), rest])).astype(np.int32)
                idx[b, h, :K] = sel
                rank[b, h, sel] = np.arange(K, dtype=np.int32)
        return idx, rank
    O.select_heads = select_heads


def _bsa_variant(kind):
    def block_sparse_attention(qc, kc, vc, block_mask, rows=None):
        qc, kc, vc = (np.asarray(x, np.float64) for x in (qc, kc, vc))
        n, d = qc.shape
        bm = np.asarray(block_mask, bool)
        Bk = O_BLOCK
        rows = np.arange(n) if rows is None else np.asarray(rows)
        out = np.empty((len(rows), d))
        for a, i in enumerate(rows):
            j = np.arange(i + 1)
            if kind == "transposed":
                vis = (j // Bk == i // Bk) | bm[j // Bk, i // Bk]
            elif kind == "no_diagonal":
                vis = bm[i // Bk, j // Bk] | (j == i)
            else:                                     # block index off by one row
                vis = (j // Bk == i // Bk) | bm[(i + 1) // Bk % bm.shape[0], j // Bk]
            x = kc[j[vis]] @ qc[i] / math.sqrt(d)
            p = np.exp(x - x.max())
            out[a] = p @ vc[j[vis]] / p.sum()
        return out
    return block_sparse_attention


O_BLOCK = 64


def m_bsa_transposed(O):
    O.block_sparse_attention = _bsa_variant("transposed")


def m_bsa_no_diagonal(O):
    O.block_sparse_attention = _bsa_variant("no_diagonal")


def m_bsa_off_by_one(O):
    O.block_sparse_attention = _bsa_variant("off_by_one")


def m_mask_bits_msb_first(O):
    def unpack(words, nb):
        words = np.asarray(words, dtype=np.uint64)
        kb = np.arange(nb)
        return ((words[:, kb // 32] >> (31 - kb % 32).astype(np.uint64)) & 1).astype(bool)
    O.unpack_block_mask = unpack


MUTANTS = [m_no_causal, m_strict_causal, m_no_divide_w, m_no_scale, m_head_mod, m_first_rows,
           m_budget_strict, m_budget_prune_crossing, m_budget_descending, m_budget_max_head,
           m_budget_no_tau0, m_select_high_index_ties, m_select_unsorted,
           m_select_ascending_scores, m_attn_nomask, m_attn_strict, m_gather_wrong_kv,
           m_scatter_compact, m_noncausal_ignored, m_per_head_head_count_threshold,
           m_keep_ignored_in_budget, m_keep_window_at_start, m_bsa_transposed, m_bsa_no_diagonal,
           m_bsa_off_by_one, m_mask_bits_msb_first]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_mutant_is_caught(mutant):
    O = fresh_oracle()
    mutant(O)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches {mutant.__name__}"

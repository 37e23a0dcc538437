"""Plain fp64 CPU oracle for the Token Sparse Attention prefill op.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code, header, table or constant with it.

Source: "Token Sparse Attention: Efficient Long-Context Inference with
Interleaved Token Selection" (Jo, Kang, Song, Kim, 2026).  The only page with
method detail is the gist.science structured summary (page in Spanish),
section 2 "Methodology", whose sub-sections are cited below as:

  [Compression]     section 2, "Core architecture", stage 1 (QKV selection)
  [Decompression]   section 2, "Core architecture", stage 2 (output restore)
  [Scoring]         section 2, "Dynamic Token Coverage", scoring bullet
  [Budget]          section 2, "Dynamic Token Coverage", budget bullet
  [Per-head]        section 2, "Dynamic Token Coverage", per-head selection bullet

Everything is float64 NumPy with no blocking or reordering beyond what the
steps state (query rows of the attention are processed in blocks only so that
no K x K buffer is ever held; each row's arithmetic is unchanged).

Readings taken where the pages are silent (each is also listed in the
design notes of the repository):
  * proxy queries are the last ``w`` positions; each proxy row is causal
    (row r sees keys j <= r); logits are scaled by 1/sqrt(d); one plain
    softmax per proxy row;
  * "summing vertically" is the column sum over the w proxy rows divided by
    w, so each head's importance sums to 1;
  * the global budget of a sequence uses the mean over all query heads of
    the per-head importance; the pruned mass C(p) of the p least important
    tokens is compared with tau and the token whose pruning would push it
    above tau is kept: P = max{p in [0, L-1] : C(p) <= tau}, K = L - P, and
    tau = 0 prunes nothing;
  * masses are exact sums of scores truncated to multiples of 2^-50
    (``SCORE_FRAC_BITS``), compared with the float32 value of tau exactly;
  * per-head top-K orders tokens by (score descending, index ascending) and
    stores the chosen indices in ascending order;
  * query head h reads K/V rows of KV head h // (Hq/Hkv) at its own indices;
  * each batch element is an independent sequence with its own budget.

Alternative readings (ablations), each a keyword argument defaulting to the
main reading above:
  * ``causal=False`` in proxy_scores: every proxy row sees all L keys;
  * ``per_head=True`` in coverage_budget: each head cuts its own importance
    curve against tau, giving one budget K_h per (b, h) (a [B,Hq] array);
  * ``keep=w`` in coverage_budget and select_heads: the last ``keep``
    positions (the proxy window) are never pruned; only tokens before them
    are candidates for pruning, and every head's set is its top-(K - keep)
    candidates plus the window.
Every function that takes a budget accepts either shape: [B] (one budget per
sequence) or [B,Hq] (one per head).

Composition with block-sparse attention on the compressed tensors (the pages
name it as compatible, without fixing a format): ``block_sparse_attention``
restricts the causal attention of the compact rows to the (query block, key
block) pairs a caller marks visible, in blocks of ``BLOCK`` = 64 compact rows;
the diagonal block of every query block is always visible, so no row is left
without keys.

Pins (tests/test_oracle_pins.py) tie every function to closed forms, library
routines, brute force and a hand-derived worked example.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

SCORE_FRAC_BITS = 50   # importance masses are counted in units of 2^-50
BLOCK = 64             # rows per block of the block-sparse composition


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    return h // (Hq // Hkv)


def head_budget(budget, b: int, h: int) -> int:
    """K of head (b, h) from a [B] (per sequence) or [B,Hq] (per head) budget."""
    budget = np.asarray(budget)
    return int(budget[b, h]) if budget.ndim == 2 else int(budget[b])


# ---------------------------------------------------------------------------
# Step 1 [Scoring]: proxy attention of the last w queries against all keys,
# softmax per row, column sums (divided by w) give per-token importance.
# ---------------------------------------------------------------------------
def proxy_scores(q, k, w: int, causal: bool = True) -> np.ndarray:
    """Per-head token importance s[b,h,j] in float64.

    q: [B,Hq,L,d]; k: [B,Hkv,L,d]; returns [B,Hq,L] with each row summing to 1.
    causal=False: every proxy row sees all L keys (alternative reading).
    """
    q = _f64(q)
    k = _f64(k)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    assert 1 <= w <= L and Hq % Hkv == 0
    rows = np.arange(L - w, L)
    cols = np.arange(L)
    visible = (cols[None, :] <= rows[:, None]) if causal else np.ones((w, L), dtype=bool)
    s = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            x = (q[b, h, L - w:] @ k[b, g].T) / math.sqrt(d)
            x = np.where(visible, x, -np.inf)
            x = x - x.max(axis=1, keepdims=True)
            p = np.exp(x)
            p = p / p.sum(axis=1, keepdims=True)
            s[b, h] = p.sum(axis=0) / w
    return s


# ---------------------------------------------------------------------------
# Step 2 [Budget]: Dynamic Token Coverage.  Sort the (head-mean) importance
# ascending and prune the tail while the pruned mass stays within tau.
# ---------------------------------------------------------------------------
def quantised_masses(s) -> np.ndarray:
    """Importance in integer units of 2^-SCORE_FRAC_BITS: floor(clip(s,0,1) * 2^F).

    Values are clipped to [0, 1] (NaN counts as 0).  Returns int64 [B,H,L].
    """
    s = np.nan_to_num(_f64(s), nan=0.0, posinf=1.0, neginf=0.0)
    s = np.clip(s, 0.0, 1.0)
    return np.floor(np.ldexp(s, SCORE_FRAC_BITS)).astype(np.int64)


def head_sum_masses(s) -> np.ndarray:
    """sigma[b,j] = sum over query heads of the quantised importance (exact ints)."""
    qm = quantised_masses(s)
    return qm.astype(object).sum(axis=1)


def tau_threshold(tau: float, Hq: int) -> int:
    """floor(Hq * tau * 2^F) for the float32 value of tau, in exact arithmetic."""
    t = Fraction(float(np.float32(tau)))
    return math.floor(t * Hq * (1 << SCORE_FRAC_BITS))


def pruned_mass_curve(sigma_b) -> list:
    """C(p) for p = 0..L: exact sum of the p smallest head-summed masses."""
    srt = sorted(int(x) for x in sigma_b)
    c = [0]
    for x in srt:
        c.append(c[-1] + x)
    return c


def _cut(masses, thr: int, pmax: int) -> int:
    """P = max{p in [0, pmax] : C(p) <= thr}, C(p) = exact sum of the p smallest masses."""
    c = pruned_mass_curve(masses)
    p = 0
    for pp in range(pmax + 1):       # C is non-decreasing: take the largest p with C(p) <= thr
        if c[pp] <= thr:
            p = pp
        else:
            break
    return p


def coverage_budget(s, tau: float, per_head: bool = False, keep: int = 0) -> np.ndarray:
    """Budget K = L - P: int32 [B] (one per sequence) or, with per_head, [B,Hq].

    Main reading: P_b = max{p in [0, L-1] : C(p) <= tau} with C measured as the
    head-mean pruned mass; tau = 0 gives P_b = 0.
    per_head: each head's own importance curve is cut against tau.
    keep: the last ``keep`` positions are never pruned; candidates are the
    first L - keep tokens and P = max{p in [0, min(L - keep, L - 1)] : C(p) <= tau}.
    """
    s = _f64(s)
    B, Hq, L = s.shape
    assert 0 <= keep <= L
    tau32 = float(np.float32(tau))
    assert 0.0 <= tau32 < 1.0
    ncand = L - keep
    pmax = min(ncand, L - 1)
    out = np.zeros((B, Hq) if per_head else B, dtype=np.int32)
    if tau32 == 0.0:
        out[...] = L
        return out
    if per_head:
        thr = tau_threshold(tau32, 1)
        qm = quantised_masses(s)
        for b in range(B):
            for h in range(Hq):
                out[b, h] = L - _cut(qm[b, h, :ncand], thr, pmax)
        return out
    thr = tau_threshold(tau32, Hq)
    sig = head_sum_masses(s)
    for b in range(B):
        out[b] = L - _cut(sig[b][:ncand], thr, pmax)
    return out


# ---------------------------------------------------------------------------
# Step 3 [Per-head]: each head independently keeps its own top-K.
# ---------------------------------------------------------------------------
def select_topk(s_row, K: int):
    """Ascending indices of the K best tokens under (score desc, index asc)."""
    s_row = _f64(s_row)
    L = s_row.shape[0]
    order = np.lexsort((np.arange(L), -s_row))   # primary key: -score; then index
    return np.sort(order[:K]).astype(np.int32)


def select_heads(s, budget, keep: int = 0):
    """idx [B,H,L] (ascending set then -1) and rank [B,H,L] (slot or -1).

    keep: the last ``keep`` positions are always in the set; the other K - keep
    come from the first L - keep tokens by (score desc, index asc).
    """
    s = _f64(s)
    B, H, L = s.shape
    idx = np.full((B, H, L), -1, dtype=np.int32)
    rank = np.full((B, H, L), -1, dtype=np.int32)
    window = np.arange(L - keep, L, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            K = head_budget(budget, b, h)
            assert keep <= K <= L
            sel = np.concatenate([select_topk(s[b, h, :L - keep], K - keep), window])
            idx[b, h, :K] = sel
            rank[b, h, sel] = np.arange(K, dtype=np.int32)
    return idx, rank


# ---------------------------------------------------------------------------
# Step 4 [Compression]: gather Q, K, V rows of each head's set into dense
# compressed tensors of length K (query head h reads its KV head's rows).
# ---------------------------------------------------------------------------
def gather(q, k, v, idx, budget):
    """Compact Qc, Kc, Vc of shape [B,Hq,L,d]; rows >= K_b are left zero."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    qc = np.zeros((B, Hq, L, d))
    kc = np.zeros((B, Hq, L, d))
    vc = np.zeros((B, Hq, L, d))
    for b in range(B):
        for h in range(Hq):
            K = head_budget(budget, b, h)
            g = _kv_head(h, Hq, Hkv)
            sel = idx[b, h, :K]
            qc[b, h, :K] = q[b, h, sel]
            kc[b, h, :K] = k[b, g, sel]
            vc[b, h, :K] = v[b, g, sel]
    return qc, kc, vc


# ---------------------------------------------------------------------------
# Step 5 [Compression]: ordinary causal attention on the compressed tensors.
# With ascending indices the compact causal mask equals the original one
# restricted to the selected tokens.
# ---------------------------------------------------------------------------
def causal_attention(qc, kc, vc, rows=None, block: int = 256) -> np.ndarray:
    """O_i = sum_{j<=i} softmax_j(Qc_i . Kc_j / sqrt(d)) Vc_j for one head.

    qc, kc, vc: [n, d].  ``rows``: optional subset of output rows to compute
    (returned in that order); default is all n rows.
    """
    qc, kc, vc = _f64(qc), _f64(kc), _f64(vc)
    n, d = qc.shape
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], d))
    scale = 1.0 / math.sqrt(d)
    for a in range(0, rows.shape[0], block):
        rr = rows[a:a + block]
        hi = int(rr.max()) + 1
        x = (qc[rr] @ kc[:hi].T) * scale
        x = np.where(np.arange(hi)[None, :] <= rr[:, None], x, -np.inf)
        x = x - x.max(axis=1, keepdims=True)
        p = np.exp(x)
        out[a:a + block] = (p @ vc[:hi]) / p.sum(axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------------------
# Composition [Compression]: block-sparse attention on the compressed tensors.
# ---------------------------------------------------------------------------
def block_sparse_attention(qc, kc, vc, block_mask, rows=None) -> np.ndarray:
    """O_i = sum over visible j of softmax_j(Qc_i . Kc_j / sqrt(d)) Vc_j for one head.

    Key j is visible to row i when j <= i and either i and j lie in the same
    block of BLOCK rows or block_mask[i // BLOCK, j // BLOCK] is true.
    block_mask: bool array with at least ceil(n / BLOCK) rows and columns.
    """
    qc, kc, vc = _f64(qc), _f64(kc), _f64(vc)
    n, d = qc.shape
    bm = np.asarray(block_mask, dtype=bool)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], d))
    scale = 1.0 / math.sqrt(d)
    for a, i in enumerate(rows):
        j = np.arange(i + 1)
        vis = (j // BLOCK == i // BLOCK) | bm[i // BLOCK, j // BLOCK]
        x = (kc[j[vis]] @ qc[i]) * scale
        p = np.exp(x - x.max())
        out[a] = (p @ vc[j[vis]]) / p.sum()
    return out


def unpack_block_mask(words, nb: int) -> np.ndarray:
    """[nb, ceil(nb/32)] uint32 words -> [nb, nb] bool: bit kb % 32 of word kb // 32."""
    words = np.asarray(words, dtype=np.uint64)
    kb = np.arange(nb)
    return ((words[:, kb // 32] >> (kb % 32).astype(np.uint64)) & 1).astype(bool)


def attention_heads(qc, kc, vc, budget) -> np.ndarray:
    """Causal attention per (b, h) over the first K_b compact rows; [B,H,L,d]."""
    qc = _f64(qc)
    B, H, L, d = qc.shape
    oc = np.zeros((B, H, L, d))
    for b in range(B):
        for h in range(H):
            K = head_budget(budget, b, h)
            oc[b, h, :K] = causal_attention(qc[b, h, :K], kc[b, h, :K], vc[b, h, :K])
    return oc


def dense_causal_attention(q, k, v) -> np.ndarray:
    """Causal attention over all L rows with the GQA head map (the dense baseline)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    o = np.zeros((B, Hq, L, d))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            o[b, h] = causal_attention(q[b, h], k[b, g], v[b, g])
    return o


# ---------------------------------------------------------------------------
# Step 6 [Decompression]: scatter the compact output back into a zero L x d
# tensor at the head's indices; unselected rows stay zero.
# ---------------------------------------------------------------------------
def scatter(oc, idx, budget) -> np.ndarray:
    oc = _f64(oc)
    B, H, L, d = oc.shape
    o = np.zeros((B, H, L, d))
    for b in range(B):
        for h in range(H):
            K = head_budget(budget, b, h)
            o[b, h, idx[b, h, :K]] = oc[b, h, :K]
    return o


# ---------------------------------------------------------------------------
# The whole op: score -> budget -> per-head top-K -> gather -> attention -> scatter.
# ---------------------------------------------------------------------------
def forward(q, k, v, w: int, tau: float, causal: bool = True, per_head: bool = False,
            keep_window: bool = False) -> dict:
    """The main reading by default; the keyword flags select the alternative
    readings (keep_window keeps the w proxy positions)."""
    keep = w if keep_window else 0
    s = proxy_scores(q, k, w, causal=causal)
    budget = coverage_budget(s, tau, per_head=per_head, keep=keep)
    idx, rank = select_heads(s, budget, keep=keep)
    qc, kc, vc = gather(q, k, v, idx, budget)
    oc = attention_heads(qc, kc, vc, budget)
    o = scatter(oc, idx, budget)
    return {"s": s, "budget": budget, "idx": idx, "rank": rank, "o": o}

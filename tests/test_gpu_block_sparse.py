"""Block-sparse attention on the compressed tensors (GPU) against the fp64 oracle.

The caller's mask marks (64-row query block, 64-key block) pairs visible;
diagonal blocks always are.  The kernel skips every other tile, and must
match the oracle's block_sparse_attention within the output tolerance; an
all-visible mask reproduces tsa_attention bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import tsa_oracle as O
from tests.parity import assert_outputs_close, say, to_dev, to_np
from token_sparse_attention_proxy_amd import inputs
from token_sparse_attention_proxy_amd import tsa as T

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _mask_dev(m):
    return torch.from_numpy(m.view(np.int32)).cuda()


def _oracle(qc, kc, vc, m, budgets, rows=None):
    """Per-head oracle over the first K_b compact rows; returns [B,H,L,d] (or rows only)."""
    B, H, L, d = qc.shape
    nb = (L + 63) // 64
    out = np.zeros((B, H, L, d))
    for b in range(B):
        n = L if budgets is None else int(budgets[b])
        for h in range(H):
            bm = O.unpack_block_mask(m[b, h], nb)
            g = h // (H // kc.shape[1])
            out[b, h, :n] = O.block_sparse_attention(qc[b, h, :n], kc[b, g, :n], vc[b, g, :n], bm)
    return out


CASES = [
    # dtype, B, Hq, Hk, L, d, budgets (None = all rows), kv_group, pattern, density
    ("bf16", 1, 4, 4, 1000, 128, [1000], 1, "random", 0.5),
    ("bf16", 2, 4, 4, 777, 128, [777, 300], 1, "random", 0.3),
    ("bf16", 1, 8, 2, 1000, 128, None, 4, "vertical_slash", 0.0),
    ("bf16", 1, 3, 3, 1500, 64, [1337], 1, "random", 0.2),
    ("bf16", 1, 2, 2, 700, 128, [700], 1, "none", 0.0),
    ("bf16", 1, 2, 2, 129, 128, [65], 1, "random", 0.5),
    ("f32", 1, 4, 4, 1000, 64, [900], 1, "random", 0.4),
    ("f32", 1, 4, 2, 300, 128, None, 2, "vertical_slash", 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_block_sparse_matches_oracle(case):
    dt, B, Hq, Hk, L, d, budgets, G, pattern, dens = case
    say(f"case block-sparse {case}")
    q = inputs.make_dense((B, Hq, L, d), 71, dt)
    k = inputs.make_dense((B, Hk, L, d), 72, dt, scale=1.5)
    v = inputs.make_dense((B, Hk, L, d), 73, dt)
    m = inputs.make_block_mask(B, Hq, L, seed=74, pattern=pattern, density=dens, band=2, columns=3)
    prob = T.Problem(B, Hq, Hq // G, L, d, 1, 0.05, dt)
    bd = None if budgets is None else torch.tensor(budgets, dtype=torch.int32, device="cuda")
    o = torch.full((B, Hq, L, d), float("nan"), dtype=torch.bfloat16 if dt == "bf16" else torch.float32,
                   device="cuda")
    T.tsa_attention_block_sparse(prob, to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), _mask_dev(m), bd, G, o)
    got = to_np(o)
    ref = _oracle(q, k, v, m, budgets)
    for b in range(B):
        n = L if budgets is None else budgets[b]
        assert np.isnan(got[b, :, n:]).all()          # rows past the budget are not written
        assert_outputs_close(got[b:b + 1, :, :n], ref[b:b + 1, :, :n], dt, what=f" {pattern} b={b}")


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_all_visible_equals_dense_kernel(dt, d):
    """Every bit set: the same tiles in the same order as tsa_attention, bit for bit."""
    B, H, L = 1, 4, 1100
    say(f"case block-sparse all-visible {dt} d={d}")
    q, k, v = (to_dev(inputs.make_dense((B, H, L, d), s, dt), dt) for s in (81, 82, 83))
    prob = T.Problem(B, H, H, L, d, 1, 0.05, dt)
    m = inputs.make_block_mask(B, H, L, seed=84, pattern="all")
    bd = torch.tensor([1000], dtype=torch.int32, device="cuda")
    a = T.tsa_attention_block_sparse(prob, q, k, v, _mask_dev(m), bd, 1)
    b = T.tsa_attention(prob, q, k, v, bd, 1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(a[:, :, :1000]), _bits(b[:, :, :1000]))


def test_block_sparse_recompute_path():
    """A large late logit in a visible block forces the exact-max recompute; the
    second pass must walk the same tiles."""
    say("case block-sparse recompute")
    B, H, L, d = 1, 2, 900, 128
    rng = np.random.default_rng(77)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d))
    v = rng.standard_normal((B, H, L, d))
    q[:, :, 700:] += 10.0 * u
    k[:, :, 700] = 80.0 * u
    qb, kb_, vb = (to_dev(x.astype(np.float32), "bf16") for x in (q, k, v))
    q, k, v = (to_np(x) for x in (qb, kb_, vb))
    m = inputs.make_block_mask(B, H, L, seed=78, pattern="random", density=0.5)
    prob = T.Problem(B, H, H, L, d, 1, 0.05, "bf16")
    o = to_np(T.tsa_attention_block_sparse(prob, qb, kb_, vb, _mask_dev(m), None, 1))
    ref = _oracle(q, k, v, m, None)
    assert_outputs_close(o, ref, "bf16", what=" recompute")


def test_tsa_then_block_sparse_end_to_end():
    """The composition: score -> budget -> select -> gather -> block-sparse attention
    on the compressed tensors -> scatter, against the oracle on the GPU's own sets."""
    wl = inputs.small_workload("bf16", B=1, Hq=8, Hkv=2, L=2000, d=128, w=64, tau=0.1,
                               seed_base=9700)
    say("case tsa + block-sparse")
    q, k, v = inputs.make_qkv(wl)
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, 0.1, "bf16")
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    s = T.tsa_score(prob, qd, kd)
    bud = T.tsa_budget(prob, s)
    idx, rank = T.tsa_select(prob, s, bud)
    qc, kc, vc = T.tsa_gather(prob, qd, kd, vd, idx, bud)
    m = inputs.make_block_mask(wl.B, wl.Hq, wl.L, seed=79, pattern="vertical_slash", band=3,
                               columns=4)
    oc = T.tsa_attention_block_sparse(prob, qc, kc, vc, _mask_dev(m), bud, 1)
    o = to_np(T.tsa_scatter(prob, oc, rank))
    K = int(to_np(bud)[0])
    idx_np = to_np(idx)
    ref_s = O.proxy_scores(q, k, wl.w)
    assert K == int(O.coverage_budget(ref_s, 0.1)[0])
    nb = (wl.L + 63) // 64
    for h in range(wl.Hq):
        sel = idx_np[0, h, :K]
        g = h // wl.G
        want = O.block_sparse_attention(q[0, h, sel], k[0, g, sel], v[0, g, sel],
                                        O.unpack_block_mask(m[0, h], nb))
        assert_outputs_close(o[0, h, sel], want, "bf16", what=f" h={h}", quiet=True)
        rest = np.ones(wl.L, bool)
        rest[sel] = False
        assert np.all(o[0, h, rest] == 0.0)


@pytest.mark.parametrize("pattern,dens", [("random", 0.3), ("vertical_slash", 0.0)])
def test_block_sparse_full_size(pattern, dens):
    """The compact 128K shape (K = 123997 rows of 32 heads), sampled rows."""
    B, H, L, d, K = 1, 32, 131072, 128, 123997
    say(f"case block-sparse full {pattern}")
    g = torch.Generator(device="cuda").manual_seed(5)
    q, k, v = (torch.randn((B, H, L, d), device="cuda", generator=g).to(torch.bfloat16)
               for _ in range(3))
    m = inputs.make_block_mask(B, H, L, seed=91, pattern=pattern, density=dens, band=16,
                               columns=32)
    prob = T.Problem(B, H, H, L, d, 64, 0.05, "bf16")
    bd = torch.tensor([K], dtype=torch.int32, device="cuda")
    o = T.tsa_attention_block_sparse(prob, q, k, v, _mask_dev(m), bd, 1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(92)
    nb = (L + 63) // 64
    for h in (0, 17, 31):
        rows = np.unique(np.concatenate([[0, 63, 64, K - 1], rng.integers(0, K, 4)]))
        qh, kh, vh = (to_np(x[0, h, :K]) for x in (q, k, v))
        want = O.block_sparse_attention(qh, kh, vh, O.unpack_block_mask(m[0, h], nb), rows=rows)
        got = to_np(o[0, h, rows])
        assert_outputs_close(got, want, "bf16", what=f" full h={h}")

"""Seeded synthetic inputs for Token Sparse Attention.

This module only draws random tensors.  It holds none of the method's
arithmetic (no scoring, budgeting, selection or attention): both the fp64
CPU oracle and the HIP path read what it produces.

The shapes follow the long-context prefill workloads of "Token Sparse
Attention: Efficient Long-Context Inference with Interleaved Token Selection"
(gist.science summary, section 4: LLaMA-3.1-8B / Mistral-Nemo-12B class
attention layers at up to 128K context).  The datasets used there (RULER,
InfiniteBench, Needle-in-a-Haystack) are not available; these generators
stand in for them and reproduce none of their items.

Recipe (all draws from ``numpy.random.default_rng(seed)``, in this order):

1. Q ~ N(0,1) of shape [B,Hq,L,d], then K, then V ~ N(0,1) of shape
   [B,Hkv,L,d], all float32.
2. u = a unit vector drawn as N(0, I_d) / ||.||, once per draw.
3. Planted heavy keys: for each (b, kv head) in order, a subset of
   round(frac*L) positions from ``rng.choice(L, n, replace=False)``; those key
   rows get ``+amp*u``.  ``plant="shared"`` draws one subset per b used by every
   KV head; ``plant="per_head"`` draws one per (b, kv head);
   ``plant="half"`` leaves the first half of the KV heads unplanted.
4. Zipf key-norm bias (``zipf_s > 0``): for each (b, kv head) a rank
   permutation r = rng.permutation(L)+1 and K[b,g,j] *= sqrt(1 + 2 s ln(L/r_j)).
   For q ~ N(0, I) the expected proxy weight of key j then scales as r_j^-s,
   and the permutation differs per KV head so heads disagree.
5. Cast to the storage dtype (bf16 round-to-nearest-even via torch), or kept
   float32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32" or "bf16": the storage / arithmetic type
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    w: int
    taus: tuple
    plant: str = "per_head"   # "shared" | "per_head" | "half" | "none"
    plant_frac: float = 0.05
    plant_amp: float = 3.0
    zipf_s: float = 0.0
    seed_base: int = 0

    def seed(self, rep: int = 0) -> int:
        return self.seed_base + rep

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# The five workloads: tiny MHA correctness case, Llama-3-8B-shaped layer at
# 8K, the 32K tau sweep with Zipf-skewed heads, the 128K headline layer, and
# the wide-GQA B=2 stress case; and a sixth, the 32K recipe (Zipf-skewed
# heads) at the headline's 128K length, for the speedup at long context when
# importance is concentrated.
WORKLOADS = {
    "tiny_mha_f32_L1k": Workload("tiny_mha_f32_L1k", "f32", 1, 4, 4, 1024, 64, 16, (0.05,),
                                 plant="shared", plant_frac=0.05, plant_amp=3.0, seed_base=1000),
    "llama8b_bf16_L8k": Workload("llama8b_bf16_L8k", "bf16", 1, 32, 8, 8192, 128, 64, (0.05,),
                                 plant="per_head", plant_frac=0.05, plant_amp=3.0, seed_base=2000),
    "llama8b_bf16_L32k_zipf": Workload("llama8b_bf16_L32k_zipf", "bf16", 1, 32, 8, 32768, 128, 64,
                                       (0.01, 0.05, 0.1), plant="none", zipf_s=1.1,
                                       seed_base=3000),
    "llama8b_bf16_L128k": Workload("llama8b_bf16_L128k", "bf16", 1, 32, 8, 131072, 128, 64, (0.05,),
                                   plant="per_head", plant_frac=0.05, plant_amp=3.0,
                                   seed_base=4000),
    "gqa7_bf16_B2_L64k": Workload("gqa7_bf16_B2_L64k", "bf16", 2, 28, 4, 65536, 128, 128, (0.1,),
                                  plant="half", plant_frac=0.01, plant_amp=5.0, seed_base=5000),
    "llama8b_bf16_L128k_zipf": Workload("llama8b_bf16_L128k_zipf", "bf16", 1, 32, 8, 131072, 128,
                                        64, (0.05, 0.1, 0.2), plant="none", zipf_s=1.1,
                                        seed_base=6000),
}

HEADLINE = "llama8b_bf16_L128k"


def small_workload(dtype="bf16", B=1, Hq=8, Hkv=2, L=1000, d=128, w=64, tau=0.05,
                   plant="per_head", plant_frac=0.05, plant_amp=3.0, zipf_s=0.0,
                   seed_base=9000, name=None) -> Workload:
    """A reduced-size workload with the same recipe, for oracle-sized tests."""
    return Workload(name or f"small_{dtype}_B{B}_H{Hq}x{Hkv}_L{L}_d{d}_w{w}", dtype, B, Hq, Hkv, L,
                    d, w, (tau,), plant=plant, plant_frac=plant_frac, plant_amp=plant_amp,
                    zipf_s=zipf_s, seed_base=seed_base)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 data to the storage dtype; returns float32 holding exact values."""
    if dtype == "f32":
        return x
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.to(torch.float32).numpy()


def make_qkv(wl: Workload, rep: int = 0):
    """Draw (Q, K, V) as float32 numpy arrays holding storage-dtype values.

    For bf16 workloads every element is exactly a bf16 value, so upcasting to
    float64 (oracle) or reinterpreting as bf16 (device) is lossless.
    """
    rng = np.random.default_rng(wl.seed(rep))
    B, Hq, Hkv, L, d = wl.B, wl.Hq, wl.Hkv, wl.L, wl.d
    q = rng.standard_normal((B, Hq, L, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, L, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, L, d), dtype=np.float32)
    u = rng.standard_normal(d).astype(np.float64)
    u = (u / np.linalg.norm(u)).astype(np.float32)
    n_plant = int(round(wl.plant_frac * L))
    if wl.plant != "none" and n_plant > 0:
        for b in range(B):
            shared = rng.choice(L, n_plant, replace=False) if wl.plant == "shared" else None
            for g in range(Hkv):
                if wl.plant == "shared":
                    sub = shared
                elif wl.plant == "half" and g < Hkv // 2:
                    continue
                else:
                    sub = rng.choice(L, n_plant, replace=False)
                k[b, g, sub, :] += np.float32(wl.plant_amp) * u
    if wl.zipf_s > 0:
        for b in range(B):
            for g in range(Hkv):
                r = rng.permutation(L).astype(np.float64) + 1.0
                scale = np.sqrt(1.0 + 2.0 * wl.zipf_s * np.log(L / r)).astype(np.float32)
                k[b, g] *= scale[:, None]
    return _to_storage(q, wl.dtype), _to_storage(k, wl.dtype), _to_storage(v, wl.dtype)


def make_scores(B: int, H: int, L: int, seed: int, ties: bool = False,
                zero_frac: float = 0.0, alpha: float = 1.0) -> np.ndarray:
    """Random per-head probability rows [B,H,L] as float32 (each row sums to ~1).

    ``ties=True`` draws values from a small set of dyadic levels so that many
    scores are exactly equal; ``zero_frac`` zeroes a random fraction of entries.
    Used to drive the budget and selection entry points with controlled inputs.
    """
    rng = np.random.default_rng(seed)
    if ties:
        levels = rng.integers(1, 9, size=(B, H, L)).astype(np.float64)
        x = levels
    else:
        x = rng.gamma(alpha, size=(B, H, L))
    if zero_frac > 0:
        x = np.where(rng.random((B, H, L)) < zero_frac, 0.0, x)
    tot = x.sum(axis=-1, keepdims=True)
    tot[tot == 0] = 1.0
    if ties:
        # keep the levels dyadic: scale by a power of two so the sum stays <= 1
        p2 = 2.0 ** np.ceil(np.log2(tot))
        x = x / p2
    else:
        x = x / tot
    return x.astype(np.float32)


def make_indices(B: int, H: int, L: int, budget: np.ndarray, seed: int):
    """Random ascending index sets of size budget[b] per (b, h), plus the rank map.

    Returns (idx, rank) int32 arrays [B,H,L]: idx holds the set in ascending
    order then -1; rank[j] is the slot of j in the set or -1.  These are
    inputs for the gather and scatter entry points.
    """
    rng = np.random.default_rng(seed)
    idx = np.full((B, H, L), -1, dtype=np.int32)
    rank = np.full((B, H, L), -1, dtype=np.int32)
    for b in range(B):
        kb = int(budget[b])
        for h in range(H):
            sel = np.sort(rng.choice(L, kb, replace=False)).astype(np.int32)
            idx[b, h, :kb] = sel
            rank[b, h, sel] = np.arange(kb, dtype=np.int32)
    return idx, rank


def make_dense(shape, seed: int, dtype: str = "bf16", scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) tensor in the storage dtype (float32 array holding exact values)."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))
    return _to_storage(x, dtype)


def make_block_mask(B: int, H: int, L: int, seed: int, pattern: str = "random",
                    density: float = 0.5, band: int = 4, columns: int = 8) -> np.ndarray:
    """A seeded block mask for the block-sparse composition, packed as the library
    takes it: uint32 [B,H,NB,NW] with NB = ceil(L/64), NW = ceil(NB/32); bit
    kb % 32 of word [b,h,qb,kb // 32] marks key block kb visible to query block qb.

    Patterns (only blocks below the diagonal are drawn; the rest is left 0):
      "random":         each block visible with probability ``density``;
      "vertical_slash": the ``band`` blocks just below the diagonal plus
                        ``columns`` key-block columns drawn per (b, h), the
                        shape of the sparse prefill patterns the compressed
                        tensors are combined with;
      "none" / "all":   no block / every block.
    """
    rng = np.random.default_rng(seed)
    nb = (L + 63) // 64
    nw = (nb + 31) // 32
    vis = np.zeros((B, H, nb, nb), dtype=bool)
    below = np.tril(np.ones((nb, nb), dtype=bool), k=-1)
    for b in range(B):
        for h in range(H):
            if pattern == "random":
                m = rng.random((nb, nb)) < density
            elif pattern == "vertical_slash":
                m = np.zeros((nb, nb), dtype=bool)
                for off in range(1, band + 1):
                    m |= np.eye(nb, k=-off, dtype=bool)
                cols = rng.choice(nb, size=min(columns, nb), replace=False)
                m[:, cols] = True
            elif pattern == "all":
                m = np.ones((nb, nb), dtype=bool)
            elif pattern == "none":
                m = np.zeros((nb, nb), dtype=bool)
            else:
                raise ValueError(pattern)
            vis[b, h] = m & below
    words = np.zeros((B, H, nb, nw), dtype=np.uint64)
    for kb in range(nb):
        words[..., kb // 32] |= vis[..., kb].astype(np.uint64) << np.uint64(kb % 32)
    return words.astype(np.uint32)

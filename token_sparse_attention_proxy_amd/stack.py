"""A synthetic multi-layer stack that re-runs token selection in every layer.

The method keeps no token evicted for good: every sparse layer scores and
selects again on its own Q, K, V, and the output goes back into the residual
stream at full length (gist.science summary, section 2, "Core architecture",
stage 2, and section 3, contribution 1, reversible token-level sparsity).
This module shows that re-selection across layers with random weights: it
makes no accuracy claim and uses no trained model.

Layer l: q, k, v = x W_q, x W_k, x W_v (heads split, no positional
encoding), o = TSA(q, k, v), x <- x + o W_o.  The projections are plain
library GEMMs (torch.matmul on the device); the attention of every layer
is this library's op.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

from . import tsa as T


@dataclasses.dataclass
class StackConfig:
    B: int
    L: int
    Hq: int
    Hkv: int
    d: int
    layers: int
    w: int
    tau: float
    flags: int = 0
    fused: bool = False

    @property
    def model_dim(self) -> int:
        return self.Hq * self.d


def make_weights(cfg: StackConfig, seed: int, device) -> List[dict]:
    """Random bf16 projection weights, N(0, 1/D) so activations keep unit scale."""
    g = torch.Generator(device=device).manual_seed(seed)
    D = cfg.model_dim
    out = []
    for _ in range(cfg.layers):
        def mat(n_in, n_out):
            return (torch.randn((n_in, n_out), generator=g, device=device) / math.sqrt(n_in)).to(torch.bfloat16)
        out.append({"wq": mat(D, cfg.Hq * cfg.d), "wk": mat(D, cfg.Hkv * cfg.d),
                    "wv": mat(D, cfg.Hkv * cfg.d), "wo": mat(cfg.Hq * cfg.d, D)})
    return out


def _heads(t: torch.Tensor, B: int, L: int, H: int, d: int) -> torch.Tensor:
    return t.view(B, L, H, d).transpose(1, 2).contiguous()


def layer_qkv(cfg: StackConfig, x: torch.Tensor, wt: dict):
    """q [B,Hq,L,d], k, v [B,Hkv,L,d] (bf16, contiguous) from the residual stream x [B,L,D]."""
    B, L = cfg.B, cfg.L
    q = _heads(torch.matmul(x, wt["wq"]), B, L, cfg.Hq, cfg.d)
    k = _heads(torch.matmul(x, wt["wk"]), B, L, cfg.Hkv, cfg.d)
    v = _heads(torch.matmul(x, wt["wv"]), B, L, cfg.Hkv, cfg.d)
    return q, k, v


def run_stack(cfg: StackConfig, x: torch.Tensor, weights: List[dict], dense: bool = False,
              keep: Optional[list] = None):
    """Run the stack on x [B,L,D] bf16.  Returns (x_out, per-layer records).

    Each record holds the layer's budget and index set (on the device) unless
    ``dense``, in which case the attention is the dense causal kernel.
    ``keep``: optional list that receives each layer's (q, k, v) for checks; the
    records then also hold each layer's attention output "o".
    """
    prob = T.Problem(cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, cfg.w, cfg.tau, "bf16", cfg.flags)
    recs = []
    for wt in weights:
        q, k, v = layer_qkv(cfg, x, wt)
        if keep is not None:
            keep.append((q, k, v))
        if dense:
            o = T.tsa_attention(prob, q, k, v, None, cfg.Hq // cfg.Hkv)
            recs.append({})
        else:
            fwd = T.tsa_forward_fused if cfg.fused else T.tsa_forward
            o, budget, idx = fwd(prob, q, k, v)
            recs.append({"budget": budget, "idx": idx})
            if keep is not None:
                recs[-1]["o"] = o
        x = x + torch.matmul(o.transpose(1, 2).reshape(cfg.B, cfg.L, cfg.model_dim), wt["wo"])
    return x, recs


def reselection(cfg: StackConfig, recs: List[dict]) -> List[dict]:
    """Per pair of consecutive layers: mean Jaccard overlap of each head's index set,
    and the fraction of tokens pruned in one layer that the next layer keeps."""
    out = []
    for a, b in zip(recs[:-1], recs[1:]):
        ja, back = [], []
        ba, bb = a["budget"].cpu(), b["budget"].cpu()
        ia, ib = a["idx"].cpu(), b["idx"].cpu()
        for bi in range(cfg.B):
            for h in range(cfg.Hq):
                ka = int(ba[bi, h] if ba.dim() == 2 else ba[bi])
                kb = int(bb[bi, h] if bb.dim() == 2 else bb[bi])
                sa = torch.zeros(cfg.L, dtype=torch.bool)
                sb = torch.zeros(cfg.L, dtype=torch.bool)
                sa[ia[bi, h, :ka].long()] = True
                sb[ib[bi, h, :kb].long()] = True
                inter = int((sa & sb).sum())
                union = int((sa | sb).sum())
                ja.append(inter / max(union, 1))
                pruned = ~sa
                if int(pruned.sum()):
                    back.append(int((pruned & sb).sum()) / int(pruned.sum()))
        out.append({"jaccard": sum(ja) / len(ja),
                    "pruned_then_kept": (sum(back) / len(back)) if back else None})
    return out

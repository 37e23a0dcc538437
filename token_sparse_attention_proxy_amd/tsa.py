"""Python binding of libtsa.so with the same entry-point names as include/tsa.h.

PyTorch provides device memory and the stream handle; the wrappers only
allocate outputs, pass raw pointers and check the status code.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import (TSA_BF16, TSA_F32, TSA_FLAG_KEEP_WINDOW, TSA_FLAG_NONCAUSAL_PROXY,
                   TSA_FLAG_PER_HEAD_BUDGET, TsaError, TsaProblem, check)

_DTYPES = {"f32": (TSA_F32, torch.float32), "bf16": (TSA_BF16, torch.bfloat16)}


@dataclasses.dataclass(frozen=True)
class Problem:
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    w: int
    tau: float
    dtype: str = "bf16"          # "f32" or "bf16"
    flags: int = 0               # TSA_FLAG_* bits (alternative readings)

    @classmethod
    def from_qkv(cls, q: torch.Tensor, k: torch.Tensor, w: int, tau: float,
                 flags: int = 0) -> "Problem":
        B, Hq, L, d = q.shape
        dt = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(q.dtype)
        if dt is None:
            raise TypeError(f"unsupported dtype {q.dtype}")
        return cls(B, Hq, k.shape[1], L, d, w, float(tau), dt, int(flags))

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype][1]

    def c(self) -> TsaProblem:
        code = _DTYPES[self.dtype][0] if self.dtype in _DTYPES else 99
        return TsaProblem(self.B, self.Hq, self.Hkv, self.L, self.d, self.w, self.tau, code,
                          self.flags)

    @property
    def budget_shape(self) -> tuple:
        """[B], or [B,Hq] with per-head budgets."""
        return (self.B, self.Hq) if self.flags & TSA_FLAG_PER_HEAD_BUDGET else (self.B,)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live in device memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _expect(name: str, t: Optional[torch.Tensor], shape: tuple, dtype: torch.dtype) -> None:
    """Raise ValueError unless t has exactly this shape and dtype (the kernels read and write
    whole tensors of the size the problem implies, so a smaller one would be overrun)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected shape {tuple(shape)} and dtype {dtype}, "
                         f"got {tuple(t.shape)} and {t.dtype}")


def _heads(prob: "Problem", n_heads: int) -> tuple:
    return (prob.B, n_heads, prob.L, prob.d)


def _check_qkv(prob: "Problem", q, k, v, kv_heads: int) -> None:
    dt = prob.torch_dtype
    _expect("q", q, _heads(prob, prob.Hq), dt)
    _expect("k", k, _heads(prob, kv_heads), dt)
    _expect("v", v, _heads(prob, kv_heads), dt)


def _check_rows(prob: "Problem", **tensors) -> None:
    """[B,Hq,L] int32 index and rank maps."""
    for name, t in tensors.items():
        _expect(name, t, (prob.B, prob.Hq, prob.L), torch.int32)


def _check_budget(prob: "Problem", budget, optional: bool = False) -> None:
    if budget is None and optional:
        return
    _expect("budget", budget, prob.budget_shape, torch.int32)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _empty(shape, dtype, like: torch.Tensor) -> torch.Tensor:
    return torch.empty(shape, dtype=dtype, device=like.device)


def workspace_bytes(prob: Problem) -> int:
    return int(_lib.load().tsa_workspace_bytes(ctypes.byref(prob.c())))


def forward_workspace_bytes(prob: Problem) -> int:
    return int(_lib.load().tsa_forward_workspace_bytes(ctypes.byref(prob.c())))


def fused_workspace_bytes(prob: Problem) -> int:
    return int(_lib.load().tsa_fused_workspace_bytes(ctypes.byref(prob.c())))


def _ws(prob: Problem, like: torch.Tensor, ws: Optional[torch.Tensor], nbytes: int) -> torch.Tensor:
    if ws is None:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=like.device)
    elif ws.dtype != torch.uint8:
        raise ValueError(f"ws must be a uint8 byte buffer, got {ws.dtype}")
    return ws


def tsa_score(prob: Problem, q, k, s=None, ws=None):
    lib = _lib.load()
    p = prob.c()
    if s is None:
        s = _empty((prob.B, prob.Hq, prob.L), torch.float32, q)
    _expect("q", q, _heads(prob, prob.Hq), prob.torch_dtype)
    _expect("k", k, _heads(prob, prob.Hkv), prob.torch_dtype)
    _expect("s", s, (prob.B, prob.Hq, prob.L), torch.float32)
    ws = _ws(prob, q, ws, workspace_bytes(prob))
    check(lib.tsa_score(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(s), _ptr(ws), ws.numel(),
                        _stream(q.device)), "tsa_score")
    return s


def tsa_budget(prob: Problem, s, budget=None, ws=None):
    lib = _lib.load()
    p = prob.c()
    if budget is None:
        budget = _empty(prob.budget_shape, torch.int32, s)
    _expect("s", s, (prob.B, prob.Hq, prob.L), torch.float32)
    _check_budget(prob, budget)
    ws = _ws(prob, s, ws, workspace_bytes(prob))
    check(lib.tsa_budget(ctypes.byref(p), _ptr(s), _ptr(budget), _ptr(ws), ws.numel(),
                         _stream(s.device)), "tsa_budget")
    return budget


def tsa_select(prob: Problem, s, budget, idx=None, rank=None, ws=None):
    lib = _lib.load()
    p = prob.c()
    shape = (prob.B, prob.Hq, prob.L)
    idx = _empty(shape, torch.int32, s) if idx is None else idx
    rank = _empty(shape, torch.int32, s) if rank is None else rank
    _expect("s", s, shape, torch.float32)
    _check_budget(prob, budget)
    _check_rows(prob, idx=idx, rank=rank)
    ws = _ws(prob, s, ws, workspace_bytes(prob))
    check(lib.tsa_select(ctypes.byref(p), _ptr(s), _ptr(budget), _ptr(idx), _ptr(rank), _ptr(ws),
                         ws.numel(), _stream(s.device)), "tsa_select")
    return idx, rank


def tsa_gather(prob: Problem, q, k, v, idx, budget, qc=None, kc=None, vc=None, with_q=True):
    """with_q=False gathers K and V only and returns (None, kc, vc)."""
    lib = _lib.load()
    p = prob.c()
    shape = (prob.B, prob.Hq, prob.L, prob.d)
    if with_q:
        qc = _empty(shape, q.dtype, q) if qc is None else qc
    kc = _empty(shape, q.dtype, q) if kc is None else kc
    vc = _empty(shape, q.dtype, q) if vc is None else vc
    _check_qkv(prob, q, k, v, prob.Hkv)
    _check_rows(prob, idx=idx)
    _check_budget(prob, budget)
    if with_q:
        _expect("qc", qc, shape, prob.torch_dtype)
    _expect("kc", kc, shape, prob.torch_dtype)
    _expect("vc", vc, shape, prob.torch_dtype)
    check(lib.tsa_gather(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(budget),
                         _ptr(qc) if with_q else None, _ptr(kc), _ptr(vc), _stream(q.device)),
          "tsa_gather")
    return (qc if with_q else None), kc, vc


def tsa_gather_kv(prob: Problem, k, v, rank, kc=None, vc=None):
    """K and V only, source-driven through the rank map (tsa_forward's gather)."""
    lib = _lib.load()
    p = prob.c()
    shape = _heads(prob, prob.Hq)
    kc = _empty(shape, k.dtype, k) if kc is None else kc
    vc = _empty(shape, k.dtype, k) if vc is None else vc
    _expect("k", k, _heads(prob, prob.Hkv), prob.torch_dtype)
    _expect("v", v, _heads(prob, prob.Hkv), prob.torch_dtype)
    _check_rows(prob, rank=rank)
    _expect("kc", kc, shape, prob.torch_dtype)
    _expect("vc", vc, shape, prob.torch_dtype)
    check(lib.tsa_gather_kv(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(rank), _ptr(kc), _ptr(vc),
                            _stream(k.device)), "tsa_gather_kv")
    return kc, vc


def tsa_attention(prob: Problem, q, k, v, budget=None, kv_group: int = 1, o=None):
    lib = _lib.load()
    p = prob.c()
    if kv_group < 1 or prob.Hq % kv_group:
        raise ValueError(f"kv_group={kv_group} must divide Hq={prob.Hq}")
    o = _empty(q.shape, q.dtype, q) if o is None else o
    _check_qkv(prob, q, k, v, prob.Hq // kv_group)
    _expect("o", o, _heads(prob, prob.Hq), prob.torch_dtype)
    _check_budget(prob, budget, optional=True)
    check(lib.tsa_attention(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(budget), kv_group,
                            _ptr(o), _stream(q.device)), "tsa_attention")
    return o


def block_mask_words(prob: Problem) -> int:
    return int(_lib.load().tsa_block_mask_words(ctypes.byref(prob.c())))


def tsa_attention_block_sparse(prob: Problem, q, k, v, block_mask, budget=None, kv_group: int = 1,
                               o=None):
    """block_mask: int32/uint32-valued tensor of block_mask_words(prob) words
    ([B,Hq,NB,NW]), bit kb % 32 of word [b,h,qb,kb // 32]."""
    lib = _lib.load()
    p = prob.c()
    if block_mask.numel() != block_mask_words(prob) or block_mask.element_size() != 4:
        raise ValueError("block_mask must hold block_mask_words(prob) 32-bit words")
    if kv_group < 1 or prob.Hq % kv_group:
        raise ValueError(f"kv_group={kv_group} must divide Hq={prob.Hq}")
    o = _empty(q.shape, q.dtype, q) if o is None else o
    _check_qkv(prob, q, k, v, prob.Hq // kv_group)
    _expect("o", o, _heads(prob, prob.Hq), prob.torch_dtype)
    _check_budget(prob, budget, optional=True)
    check(lib.tsa_attention_block_sparse(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(budget),
                                         kv_group, _ptr(block_mask), _ptr(o), _stream(q.device)),
          "tsa_attention_block_sparse")
    return o


def tsa_scatter(prob: Problem, oc, rank, o=None):
    lib = _lib.load()
    p = prob.c()
    o = _empty(oc.shape, oc.dtype, oc) if o is None else o
    _expect("oc", oc, _heads(prob, prob.Hq), prob.torch_dtype)
    _expect("o", o, _heads(prob, prob.Hq), prob.torch_dtype)
    _check_rows(prob, rank=rank)
    check(lib.tsa_scatter(ctypes.byref(p), _ptr(oc), _ptr(rank), _ptr(o), _stream(oc.device)),
          "tsa_scatter")
    return o


def _check_forward(prob: Problem, q, k, v, o, budget, idx) -> None:
    _check_qkv(prob, q, k, v, prob.Hkv)
    _expect("o", o, _heads(prob, prob.Hq), prob.torch_dtype)
    _check_budget(prob, budget)
    _check_rows(prob, idx=idx)


def tsa_forward(prob: Problem, q, k, v, o=None, budget=None, idx=None, ws=None):
    lib = _lib.load()
    p = prob.c()
    o = _empty(q.shape, q.dtype, q) if o is None else o
    budget = _empty(prob.budget_shape, torch.int32, q) if budget is None else budget
    idx = _empty((prob.B, prob.Hq, prob.L), torch.int32, q) if idx is None else idx
    _check_forward(prob, q, k, v, o, budget, idx)
    ws = _ws(prob, q, ws, forward_workspace_bytes(prob))
    check(lib.tsa_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(budget),
                          _ptr(idx), _ptr(ws), ws.numel(), _stream(q.device)), "tsa_forward")
    return o, budget, idx


def tsa_attention_indexed(prob: Problem, q, k, v, idx, budget, o=None):
    """Writes only the selected rows of o; a new o is zero-filled first."""
    lib = _lib.load()
    p = prob.c()
    o = torch.zeros_like(q) if o is None else o
    _check_qkv(prob, q, k, v, prob.Hkv)
    _expect("o", o, _heads(prob, prob.Hq), prob.torch_dtype)
    _check_rows(prob, idx=idx)
    _check_budget(prob, budget)
    check(lib.tsa_attention_indexed(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                    _ptr(budget), _ptr(o), _stream(q.device)),
          "tsa_attention_indexed")
    return o


def tsa_attention_qo_indexed(prob: Problem, q, kc, vc, idx, budget, o=None):
    """Writes only the selected rows of o; a new o is zero-filled first."""
    lib = _lib.load()
    p = prob.c()
    o = torch.zeros_like(q) if o is None else o
    _check_qkv(prob, q, kc, vc, prob.Hq)
    _expect("o", o, _heads(prob, prob.Hq), prob.torch_dtype)
    _check_rows(prob, idx=idx)
    _check_budget(prob, budget)
    check(lib.tsa_attention_qo_indexed(ctypes.byref(p), _ptr(q), _ptr(kc), _ptr(vc), _ptr(idx),
                                       _ptr(budget), _ptr(o), _stream(q.device)),
          "tsa_attention_qo_indexed")
    return o


def tsa_zero_unselected(prob: Problem, rank, o):
    lib = _lib.load()
    p = prob.c()
    _check_rows(prob, rank=rank)
    _expect("o", o, _heads(prob, prob.Hq), prob.torch_dtype)
    check(lib.tsa_zero_unselected(ctypes.byref(p), _ptr(rank), _ptr(o), _stream(o.device)),
          "tsa_zero_unselected")
    return o


def tsa_forward_fused(prob: Problem, q, k, v, o=None, budget=None, idx=None, ws=None):
    lib = _lib.load()
    p = prob.c()
    o = _empty(q.shape, q.dtype, q) if o is None else o
    budget = _empty(prob.budget_shape, torch.int32, q) if budget is None else budget
    idx = _empty((prob.B, prob.Hq, prob.L), torch.int32, q) if idx is None else idx
    _check_forward(prob, q, k, v, o, budget, idx)
    ws = _ws(prob, q, ws, fused_workspace_bytes(prob))
    check(lib.tsa_forward_fused(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                _ptr(budget), _ptr(idx), _ptr(ws), ws.numel(),
                                _stream(q.device)), "tsa_forward_fused")
    return o, budget, idx


def forward(q, k, v, w: int, tau: float, fused: bool = False, flags: int = 0):
    """The whole op on torch device tensors: returns (o, budget, idx)."""
    prob = Problem.from_qkv(q, k, w, tau, flags)
    return (tsa_forward_fused if fused else tsa_forward)(prob, q, k, v)


__all__ = ["Problem", "TsaError", "workspace_bytes", "forward_workspace_bytes",
           "fused_workspace_bytes", "tsa_score", "tsa_budget", "tsa_select", "tsa_gather",
           "tsa_gather_kv",
           "tsa_attention", "tsa_scatter", "tsa_forward", "tsa_attention_indexed",
           "tsa_forward_fused", "tsa_zero_unselected", "block_mask_words",
           "tsa_attention_block_sparse", "forward", "TSA_FLAG_NONCAUSAL_PROXY",
           "TSA_FLAG_PER_HEAD_BUDGET", "TSA_FLAG_KEEP_WINDOW"]


# ---------------------------------------------------------------- measurement probe
def probe_sink_bytes() -> int:
    return int(_lib.load_probe().tsa_probe_sink_bytes())


def probe_mfma_bf16(random_operands: bool, iters: int, sink: torch.Tensor) -> float:
    """Enqueue the bf16 MFMA ceiling probe (include/tsa_probe.h) on the current stream;
    returns the launch's MFMA FLOPs.  sink: a device tensor of probe_sink_bytes() bytes."""
    lib = _lib.load_probe()
    flops = ctypes.c_double(0.0)
    rc = lib.tsa_probe_mfma_bf16(int(bool(random_operands)), int(iters), _ptr(sink),
                                 sink.numel() * sink.element_size(), ctypes.byref(flops),
                                 _stream(sink.device))
    if rc != 0:
        raise RuntimeError(f"tsa_probe_mfma_bf16 failed with status {rc}")
    return flops.value

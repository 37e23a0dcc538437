#!/usr/bin/env python3
"""Benchmark of the Token Sparse Attention prefill op on one MI355X.

One step = one pass of the whole op over one batch of seeded synthetic Q, K,
V already resident in HBM.  Two paths compute it, bit for bit alike:
  fused: tsa_forward_fused = score -> budget -> select -> zero the
      unselected output rows -> attention reading Q, K, V through the index
      set and writing O rows to their sequence positions;
  steps (default): tsa_forward = score -> budget -> select -> gather -> attention on
      the compact tensors -> scatter.
The chosen path is timed for K steps; the other is timed too and reported.
Printed as one JSON line, with:
  * the dense causal attention baseline (same attention kernel, GQA head map,
    no selection) and the speedup against it;
  * a per-kernel breakdown of both paths timed with HIP events on the launch
    stream, and the roofline of the dominant kernel (the attention of the
    timed path) from those launches, beside the sustained rate of a bare bf16
    MFMA loop on the same GPU with random and with constant operands (the
    chip's clock depends on how much the operands toggle);
  * the fp64 CPU oracle timed on a bounded sample of the same workload;
  * the alternative readings (TSA_FLAG_* bits): K/L and ms per layer of the
    timed path under each, against the same dense baseline;
  * the block-sparse composition: the attention on the compressed tensors
    under seeded block masks of several densities (ms, visible fraction,
    TFLOP/s on the visible block pairs);
  * a synthetic 4-layer stack with random weights at the 32K shape (Hq=32,
    Hkv=8, d=128): every layer re-selects; per-layer K/L, overlap of the
    index sets of consecutive layers, and the stack's time against the same
    stack with dense attention;
  * a sweep over the other workloads (8K; 32K with Zipf-biased keys at
    tau = 0.01, 0.05, 0.1; B=2 64K with 7 query heads per KV head; the
    Zipf-biased keys at 128K, tau = 0.05, 0.1, 0.2): ms per
    layer of the op and of the dense attention, speedup, K/L, the share of
    the non-attention kernels and the attention's MFMA fraction;
  * the compact attention on operands that barely toggle (all ones; random
    signs of powers of two) beside its time on the compressed tensors;
  * beside every K/L, the importance mass the top 1% of tokens hold per
    head (how skewed the scores are, which bounds what tau can prune);
  * per kernel, the HBM bytes that rocprofv3 counters recorded for the same
    kernel source (profiles/traffic.json) beside its algorithmic bytes;
  * provenance: source hashes, GPU, ROCm and torch versions, seeds, and a
    parity check of a small case against the fp64 oracle.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--path fused|steps]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TSA attention ms/layer at 128K bf16; speedup vs own dense; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3          # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "token_sparse_attention_proxy_amd", "csrc", "attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_flops(budget, Hq: int, d: int) -> float:
    """Algorithmic FLOPs of causal attention over K rows: 4d per visible (i, j) pair.
    budget: [B] (every head of a sequence has K_b rows) or [B,Hq] (per head)."""
    budget = np.asarray(budget)
    if budget.ndim == 2:
        return float(sum(2.0 * d * int(K) * (int(K) + 1) for K in budget.ravel()))
    return float(sum(2.0 * d * int(K) * (int(K) + 1) * Hq for K in budget))


def block_sparse_flops(words: np.ndarray, n: int, d: int) -> float:
    """Algorithmic FLOPs (4d per visible causal pair) of block-sparse attention over the
    first n compact rows of every head: visible off-diagonal blocks plus the diagonal."""
    B, H, nb, nw = words.shape
    bits = np.unpackbits(words.view(np.uint8).reshape(B, H, nb, nw * 4), axis=-1,
                         bitorder="little")[..., :nb].astype(bool)
    size = np.minimum(64, np.maximum(0, n - 64 * np.arange(nb)))          # rows per block
    below = np.tril(np.ones((nb, nb), dtype=bool), k=-1)
    pairs_off = (bits & below) * (size[:, None] * size[None, :])
    pairs_diag = size * (size + 1) // 2
    total = pairs_off.sum(axis=(-2, -1)).astype(np.float64) + pairs_diag.sum()
    return float(4.0 * d * total.sum())


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


CSRC = os.path.join(ROOT, "token_sparse_attention_proxy_amd", "csrc")


def load_traffic():
    try:
        with open(TRAFFIC_FILE) as f:
            return json.load(f)
    except (OSError, ValueError):
        return {}


def counter_bytes(tab: dict, kernels, workload: str):
    """Sum of the counter bytes per launch of these kernels (short names), or None unless
    every one was recorded for this workload from the kernel source as it is now."""
    total = 0.0
    for kn in kernels:
        ent = tab.get(kn, {}).get(workload)
        src = ent and os.path.join(CSRC, ent.get("source", "attention.hip"))
        if not ent or not os.path.exists(src) or ent.get("source_sha") != source_hash(src):
            return None
        total += ent["bytes_per_launch"]
    return total


def provenance(wl, tau):
    """Where and from what this line was measured."""
    import subprocess
    import torch
    sha = None
    try:
        sha = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"], cwd=ROOT, capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h")))
    h = hashlib.sha256()
    for f in srcs:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    props = torch.cuda.get_device_properties(0)
    return {"git_sha": sha, "csrc_sha": h.hexdigest()[:16], "bench_sha": source_hash(__file__),
            "gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": torch.version.hip,
            "torch": torch.__version__, "seed": wl.seed(0), "tau": tau}


def parity_check():
    """A small whole op against the fp64 oracle: budgets and index sets exact, outputs within
    2e-2 of the largest reference output per head (the library's bf16 tolerance)."""
    import torch
    from oracle import tsa_oracle as O
    from token_sparse_attention_proxy_amd import inputs
    from token_sparse_attention_proxy_amd import tsa as T
    wl = inputs.small_workload("bf16", B=1, Hq=8, Hkv=2, L=1500, d=128, w=64, tau=0.05,
                               seed_base=9700)
    q, k, v = inputs.make_qkv(wl)
    dev = torch.device("cuda:0")
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, 0.05, "bf16")
    o, budget, idx = T.tsa_forward(prob, qd, kd, vd)
    torch.cuda.synchronize()
    ref = O.forward(q, k, v, wl.w, 0.05)
    kb = int(budget.cpu()[0])
    ok_budget = kb == int(ref["budget"][0])
    idx_np = idx.cpu().numpy()
    ok_sets = ok_budget and bool(np.array_equal(idx_np[0, :, :kb], ref["idx"][0, :, :kb]))
    o_np = o.float().cpu().numpy().astype(np.float64)
    worst = max(float(np.abs(o_np[0, h] - ref["o"][0, h]).max() / np.abs(ref["o"][0, h]).max())
                for h in range(wl.Hq))
    return {"case": wl.name, "budget_exact": ok_budget, "sets_exact": ok_sets,
            "worst_rel_err": float(f"{worst:.3e}"), "ok": bool(ok_sets and worst <= 2e-2)}


def top1_mass_share(s) -> dict:
    """Per (b, h): the importance mass held by the top 1% of tokens (the head's largest
    ceil(L/100) scores over its total), the skew that bounds what any coverage budget prunes."""
    import torch
    L = s.shape[-1]
    kk = max(1, (L + 99) // 100)
    share = (torch.topk(s, kk, dim=-1).values.sum(-1) / s.sum(-1)).flatten().cpu().numpy()
    return {"per_head": [round(float(x), 4) for x in share], "mean": round(float(share.mean()), 4),
            "min": round(float(share.min()), 4), "max": round(float(share.max()), 4)}


def sweep_one(name: str, taus, dev, steps: int):
    """One workload of the sweep: the op (tsa_forward) per tau against the dense attention."""
    import torch
    from token_sparse_attention_proxy_amd import inputs
    from token_sparse_attention_proxy_amd import tsa as T
    from token_sparse_attention_proxy_amd._lib import FORWARD_FUSED_MAX_L
    wl = inputs.WORKLOADS[name]
    q, k, v = inputs.make_qkv(wl)
    qd, kd, vd = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (q, k, v))
    del q, k, v
    st = torch.cuda.current_stream(dev)
    shape = (wl.B, wl.Hq, wl.L, wl.d)
    o = torch.empty(shape, dtype=torch.bfloat16, device=dev)

    # Each repetition of each call is timed on its own after a 512 MiB write, so that neither
    # the 256 MiB Infinity Cache nor the L2 holds this workload's tensors from the previous
    # one. The calls compared are interleaved, in alternating order from one repetition to
    # the next, so none of them is favoured by its place in the run; medians are reported.
    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def timed(fns: dict, reps):
        for fn in fns.values():
            fn()
        torch.cuda.synchronize()
        ts = {n: [] for n in fns}
        items = list(fns.items())
        for r in range(reps):
            for n, fn in (items if r % 2 == 0 else items[::-1]):
                evict.fill_(r & 0xff)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                fn()
                e1.record(st)
                torch.cuda.synchronize()
                ts[n].append(e0.elapsed_time(e1))
        return {n: float(np.median(v)) for n, v in ts.items()}

    prob0 = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, float(taus[0]), "bf16")
    dense_tf = attention_flops([wl.L] * wl.B, wl.Hq, wl.d)
    o2 = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    out = []
    for tau in taus:
        prob = dataclasses.replace(prob0, tau=float(tau))
        ws = torch.empty(T.forward_workspace_bytes(prob), dtype=torch.uint8, device=dev)
        budget = torch.empty((wl.B,), dtype=torch.int32, device=dev)
        idx = torch.empty((wl.B, wl.Hq, wl.L), dtype=torch.int32, device=dev)
        T.tsa_forward(prob, qd, kd, vd, o, budget, idx, ws)
        bud = budget.cpu().numpy()
        # the op's attention alone needs the compact K and V: its own workspace
        s = torch.empty((wl.B, wl.Hq, wl.L), dtype=torch.float32, device=dev)
        step_ws = torch.empty(T.workspace_bytes(prob), dtype=torch.uint8, device=dev)
        T.tsa_score(prob, qd, kd, s, step_ws)
        _, rank = T.tsa_select(prob, s, budget, None, None, step_ws)
        kc, vc = T.tsa_gather_kv(prob, kd, vd, rank)
        # tsa_forward; the same op through the fused path (the attention reads K and V through
        # the index set instead of compact copies: the same bits, another cost split; up to
        # 32K tokens tsa_forward runs these kernels itself); the attention tsa_forward runs,
        # alone; the dense attention on the same tensors
        if wl.L <= FORWARD_FUSED_MAX_L:
            attn = lambda: T.tsa_attention_indexed(prob, qd, kd, vd, idx, budget, o2)   # noqa: E731
        else:
            attn = lambda: T.tsa_attention_qo_indexed(prob, qd, kc, vc, idx, budget, o2)   # noqa: E731
        t = timed({"op": lambda: T.tsa_forward(prob, qd, kd, vd, o, budget, idx, ws),
                   "fused": lambda: T.tsa_forward_fused(prob, qd, kd, vd, o, budget, idx, ws),
                   "attention": attn,
                   "dense": lambda: T.tsa_attention(prob0, qd, kd, vd, None, wl.G, o2)}, steps)
        ms, fused_ms, attn_ms, dense_ms = t["op"], t["fused"], t["attention"], t["dense"]
        fl = attention_flops(bud, wl.Hq, wl.d)
        kl = bud / wl.L
        rec = {"workload": name, "tau": float(tau), "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv,
               "L": wl.L, "w": wl.w, "keep_frac": [round(float(x), 5) for x in kl],
               "top1pct_mass": top1_mass_share(s),
               "ms_per_layer": round(ms, 4), "fused_ms_per_layer": round(fused_ms, 4),
               "dense_ms": round(dense_ms, 4),
               "speedup_vs_dense": round(dense_ms / ms, 4),
               "attention_ms": round(attn_ms, 4),
               "overhead_share": round((ms - attn_ms) / attn_ms, 4),
               "attention_mfma_frac": round(fl / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               "dense_mfma_frac": round(dense_tf / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] sweep {name} tau={tau}: {ms:.3f} ms (fused path {fused_ms:.3f}) vs dense "
            f"{dense_ms:.3f} ms "
            f"(x{dense_ms / ms:.3f}), K/L {kl.round(4)}, attention {attn_ms:.3f} ms, "
            f"overhead {rec['overhead_share']:.4f}")
        out.append(rec)
        del ws, budget, idx, s, step_ws, rank, kc, vc
    del qd, kd, vd, o, o2, evict
    torch.cuda.empty_cache()
    return out


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counters, if they match this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            tab = json.load(f)
    except (OSError, ValueError):
        return None
    ent = tab.get(kernel, {}).get(workload)
    if not ent or ent.get("source_sha") != source_hash(ATTN_SRC):
        return None
    return ent.get("bytes_per_launch")


def operand_dependence(prob, shape, budget, flops, st, reps: int = 3):
    """The compact attention (the breakdown's `attention` call: same kernel, launch and
    budget) on operands of the same shapes whose values barely toggle: all ones, and random
    signs of powers of two (q = +-1/4, k, v = +-1; exponents and signs only, zero
    mantissas).  The instruction stream is the same as on the real data; only the operand
    values change.  Median of reps launches after one warm-up, HIP events on the stream."""
    import torch
    from token_sparse_attention_proxy_amd import tsa as T
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(11)
    res = {}
    for key in ("all_ones", "random_signs"):
        if key == "all_ones":
            one = torch.ones(shape, dtype=torch.bfloat16, device=dev)
            q = k = v = one
        else:
            sgn = lambda: (torch.randint(0, 2, shape, device=dev, generator=g) * 2 - 1).to(torch.bfloat16)
            q, k, v = sgn() * 0.25, sgn(), sgn()
        o = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        T.tsa_attention(prob, q, k, v, budget, 1, o)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            T.tsa_attention(prob, q, k, v, budget, 1, o)
            e1.record(st)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        tf = flops / (ms * 1e-3) / 1e12
        res[key] = {"ms": round(ms, 4), "TFLOP_s": round(tf, 1),
                    "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        del q, k, v, o
    res["launches"] = 2 * (1 + reps)
    return res


def mfma_ceiling(st, iters: int = 60000, reps: int = 2):
    """Sustained bf16 MFMA rate of a register-only loop (two waves per SIMD, four
    accumulator chains), with random and with constant operands; best of reps launches
    of about 30-50 ms each, timed with HIP events on the launch stream."""
    import torch
    from token_sparse_attention_proxy_amd import tsa as T
    sink = torch.empty(T.probe_sink_bytes() // 4, dtype=torch.float32, device="cuda")
    res = {}
    for key, rnd in (("random_operands", True), ("constant_operands", False)):
        T.probe_mfma_bf16(rnd, 100, sink)
        best = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            fl = T.probe_mfma_bf16(rnd, iters, sink)
            e1.record(st)
            torch.cuda.synchronize()
            best = max(best, fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        res[key] = round(best, 1)
    assert bool(torch.isfinite(sink).all()), "probe accumulators not finite"
    res["unit"] = "TFLOP/s"
    res["what"] = ("v_mfma_f32_32x32x16_bf16 loop, operands in registers, 2 waves/SIMD, "
                   "one workgroup per CU; random: random signs/mantissas, magnitudes in [0.25, 2)")
    return res


def full_oracle_small():
    """The whole fp64 oracle forward, unsampled, on the 1K fp32 workload (B=1, Hq=Hkv=4,
    L=1024, d=64, w=16): the one configuration small enough to time in full here."""
    from oracle import tsa_oracle as O
    from token_sparse_attention_proxy_amd import inputs
    wl = inputs.WORKLOADS["tiny_mha_f32_L1k"]
    q, k, v = inputs.make_qkv(wl)
    t0 = time.perf_counter()
    O.forward(q, k, v, wl.w, wl.taus[0])
    return {"workload": wl.name, "ms_per_layer": round((time.perf_counter() - t0) * 1e3, 1)}


def cpu_baseline(wl, q, k, v, tau, K_gpu: int):
    """The fp64 oracle, as it stands, on a bounded sample; scaled to ms/layer."""
    from threadpoolctl import threadpool_info
    from oracle import tsa_oracle as O

    B, Hq, Hkv, L, d = wl.B, wl.Hq, wl.Hkv, wl.L, wl.d
    t0 = time.perf_counter()
    s = O.proxy_scores(q, k, wl.w)
    t_score = time.perf_counter() - t0
    t0 = time.perf_counter()
    budget = O.coverage_budget(s, tau)
    t_budget = time.perf_counter() - t0
    # per-head steps on head (0, 0), scaled by the number of heads
    K = int(budget[0])
    t0 = time.perf_counter()
    idx, _ = O.select_heads(s[:1, :1], budget[:1])
    t_select = (time.perf_counter() - t0) * B * Hq
    t0 = time.perf_counter()
    qc, kc, vc = O.gather(q[:1, :1], k[:1, :1], v[:1, :1], idx, budget[:1])
    t_gather = (time.perf_counter() - t0) * B * Hq
    # attention on the last rows of the compact sequence (the most expensive ones)
    n_rows = min(K, 24576 if L >= 65536 else 8192)
    rows = np.arange(K - n_rows, K)
    t0 = time.perf_counter()
    oc_rows = O.causal_attention(qc[0, 0, :K], kc[0, 0, :K], vc[0, 0, :K], rows=rows)
    t_attn_sample = time.perf_counter() - t0
    pairs_sample = float(np.sum(rows + 1))
    pairs_layer = float(sum(int(kb) * (int(kb) + 1) // 2 for kb in budget)) * Hq
    t_attn = t_attn_sample * pairs_layer / pairs_sample
    oc = np.zeros((1, 1, L, d))
    oc[0, 0, rows] = oc_rows
    t0 = time.perf_counter()
    O.scatter(oc, idx, budget[:1])
    t_scatter = (time.perf_counter() - t0) * B * Hq
    total = t_score + t_budget + t_select + t_gather + t_attn + t_scatter
    info = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in info] + [1])
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    host = {"cpu_model": cpu_model, "affinity": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "numpy": np.__version__,
            "blas": sorted({f"{p.get('internal_api')} {p.get('version')}" for p in info if p.get("user_api") == "blas"})}
    return {
        "value": round(total * 1e3, 1), "unit": "ms/layer", "cores": int(threads), "kind": "oracle",
        "sample": (f"fp64 oracle: scores+budget for all {B * Hq} heads in full; select, gather "
                   f"and scatter of head (0,0) x{B * Hq}; attention of the last {n_rows} compact "
                   f"rows of head (0,0) (K={K}) scaled by causal pairs x{pairs_layer / pairs_sample:.0f}"),
        "measured_s": round(t_score + t_budget + t_select / (B * Hq) + t_gather / (B * Hq)
                            + t_attn_sample + t_scatter / (B * Hq), 2),
        "budget_matches_gpu": bool(int(budget[0]) == K_gpu),
        "full_oracle_small": full_oracle_small(),
        "host": host,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_bf16_L128k")
    ap.add_argument("--tau", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--path", choices=["fused", "steps"], default="steps")
    ap.add_argument("--no-readings", action="store_true")
    ap.add_argument("--no-block-sparse", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the op runs on a single MI355X; sharding by KV head is a design note only)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from token_sparse_attention_proxy_amd import inputs
    from token_sparse_attention_proxy_amd import tsa as T

    wl = inputs.WORKLOADS[args.workload]
    tau = float(wl.taus[0] if args.tau is None else args.tau)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {wl.name} tau={tau}: generating inputs")
    q, k, v = inputs.make_qkv(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(tdt).to(dev) for x in (q, k, v))
    if args.no_cpu_baseline:
        del q, k, v
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, tau, wl.dtype)
    shape = (wl.B, wl.Hq, wl.L, wl.d)
    o = torch.empty(shape, dtype=tdt, device=dev)
    budget = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    idx = torch.empty((wl.B, wl.Hq, wl.L), dtype=torch.int32, device=dev)
    ws = torch.empty(T.forward_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream(dev)
    paths = {"fused": lambda: T.tsa_forward_fused(prob, qd, kd, vd, o, budget, idx, ws),
             "steps": lambda: T.tsa_forward(prob, qd, kd, vd, o, budget, idx, ws)}
    other = "steps" if args.path == "fused" else "fused"

    # ---- headline: K timed steps of the chosen path
    log(f"[bench] warmup {args.warmup} ({args.path})")
    for _ in range(args.warmup):
        paths[args.path]()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        paths[args.path]()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    bud = budget.cpu().numpy()
    log(f"[bench] {args.path} {ms_step:.3f} ms/step, budget {bud} K/L {bud / wl.L}")

    # ---- the other path, for comparison (same results)
    oreps = max(2, min(args.steps, 5))
    paths[other]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(oreps):
        paths[other]()
    torch.cuda.synchronize()
    other_ms = (time.perf_counter() - t0) * 1e3 / oreps
    log(f"[bench] {other} {other_ms:.3f} ms/step")

    # ---- per-kernel breakdown: the kernels called one by one, HIP events between them
    heads = wl.B * wl.Hq
    step_ws = torch.empty(T.workspace_bytes(prob), dtype=torch.uint8, device=dev)
    s = torch.empty((wl.B, wl.Hq, wl.L), dtype=torch.float32, device=dev)
    rank = torch.empty_like(idx)
    qc, kc, vc, oc = (torch.empty(shape, dtype=tdt, device=dev) for _ in range(4))
    calls = {
        "score": lambda: T.tsa_score(prob, qd, kd, s, step_ws),
        "budget": lambda: T.tsa_budget(prob, s, budget, step_ws),
        "select": lambda: T.tsa_select(prob, s, budget, idx, rank, step_ws),
        "gather": lambda: T.tsa_gather(prob, qd, kd, vd, idx, budget, qc, kc, vc),
        "gather_kv": lambda: T.tsa_gather_kv(prob, kd, vd, rank, kc, vc),
        "attention": lambda: T.tsa_attention(prob, qc, kc, vc, budget, 1, oc),
        "scatter": lambda: T.tsa_scatter(prob, oc, rank, o),
        "zero_fill": lambda: T.tsa_zero_unselected(prob, rank, o),
        "attention_indexed": lambda: T.tsa_attention_indexed(prob, qd, kd, vd, idx, budget, o),
        "attention_qo": lambda: T.tsa_attention_qo_indexed(prob, qd, kc, vc, idx, budget, o),
    }
    names = list(calls)
    per_rep = {n: [] for n in names}
    reps = max(3, min(args.steps, 10))
    # Before every repetition a 512 MiB buffer is written, so the first kernel of the
    # repetition finds neither the 256 MiB Infinity Cache nor the L2 warm from the last one.
    evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for rep in range(reps + 1):
        evict.fill_(rep & 0xff)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        ev[0].record(st)
        for i, n in enumerate(names):
            calls[n]()
            ev[i + 1].record(st)
        torch.cuda.synchronize()
        if rep > 0:       # first pass is a warm-up
            for i, n in enumerate(names):
                per_rep[n].append(ev[i].elapsed_time(ev[i + 1]))
    del evict
    steps_ms = {n: float(np.mean(per_rep[n])) for n in names}
    top1 = top1_mass_share(s)
    log("[bench] kernels ms: " + ", ".join(f"{n} {steps_ms[n]:.3f}" for n in steps_ms))

    # ---- the bf16 MFMA ceiling on this GPU, right after the attention launches: a
    # register-only MFMA loop with random and with constant operands (include/tsa_probe.h)
    ceiling = mfma_ceiling(st) if wl.dtype == "bf16" else None
    if ceiling:
        log(f"[bench] MFMA ceiling: random operands {ceiling['random_operands']} TFLOP/s, "
            f"constant operands {ceiling['constant_operands']} TFLOP/s")
    # ---- the same compact attention on operands that barely toggle
    opdep = None
    if wl.dtype == "bf16":
        opdep = operand_dependence(prob, shape, budget, attention_flops(budget.cpu().numpy(), wl.Hq, wl.d), st)
        log("[bench] compact attention by operand data: real " + f"{steps_ms['attention']:.3f} ms, " +
            ", ".join(f"{k} {v['ms']:.3f} ms (frac {v['frac']})" for k, v in opdep.items()
                      if isinstance(v, dict)))

    # ---- dense causal attention baseline (same kernel, GQA head map)
    dense_ms = None
    if not args.no_dense:
        od = torch.empty(shape, dtype=tdt, device=dev)
        for _ in range(max(1, args.warmup)):
            T.tsa_attention(prob, qd, kd, vd, None, wl.G, od)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dreps = max(2, min(args.steps, 5))
        e0.record(st)
        for _ in range(dreps):
            T.tsa_attention(prob, qd, kd, vd, None, wl.G, od)
        e1.record(st)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / dreps
        del od
        log(f"[bench] dense attention {dense_ms:.3f} ms")

    # ---- alternative readings: K/L and time of the whole op under each flag set
    readings = None
    if not args.no_readings:
        readings = {}
        NC, PH, KW = T.TSA_FLAG_NONCAUSAL_PROXY, T.TSA_FLAG_PER_HEAD_BUDGET, T.TSA_FLAG_KEEP_WINDOW
        for name, fl in [("main", 0), ("noncausal_proxy", NC), ("per_head_budget", PH),
                         ("keep_window", KW), ("all", NC | PH | KW)]:
            p2 = dataclasses.replace(prob, flags=fl)
            ws2 = torch.empty(T.forward_workspace_bytes(p2), dtype=torch.uint8, device=dev)
            b2 = torch.empty(p2.budget_shape, dtype=torch.int32, device=dev)
            fn = (lambda: T.tsa_forward_fused(p2, qd, kd, vd, o, b2, idx, ws2)) if args.path == "fused" \
                else (lambda: T.tsa_forward(p2, qd, kd, vd, o, b2, idx, ws2))
            fn()
            torch.cuda.synchronize()
            r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            rreps = max(2, min(args.steps, 3))
            r0.record(st)
            for _ in range(rreps):
                fn()
            r1.record(st)
            torch.cuda.synchronize()
            ms = r0.elapsed_time(r1) / rreps
            kb = b2.cpu().numpy()
            kl = kb.astype(np.float64) / wl.L
            readings[name] = {"flags": fl, "ms_per_layer": round(ms, 4),
                              "keep_frac_mean": round(float(kl.mean()), 5),
                              "keep_frac_min": round(float(kl.min()), 5),
                              "keep_frac_max": round(float(kl.max()), 5),
                              "attention_tflop": round(attention_flops(kb, wl.Hq, wl.d) / 1e12, 3),
                              "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms, 4)}
            log(f"[bench] reading {name}: {ms:.3f} ms, K/L mean {kl.mean():.4f} "
                f"[{kl.min():.4f}, {kl.max():.4f}]")
            del ws2, b2
        paths[args.path]()              # restore the main reading's budget, idx and o
        torch.cuda.synchronize()

    # ---- block-sparse composition on the compressed tensors of this step
    block_sparse = None
    if not args.no_block_sparse and wl.B == 1:
        block_sparse = {}
        n = int(bud[0])
        for name, pat, dens in [("all", "all", 1.0), ("random_0.5", "random", 0.5),
                                ("random_0.25", "random", 0.25), ("random_0.1", "random", 0.1),
                                ("vertical_slash", "vertical_slash", 0.0)]:
            mw = inputs.make_block_mask(wl.B, wl.Hq, wl.L, seed=1234, pattern=pat, density=dens,
                                        band=16, columns=32)
            md = torch.from_numpy(mw.view(np.int32)).to(dev)
            T.tsa_attention_block_sparse(prob, qc, kc, vc, md, budget, 1, oc)
            torch.cuda.synchronize()
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            breps = max(2, min(args.steps, 3))
            b0.record(st)
            for _ in range(breps):
                T.tsa_attention_block_sparse(prob, qc, kc, vc, md, budget, 1, oc)
            b1.record(st)
            torch.cuda.synchronize()
            ms = b0.elapsed_time(b1) / breps
            fl = block_sparse_flops(mw, n, wl.d)
            block_sparse[name] = {"ms": round(ms, 4), "visible_frac": round(fl / attention_flops(bud, wl.Hq, wl.d), 4),
                                  "TFLOP_s": round(fl / (ms * 1e-3) / 1e12, 2),
                                  "mfma_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                                  if wl.dtype == "bf16" else None}
            log(f"[bench] block-sparse {name}: {ms:.3f} ms, visible {block_sparse[name]['visible_frac']:.3f}, "
                f"{block_sparse[name]['TFLOP_s']} TFLOP/s")
            del md

    # ---- synthetic multi-layer stack: re-selection in every layer
    stack_rep = None
    if not args.no_stack:
        from token_sparse_attention_proxy_amd import stack as S
        scfg = S.StackConfig(B=1, L=32768, Hq=32, Hkv=8, d=128, layers=4, w=64, tau=0.05,
                             fused=args.path == "fused")
        sg = torch.Generator(device=dev).manual_seed(4321)
        sx = torch.randn((scfg.B, scfg.L, scfg.model_dim), generator=sg, device=dev).to(torch.bfloat16)
        sw = S.make_weights(scfg, seed=4322, device=dev)

        def stack_ms(dense):
            S.run_stack(scfg, sx, sw, dense=dense)
            torch.cuda.synchronize()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(st)
            for _ in range(2):
                out = S.run_stack(scfg, sx, sw, dense=dense)
            s1.record(st)
            torch.cuda.synchronize()
            return s0.elapsed_time(s1) / 2, out[1]
        tsa_ms, recs = stack_ms(False)
        dense_stack_ms, _ = stack_ms(True)
        kl = [round(float(r["budget"].float().mean()) / scfg.L, 4) for r in recs]
        stack_rep = {"config": dataclasses.asdict(scfg), "ms_tsa": round(tsa_ms, 3),
                     "ms_dense": round(dense_stack_ms, 3),
                     "speedup": round(dense_stack_ms / tsa_ms, 4), "keep_frac_per_layer": kl,
                     "reselection": [{k2: (round(v2, 4) if v2 is not None else None) for k2, v2 in r.items()}
                                     for r in S.reselection(scfg, recs)],
                     "note": "random weights, projections by torch.matmul; no accuracy claim"}
        log(f"[bench] stack: {tsa_ms:.2f} ms vs dense {dense_stack_ms:.2f} ms, K/L {kl}, "
            f"reselection {stack_rep['reselection']}")
        del sx, sw, recs

    # ---- roofline of the dominant kernel (the timed path's attention), algorithmic FLOPs
    bf16 = wl.dtype == "bf16"
    flops = attention_flops(bud, wl.Hq, wl.d)
    attn_step = "attention_indexed" if args.path == "fused" else "attention_qo"
    kname = ("attn_fwd_bf16" if bf16 else "attn_fwd_f32") + \
        (f"<{wl.d}, true, false, false>" if args.path == "fused" else f"<{wl.d}, false, false, true>")
    achieved = flops / (steps_ms[attn_step] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    traffic = measured_traffic(kname, wl.name) if bf16 else None
    roofline = {"bound": "mfma" if bf16 else "alu", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "kernel": kname,
                "flops_per_launch": flops, "avg_launch_ms": round(steps_ms[attn_step], 4)}
    if ceiling:
        ceiling["attention_frac_of_random"] = round(achieved / ceiling["random_operands"], 4)
        roofline["mfma_ceiling"] = ceiling
    if opdep:
        att_ms = steps_ms["attention"]
        opdep["real_data"] = {"ms": round(att_ms, 4),
                              "frac": round(flops / (att_ms * 1e-3) / 1e12 / peak, 4)}
        opdep["what"] = ("the compact attention (tsa_attention, kv_group 1, the headline budget) on "
                         "the compressed tensors (real_data) and on operands of the same shapes "
                         "that barely toggle; same kernel and instruction stream")
        roofline["operand_dependence"] = opdep

    # HBM fractions of the byte-moving steps (algorithmic bytes)
    eb = 2 if bf16 else 4
    idx_np = idx.cpu().numpy()
    uniq = 0
    for b in range(wl.B):
        for g in range(wl.Hkv):
            hs = range(g * wl.G, (g + 1) * wl.G)
            uniq += len(np.unique(np.concatenate([idx_np[b, h, :bud[b]] for h in hs])))
    Ksum = float(sum(int(x) for x in bud)) * wl.Hq
    row = wl.d * eb
    hbm_bytes = {
        "score": wl.B * wl.Hkv * wl.L * row + heads * wl.w * row + 4 * heads * wl.L,
        "budget": 4 * heads * wl.L,
        "select": 4 * heads * wl.L + 4 * Ksum + 4 * heads * wl.L,
        "gather": Ksum * row + 2 * uniq * row + 3 * Ksum * row + 4 * Ksum,
        "gather_kv": 2 * uniq * row + 2 * Ksum * row + 4 * heads * wl.L,
        "scatter": Ksum * row + heads * wl.L * row + 4 * heads * wl.L,
        "zero_fill": 4 * heads * wl.L + (heads * wl.L - Ksum) * row,
    }
    kernels = {n: {"ms": round(steps_ms[n], 4), "ms_median": round(float(np.median(per_rep[n])), 4),
                   "ms_min": round(float(np.min(per_rep[n])), 4),
                   "GB_s": round(hbm_bytes[n] / (steps_ms[n] * 1e-3) / 1e9, 1),
                   "hbm_frac": round(hbm_bytes[n] / (steps_ms[n] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "algorithmic_bytes": int(hbm_bytes[n])} for n in hbm_bytes}
    # HBM bytes from rocprofv3 FETCH_SIZE + WRITE_SIZE of the same kernel sources (null when a
    # source changed since they were recorded), and their ratio to the algorithmic bytes
    from token_sparse_attention_proxy_amd.profiling import step_kernels
    traffic_tab = load_traffic()
    for n, kns in step_kernels(wl.d, wl.d * eb // 16).items():
        cb = counter_bytes(traffic_tab, kns, wl.name) if bf16 else None
        kernels[n]["counter_bytes"] = None if cb is None else int(cb)
        kernels[n]["counter_over_algorithmic"] = None if cb is None else round(cb / hbm_bytes[n], 3)
        kernels[n]["counter_GB_s"] = None if cb is None else round(cb / (steps_ms[n] * 1e-3) / 1e9, 1)
    # proxy scoring also runs MFMA work and exps: two passes, each over every (proxy row, key)
    sc_s = steps_ms["score"] * 1e-3
    sc_rows = heads * 32 * ((wl.w + 31) // 32)          # proxy rows padded to whole 32-row tiles
    kernels["score"]["two_pass_tflop"] = round(2 * 2.0 * sc_rows * wl.L * wl.d / 1e12, 4)
    kernels["score"]["TFLOP_s"] = round(2 * 2.0 * sc_rows * wl.L * wl.d / sc_s / 1e12, 2)
    kernels["score"]["mfma_frac"] = round(kernels["score"]["TFLOP_s"] / peak, 4) if bf16 else None
    kernels["score"]["exp_per_s"] = float(f"{2.0 * heads * wl.w * wl.L / sc_s:.4g}")
    for n in ("attention", "attention_indexed", "attention_qo"):
        tf = flops / (steps_ms[n] * 1e-3) / 1e12
        kernels[n] = {"ms": round(steps_ms[n], 4), "ms_median": round(float(np.median(per_rep[n])), 4),
                      "ms_min": round(float(np.min(per_rep[n])), 4), "TFLOP_s": round(tf, 2),
                      "mfma_frac": round(tf / peak, 4)}
    path_kernels = {"fused": ["score", "budget", "select", "zero_fill", "attention_indexed"],
                    "steps": ["score", "budget", "select", "gather_kv", "zero_fill", "attention_qo"],
                    "entry_points": ["score", "budget", "select", "gather", "attention", "scatter"]}
    overhead = sum(steps_ms[n] for n in path_kernels[args.path] if n != attn_step)

    out = {
        "metric": METRIC,
        "value": round(ms_step, 4),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "L": wl.L,
                   "d": wl.d, "w": wl.w, "tau": tau, "global_batch": wl.B, "seq_len": wl.L,
                   "parallelism": "none"},
        "budget": [int(x) for x in bud],
        "keep_frac": [round(int(x) / wl.L, 5) for x in bud],
        "top1pct_mass": top1,
        "path": args.path,
        "other_path": {"path": other, "ms_per_step": round(other_ms, 4)},
        "dense_ms": None if dense_ms is None else round(dense_ms, 4),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms_step, 4),
        "attention_speedup_vs_dense": None if dense_ms is None else round(dense_ms / steps_ms[attn_step], 4),
        "overhead_share": round(overhead / steps_ms[attn_step], 4),
        "path_kernels_ms": {p: {n: round(steps_ms[n], 4) for n in ks} for p, ks in path_kernels.items()},
        "kernels": kernels,
        "roofline": roofline,
        "readings": readings,
        "block_sparse": block_sparse,
        "stack": stack_rep,
        "sweep": None,
        "provenance": provenance(wl, tau),
        "parity": None,
        "cpu_baseline": None,
    }
    log("[bench] parity check against the oracle")
    out["parity"] = parity_check()
    if not args.no_sweep:
        sweep = []
        for name, taus in [("llama8b_bf16_L8k", (0.05,)), ("llama8b_bf16_L32k_zipf", (0.01, 0.05, 0.1)),
                           ("gqa7_bf16_B2_L64k", (0.1,)), ("llama8b_bf16_L128k_zipf", (0.05, 0.1, 0.2))]:
            log(f"[bench] sweep {name}: generating inputs")
            sweep += sweep_one(name, taus, dev, max(3, min(args.steps, 10)))
        out["sweep"] = sweep
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a bounded sample)")
        out["cpu_baseline"] = cpu_baseline(wl, q, k, v, tau, int(bud[0]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

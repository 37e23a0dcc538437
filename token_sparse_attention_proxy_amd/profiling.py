"""HBM traffic of the kernels from rocprofv3 counters.

Three sub-commands, meant to run under rocprofv3 and after it:

  python -m token_sparse_attention_proxy_amd.profiling run --workload NAME --path P
      Runs, in one process: a plain device-to-device copy of COPY_BYTES
      (calibration), then the attention of one path:
        compact: the attention kernel alone on the compact shape of the
          workload with its measured budget (random bf16 inputs made on the
          GPU; traffic depends on shapes and the budget, not on values);
        fused: tsa_forward_fused on the workload's own seeded inputs (the
          indexed attention's reads follow the real index sets);
        forward: tsa_forward on the workload's own seeded inputs (its
          attention reads Q and writes O through the real index sets);
        all: tsa_forward, then the score, budget, select, gather (Q, K and
          V) and scatter entry points on the same inputs and index sets, so
          that every kernel of the library's 128K op runs on real data.
      Run it twice under ``rocprofv3 --pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``.

  python -m token_sparse_attention_proxy_amd.profiling summarize \\
        --fetch DIR --write DIR --workload NAME --budget K --path P [--out profiles/traffic.json]
      Reads the two counter CSVs, scales each counter by what it reads for
      the copy (bytes moved / counter bytes; the copy is the runtime's
      device-to-device blit kernel), and records the attention
      kernel's HBM bytes per launch, keyed by the kernel source hash, so that
      bench.py reports them only while the kernel is unchanged.

  python -m token_sparse_attention_proxy_amd.profiling summarize-all \\
        --fetch DIR --write DIR --workload NAME [--out profiles/traffic.json]
      The same for every kernel of the library found in the two runs of
      ``run --path all``: the mean counter bytes per dispatch, scaled by the
      copy, keyed by kernel and by the hash of the source file it is built
      from.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ATTN_SRC = os.path.join(ROOT, "token_sparse_attention_proxy_amd", "csrc", "attention.hip")
COPY_BYTES = 1 << 30
# template arguments (IDX, BS, QO) of the attention kernel each path runs
KERNEL_ARGS = {"compact": "false, false, false", "fused": "true, false, false",
               "forward": "false, false, true"}
CSRC = os.path.join(ROOT, "token_sparse_attention_proxy_amd", "csrc")
# source file of each kernel family (the hash keys the recorded counters)
KERNEL_SOURCES = {"score_": "score.hip", "budget_": "budget.hip", "clear_words": "budget.hip",
                  "sel_": "select.hip", "gather_rows": "gather_scatter.hip",
                  "gather_kv_by_rank": "gather_scatter.hip", "scatter_rows": "gather_scatter.hip",
                  "zero_rows": "gather_scatter.hip", "attn_fwd": "attention.hip"}


def step_kernels(d: int, vpr: int) -> dict:
    """Kernels of each step of the op (short names), for head dimension d and vpr 16-byte
    vectors per row."""
    return {
        "score": [f"score_mfma_rowstats<{d}>", "score_merge", f"score_mfma_colsum<{d}>"],
        "budget": ["clear_words", "budget_sigma", "budget_extract_cut"],
        "select": ["sel_clear", "sel_level<0>", "sel_level<1>", "sel_level<2>", "sel_compact"],
        "gather": [f"gather_rows<{vpr}, true, 32>"],
        "gather_kv": [f"gather_kv_by_rank<{vpr}>"],
        "scatter": [f"scatter_rows<{vpr}>"],
        "zero_fill": [f"zero_rows<{vpr}>"],
    }


def kernel_source(kname: str):
    for prefix, src in KERNEL_SOURCES.items():
        if kname.startswith(prefix):
            return os.path.join(CSRC, src)
    return None


def short_name(full: str) -> str:
    """'void tsa::(anonymous namespace)::gather_rows<16, false, 128>(...)' -> 'gather_rows<16, false, 128>'."""
    name = full.strip().replace("(anonymous namespace)", "anon")
    if name.startswith("void "):
        name = name[5:]
    depth = 0
    for i, ch in enumerate(name):          # the argument list: the first '(' outside <>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            name = name[:i]
            break
    return name.split("::")[-1]


def source_sha(path: str = ATTN_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cmd_run(args):
    import torch
    sys.path.insert(0, ROOT)
    from token_sparse_attention_proxy_amd import inputs
    from token_sparse_attention_proxy_amd import tsa as T

    wl = inputs.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.path in ("fused", "forward", "all"):
        q, k, v = inputs.make_qkv(wl)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        qd, kd, vd = (torch.from_numpy(x).to(tdt).to(dev) for x in (q, k, v))
        del q, k, v
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)                       # calibration: COPY_BYTES read, COPY_BYTES written
    torch.cuda.synchronize()
    del src, dst
    tau = wl.taus[0] if args.tau is None else args.tau
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, tau, wl.dtype)
    if args.path == "all":
        o, bud, idx = T.tsa_forward(prob, qd, kd, vd)
        s = torch.empty((wl.B, wl.Hq, wl.L), dtype=torch.float32, device=dev)
        T.tsa_score(prob, qd, kd, s)
        T.tsa_budget(prob, s)            # the entry point alone, with its own clear launch
        _, rank = T.tsa_select(prob, s, bud)
        qc, kc, vc = T.tsa_gather(prob, qd, kd, vd, idx, bud)
        del qc, kc, vc
        oc = torch.zeros_like(o)
        T.tsa_scatter(prob, oc, rank, o)
        torch.cuda.synchronize()
        print(f"ran copy of {COPY_BYTES} B, tsa_forward, score, budget, select, gather and scatter on "
              f"{wl.name}, budget {bud.cpu().tolist()}")
        return
    if args.path in ("fused", "forward"):
        run = T.tsa_forward_fused if args.path == "fused" else T.tsa_forward
        o, bud, idx = run(prob, qd, kd, vd)
        nbytes = (T.fused_workspace_bytes(prob) if args.path == "fused"
                  else T.forward_workspace_bytes(prob))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        for _ in range(args.reps - 1):      # back to back on the same buffers
            run(prob, qd, kd, vd, o, bud, idx, ws)
        torch.cuda.synchronize()
        print(f"ran copy of {COPY_BYTES} B and {run.__name__} x{args.reps} on {wl.name}, "
              f"budget {bud.cpu().tolist()}")
        return
    g = torch.Generator(device=dev).manual_seed(0)
    shape = (wl.B, wl.Hq, wl.L, wl.d)
    q, k, v = (torch.randn(shape, device=dev, generator=g).to(torch.bfloat16) for _ in range(3))
    bud = torch.full((wl.B,), args.budget, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    T.tsa_attention(prob, q, k, v, bud, 1, o)
    torch.cuda.synchronize()
    print(f"ran copy of {COPY_BYTES} B and attention on {shape} with budget {args.budget}")


def _read(dirpath: str, counter: str):
    rows = []
    for f in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {dirpath}")
    return rows


def _pick(rows, needle):
    vals = [v for name, v in rows if needle in name]
    if not vals:
        raise SystemExit(f"no kernel matching {needle!r}")
    return vals


def cmd_summarize(args):
    fetch = _read(args.fetch, "FETCH_SIZE")
    write = _read(args.write, "WRITE_SIZE")
    # the calibration copy is the runtime's device-to-device blit of COPY_BYTES
    copy_f = max(_pick(fetch, "copyBuffer")) * 1024.0
    copy_w = max(_pick(write, "copyBuffer")) * 1024.0
    f_scale = COPY_BYTES / copy_f
    w_scale = COPY_BYTES / copy_w
    kname = f"attn_fwd_bf16<{args.d}, {KERNEL_ARGS[args.path]}>"
    af = _pick(fetch, kname)
    aw = _pick(write, kname)
    fetch_b = sum(af) / len(af) * 1024.0 * f_scale
    write_b = sum(aw) / len(aw) * 1024.0 * w_scale
    entry = {
        "source_sha": source_sha(),
        "path": args.path,
        "budget": args.budget,
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "copy_bytes": COPY_BYTES,
    }
    tab = {}
    if os.path.exists(args.out):
        with open(args.out) as f:
            tab = json.load(f)
    tab.setdefault(kname, {})[args.workload] = entry
    with open(args.out, "w") as f:
        json.dump(tab, f, indent=1, sort_keys=True)
    print(json.dumps(entry, indent=1))


def _per_kernel(rows):
    """{short kernel name: mean counter KiB per dispatch, dispatches}."""
    acc = {}
    for full, val in rows:
        n = short_name(full)
        tot, cnt = acc.get(n, (0.0, 0))
        acc[n] = (tot + val, cnt + 1)
    return {n: (tot / cnt, cnt) for n, (tot, cnt) in acc.items()}


def cmd_summarize_all(args):
    fetch = _read(args.fetch, "FETCH_SIZE")
    write = _read(args.write, "WRITE_SIZE")
    f_scale = COPY_BYTES / (max(_pick(fetch, "copyBuffer")) * 1024.0)
    w_scale = COPY_BYTES / (max(_pick(write, "copyBuffer")) * 1024.0)
    pf, pw = _per_kernel(fetch), _per_kernel(write)
    tab = {}
    if os.path.exists(args.out):
        with open(args.out) as f:
            tab = json.load(f)
    for n in sorted(pf):
        src = kernel_source(n)
        if src is None or n not in pw:
            continue
        fb = pf[n][0] * 1024.0 * f_scale
        wb = pw[n][0] * 1024.0 * w_scale
        entry = {"source_sha": source_sha(src), "source": os.path.basename(src), "path": "all",
                 "dispatches": pf[n][1], "fetch_bytes_per_launch": fb,
                 "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb,
                 "fetch_scale": f_scale, "write_scale": w_scale, "copy_bytes": COPY_BYTES}
        tab.setdefault(n, {})[args.workload] = entry
        print(f"{n:45s} x{pf[n][1]:3d}  fetch {fb / 1e6:10.2f} MB  write {wb / 1e6:10.2f} MB")
    with open(args.out, "w") as f:
        json.dump(tab, f, indent=1, sort_keys=True)


# ---------------------------------------------------------------- markdown summaries
def _bench_line(path):
    """The JSON line a bench.py run printed (its last line that parses)."""
    line = None
    for ln in open(path):
        ln = ln.strip()
        if ln.startswith("{"):
            try:
                line = json.loads(ln)
            except ValueError:
                pass
    if line is None:
        raise SystemExit(f"no bench JSON line in {path}")
    return line


def _first(dirpath, pattern):
    got = sorted(glob.glob(os.path.join(dirpath, "**", pattern), recursive=True))
    if not got:
        raise SystemExit(f"no {pattern} under {dirpath}")
    return got[0]


def _shape_header(wl_name, tau=None):
    sys.path.insert(0, ROOT)
    from token_sparse_attention_proxy_amd import inputs
    wl = inputs.WORKLOADS[wl_name]
    return wl, (f"{wl.name}: B={wl.B}, Hq={wl.Hq}, Hkv={wl.Hkv}, L={wl.L}, d={wl.d}, "
                f"w={wl.w}, tau={wl.taus[0] if tau is None else tau}")


def cmd_trace_summary(args):
    """Kernel trace of a bench.py run: per-kernel statistics of the headline workload's
    dispatches (those before the end of the last dense attention launch on that shape;
    the parity check and the sweep that follow use other shapes)."""
    wl, hdr = _shape_header(args.workload)
    bench = _bench_line(args.bench)
    rows = list(csv.DictReader(open(_first(args.trace, "*kernel_trace.csv"))))
    gx = (wl.L + 255) // 256 * 512
    dense = [r for r in rows if short_name(r["Kernel_Name"]) == f"attn_fwd_bf16<{wl.d}, false, false, false>"
             and int(r["Grid_Size_X"]) == gx and int(r["Grid_Size_Y"]) == wl.B * wl.Hq]
    if not dense:
        raise SystemExit("no dense attention launch of the headline shape in the trace")
    end = max(int(r["End_Timestamp"]) for r in dense)
    # The plain instantiation runs three times over in a bench run: in the per-kernel
    # breakdown (on the compressed tensors, before the MFMA probe), then on operands that
    # barely toggle (the bench line says how many launches), then as the dense baseline.
    plain = f"attn_fwd_bf16<{wl.d}, false, false, false>"
    probe_end = max((int(r["End_Timestamp"]) for r in rows
                     if short_name(r["Kernel_Name"]).startswith("mfma_probe")), default=None)
    n_opdep = int(bench["roofline"].get("operand_dependence", {}).get("launches", 0))
    after_probe = 0
    per = {}
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        n = short_name(r["Kernel_Name"])
        if int(r["Start_Timestamp"]) > end or (kernel_source(n) is None and
                                               not n.startswith("mfma_probe")):
            continue             # torch's own kernels (input copies, fills) are left out
        if n == plain and probe_end is not None:
            if int(r["Start_Timestamp"]) < probe_end:
                n += " (breakdown, compressed tensors)"
            else:
                after_probe += 1
                n += (" (operands that barely toggle)" if after_probe <= n_opdep
                      else " (dense baseline)")
        per.setdefault(n, []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6)
    total = sum(sum(v) for v in per.values())
    out = [f"# Kernel trace: bench.py on the {wl.L // 1024}K workload ({hdr})", "",
           "Command (from the repository root `$R`, on one MI355X):", "", "```",
           args.command, "```", "",
           "Per-kernel durations of every dispatch of the headline workload in that run (the "
           "timed steps, the other path, the per-kernel breakdown, the MFMA ceiling probe, the "
           "compact attention on operands that barely toggle (all ones, then random signs) and "
           "the dense baseline; the parity check and the sweep that follow are left out, and so "
           "are torch's own kernels). `*_kernel_stats.csv` of the same run holds all "
           "dispatches.", "",
           f"The bench line of this run: {bench['value']} ms per layer; "
           f"`roofline.avg_launch_ms` = {bench['roofline']['avg_launch_ms']} ms for "
           f"`{bench['roofline']['kernel']}`, {bench['roofline']['achieved']} TFLOP/s, "
           f"frac {bench['roofline']['frac']}."]
    ceil = bench["roofline"].get("mfma_ceiling")
    if ceil:
        out.append(f"MFMA ceiling probe in the same run: {ceil['random_operands']} TFLOP/s with "
                   f"random operands, {ceil['constant_operands']} with constant operands; the "
                   f"attention is at {ceil['attention_frac_of_random']} of the random-operand rate.")
    out += ["", "| kernel | calls | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|"]
    for n, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{n}` | {len(v)} | {sum(v) / len(v):.4f} | {min(v):.4f} | {max(v):.4f} | "
                   f"{100 * sum(v) / total:.2f}% |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def cmd_op_trace(args):
    """Kernel trace of `run --path forward|fused --reps N`: the op's own kernels in launch
    order, each op instance starting at its first scoring pass; the first instance is left
    out (cold), the others averaged position by position."""
    wl, hdr = _shape_header(args.workload, args.tau)
    rows = sorted(csv.DictReader(open(_first(args.trace, "*kernel_trace.csv"))),
                  key=lambda r: int(r["Start_Timestamp"]))
    rows = [r for r in rows if kernel_source(short_name(r["Kernel_Name"])) is not None]
    first = short_name(rows[0]["Kernel_Name"])
    ops, cur = [], []
    for r in rows:
        if short_name(r["Kernel_Name"]) == first and cur:
            ops.append(cur)
            cur = []
        cur.append(r)
    ops.append(cur)
    if len(ops) < 2:
        raise SystemExit("need at least two op instances (run --reps 2 or more)")
    warm = ops[1:]
    names = [short_name(r["Kernel_Name"]) for r in warm[0]]
    if any([short_name(r["Kernel_Name"]) for r in op] != names for op in warm):
        raise SystemExit("op instances differ in their kernel sequence")
    dur = [[(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in op] for op in warm]
    span = [(int(op[-1]["End_Timestamp"]) - int(op[0]["Start_Timestamp"])) / 1e3 for op in warm]
    steps = {}
    for st, ks in step_kernels(wl.d, wl.d * (2 if wl.dtype == "bf16" else 4) // 16).items():
        for k in ks:
            steps.setdefault(k, st)
    out = [f"# Kernel trace of the op: {wl.L // 1024}K workload ({hdr})", "",
           "Command (from the repository root `$R`, on one MI355X):", "", "```",
           args.command, "```", "",
           f"`profiling.py run --path {args.path} --reps {len(ops)}` runs the op {len(ops)} "
           "times back to back on the same buffers (after the 1 GiB calibration copy). Each "
           "row is one kernel launch of the op, in launch order, averaged over the instances "
           f"after the first ({len(warm)}): its duration from the trace's start and end "
           "timestamps.", "",
           "| # | kernel | step | mean µs | min µs | max µs |", "|---|---|---|---|---|---|"]
    tot_other = 0.0
    per_step = {}
    for i, n in enumerate(names):
        v = [d[i] for d in dur]
        m = sum(v) / len(v)
        step = "attention" if n.startswith("attn_fwd") else steps.get(n, "")
        if n == "score_merge":
            step = "score (+ clears)"
        if n == "sel_compact":
            step = "select (+ zero fill)"
        if not n.startswith("attn_fwd"):
            tot_other += m
        per_step[step.split(" ")[0]] = per_step.get(step.split(" ")[0], 0.0) + m
        out.append(f"| {i + 1} | `{n}` | {step} | {m:.2f} | {min(v):.2f} | {max(v):.2f} |")
    mean_span = sum(span) / len(span)
    attn = per_step.get("attention", 0.0)
    out += ["", "Per step (µs): " + ", ".join(f"{k} {v:.1f}" for k, v in per_step.items()) + ".",
            f"All kernels but the attention: {tot_other:.1f} µs, {100 * tot_other / attn:.2f}% "
            f"of the attention's {attn:.1f} µs. From the first launch's start to the last one's "
            f"end: {mean_span:.1f} µs on average, so the launches follow one another with "
            f"{max(0.0, mean_span - tot_other - attn):.1f} µs between them in all."]
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def cmd_traffic_summary(args):
    """Counter bytes per step (profiles/traffic.json) against the algorithmic bytes and the
    times of a bench.py run on the same workload."""
    wl, hdr = _shape_header(args.workload)
    bench = _bench_line(args.bench)
    tab = json.load(open(args.traffic))
    eb = 2 if wl.dtype == "bf16" else 4
    steps = step_kernels(wl.d, wl.d * eb // 16)
    out = [f"# HBM traffic: every kernel of the {wl.L // 1024}K op ({hdr}, "
           f"K_b={bench['budget'][0]})", "",
           "Commands (from the repository root `$R`, one counter per process):", "", "```",
           args.command, "```", "",
           "`profiling.py run --path all` copies 1 GiB device to device (the runtime blit "
           "`__amd_rocclr_copyBuffer`, the calibration), then runs `tsa_forward`, `tsa_score`, "
           "`tsa_budget`, `tsa_select`, `tsa_gather` (Q, K and V) and `tsa_scatter` on the "
           "workload's own seeded inputs. The blit reads FETCH_SIZE = 0.5 GiB and WRITE_SIZE = 1 GiB for 1 GiB "
           "moved each way, so FETCH_SIZE is scaled by 2 and WRITE_SIZE by 1 "
           "(`profiles/traffic.json` holds the exact factors and each kernel source's hash; "
           "`bench.py` reports these bytes only while the hash matches). Times are the per-kernel "
           f"breakdown of the bench run of {args.bench_label}.", "",
           "| step | kernels | algorithmic bytes | counter bytes (fetch + write) | counter / "
           "algorithmic | ms (bench) | GB/s algorithmic | GB/s counters |",
           "|---|---|---|---|---|---|---|---|"]
    per_kernel = []
    for step, kns in steps.items():
        k = bench["kernels"][step]
        f = sum(tab[n][wl.name]["fetch_bytes_per_launch"] for n in kns)
        w = sum(tab[n][wl.name]["write_bytes_per_launch"] for n in kns)
        alg = k["algorithmic_bytes"]
        out.append(f"| {step} | {', '.join('`' + n + '`' for n in kns)} | {alg / 1e6:.1f} MB | "
                   f"{f / 1e6:.1f} + {w / 1e6:.1f} MB | {(f + w) / alg:.2f} | {k['ms']:.4f} | "
                   f"{alg / (k['ms'] * 1e-3) / 1e9:.0f} | {(f + w) / (k['ms'] * 1e-3) / 1e9:.0f} |")
    out += ["", "Per kernel (mean per dispatch):", "", "| kernel | source | fetch | write |",
            "|---|---|---|---|"]
    for n in sorted(tab):
        e = tab[n].get(wl.name)
        if not e or e.get("path") != "all":
            continue
        out.append(f"| `{n}` | {e.get('source', 'attention.hip')} | "
                   f"{e['fetch_bytes_per_launch'] / 1e6:.2f} MB | {e['write_bytes_per_launch'] / 1e6:.2f} MB |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def cmd_attention_counters(args):
    """FETCH/WRITE bytes of the three attention instantiations and the SQ counters of the
    whole op's attention, with the counted launches' durations."""
    wl, hdr = _shape_header(args.workload)
    K = args.budget
    out = [f"# Counters: attention kernels on the {wl.L // 1024}K workload ({hdr}, K_b={K})", "",
           "Commands (from the repository root `$R`; one counter pass per process):", "", "```",
           args.command, "```", "",
           "`profiling.py run` first copies 1 GiB device to device (the runtime blit kernel "
           "`__amd_rocclr_copyBuffer`, the calibration), then runs `--path forward`: "
           "`tsa_forward` on the workload's own seeded inputs; `--path fused`: "
           "`tsa_forward_fused` on the same inputs; `--path compact`: one `tsa_attention` on "
           "random bf16 tensors of the compact shape with the headline budget.", "",
           "## HBM traffic per launch", "",
           "The blit of 1 GiB reads FETCH_SIZE = 0.5 GiB and WRITE_SIZE = 1 GiB, so FETCH_SIZE is "
           "scaled by 2 and WRITE_SIZE by 1. The write scale is confirmed by the attention "
           f"kernels themselves: they write exactly the output rows, {wl.B * wl.Hq} x {K} x "
           f"{wl.d * 2} B = {wl.B * wl.Hq * K * wl.d * 2 / 1e9:.3f} GB.", "",
           "| kernel | FETCH_SIZE raw (KiB) | fetch bytes | WRITE_SIZE raw (KiB) | write bytes | "
           "total | counted launches |", "|---|---|---|---|---|---|---|"]
    for path in ("forward", "fused", "compact"):
        kname = f"attn_fwd_bf16<{wl.d}, {KERNEL_ARGS[path]}>"
        vals = {}
        for c, d in (("FETCH_SIZE", getattr(args, f"fetch_{path}")),
                     ("WRITE_SIZE", getattr(args, f"write_{path}"))):
            rows = list(csv.DictReader(open(_first(d, "*counter_collection.csv"))))
            copy = max(float(r["Counter_Value"]) for r in rows
                       if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == c)
            att = [r for r in rows if short_name(r["Kernel_Name"]) == kname and r["Counter_Name"] == c]
            raw = sum(float(r["Counter_Value"]) for r in att) / len(att)
            ms = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6 for r in att]
            vals[c] = (raw, raw * COPY_BYTES / (copy * 1024.0) * 1024.0, COPY_BYTES / (copy * 1024.0), ms)
        f, w = vals["FETCH_SIZE"], vals["WRITE_SIZE"]
        out.append(f"| `{kname}` | {f[0]:.0f} | {f[1] / 1e9:.2f} GB (x{f[2]:.4f}) | {w[0]:.0f} | "
                   f"{w[1] / 1e9:.3f} GB (x{w[2]:.2f}) | {(f[1] + w[1]) / 1e9:.2f} GB | "
                   f"{', '.join(f'{m:.2f}' for m in f[3] + w[3])} ms |")
        if path == "forward":
            fwd = (f[1] + w[1], f[1], sum(f[3] + w[3]) / len(f[3] + w[3]))
    alg = 4 * wl.B * wl.Hq * K * wl.d * 2
    flops = 2.0 * wl.d * K * (K + 1) * wl.B * wl.Hq
    out += ["", f"Algorithmic minimum: Q, K, V read once and O written once = 4 x {wl.B * wl.Hq} x "
            f"{K} x {wl.d * 2} B = {alg / 1e9:.2f} GB. About {fwd[1] / 1e9:.0f} GB are fetched because "
            "every workgroup streams all the K/V tiles below its diagonal and part of those re-reads "
            f"miss the L2. For the whole op's attention, at {fwd[2]:.1f} ms per counted launch that is "
            f"{fwd[1] / (fwd[2] * 1e-3) / 1e12:.2f} TB/s, {100 * fwd[1] / (fwd[2] * 1e-3) / 8e12:.1f}% "
            f"of the 8 TB/s HBM bound. The kernel does {flops / fwd[1]:.0f} FLOP per fetched byte "
            "against a ridge of 312: it is MFMA/issue-bound, not memory-bound.", ""]
    rows = list(csv.DictReader(open(_first(args.sq, "*counter_collection.csv"))))
    kname = f"attn_fwd_bf16<{wl.d}, {KERNEL_ARGS['forward']}>"
    att = [r for r in rows if short_name(r["Kernel_Name"]) == kname]
    vals = {r["Counter_Name"]: float(r["Counter_Value"]) for r in att}
    us = (int(att[0]["End_Timestamp"]) - int(att[0]["Start_Timestamp"])) / 1e3
    cyc = vals["GRBM_GUI_ACTIVE"] / args.xcds
    busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * args.cus * 4)
    clk = cyc / (us * 1e-6) / 1e9
    out += ["## SQ counters (the whole op's attention, one launch)", "",
            "Counted in the `--path all` run of `profiling.py` (command in "
            "`kernels_llama8b_L128k_sq.md`, which also lists every other kernel of the op); this "
            f"counted launch ran {us / 1e3:.2f} ms.", "", "| counter | value |", "|---|---|"]
    for c in SQ_COUNTERS:
        out.append(f"| {c} | {vals[c]:.4g} |")
    mf = vals["SQ_INSTS_MFMA"]
    out += ["",
            f"- MFMA pipe busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {args.xcds} XCDs x "
            f"{args.cus * 4} SIMDs) = {busy:.3f}; SQ_INSTS_MFMA = {mf:.4g} against "
            f"{flops / 32768:.4g} for the algorithmic FLOPs ({mf * 32768 / flops:.3f}x).",
            f"- Non-MFMA VALU instructions per MFMA = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / "
            f"SQ_INSTS_MFMA = {(vals['SQ_INSTS_VALU'] - mf) / mf:.2f}.",
            f"- Clock: GRBM_GUI_ACTIVE / {args.xcds} = {cyc:.4g} cycles over the counted "
            f"{us / 1e3:.2f} ms = {clk:.2f} GHz. At that clock the MFMA peak is 2.5 PF x "
            f"{clk:.2f}/2.4 = {2.5 * clk / 2.4:.2f} PF, and {busy:.3f} busy of it is "
            f"{busy * 2.5 * clk / 2.4 * 1000:.0f} TFLOP/s."]
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def cmd_counter_table(args):
    """Every counter of the named kernel from one or more counter runs, with the counted
    launch's duration, raw and per cycle of the launch (GRBM_GUI_ACTIVE / xcds)."""
    wl, hdr = _shape_header(args.workload)
    out = [f"# Counters of `{args.kernel}` on the {wl.L // 1024}K workload ({hdr})", "",
           "Commands (from the repository root `$R`; one pass per process):", "", "```",
           args.command, "```", "", args.note, "",
           "| pass | counter | value | per launch cycle | counted launch ms |",
           "|---|---|---|---|---|"]
    for i, d in enumerate(args.dirs):
        rows = [r for r in csv.DictReader(open(_first(d, "*counter_collection.csv")))
                if short_name(r["Kernel_Name"]) == args.kernel]
        if not rows:
            raise SystemExit(f"no {args.kernel} in {d}")
        vals = {r["Counter_Name"]: float(r["Counter_Value"]) for r in rows}
        ms = (int(rows[0]["End_Timestamp"]) - int(rows[0]["Start_Timestamp"])) / 1e6
        cyc = vals.get("GRBM_GUI_ACTIVE", 0.0) / args.xcds
        for c in sorted(vals):
            per = f"{vals[c] / cyc:.4g}" if cyc else "-"
            out.append(f"| {chr(ord('A') + i)} | {c} | {vals[c]:.4g} | {per} | {ms:.2f} |")
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


SQ_COUNTERS = ["SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
               "SQ_INSTS_LDS", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"]


def cmd_sq_summary(args):
    """SQ counters of every library kernel of a `run --path all` process."""
    wl, hdr = _shape_header(args.workload)
    rows = list(csv.DictReader(open(_first(args.sq, "*counter_collection.csv"))))
    per = {}
    for r in rows:
        n = short_name(r["Kernel_Name"])
        if kernel_source(n) is None:
            continue
        d = per.setdefault(n, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    simds = args.cus * 4
    out = [f"# SQ counters: the kernels of the {wl.L // 1024}K op ({hdr})", "",
           "Command (from the repository root `$R`):", "", "```", args.command, "```", "",
           f"Means per dispatch. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / "
           f"{args.xcds} XCDs x {simds} SIMDs). VALU / MFMA counts the non-MFMA VALU "
           "instructions (SQ_INSTS_VALU includes the MFMAs). For short kernels the counter "
           "window is longer than the kernel, so their busy figures are lower bounds.", "",
           "| kernel | dispatch us (counted) | waves | MFMA busy | VALU / MFMA | VALU instr per wave "
           "| LDS instr per wave |", "|---|---|---|---|---|---|---|"]
    clock = None
    for n in sorted(per, key=lambda k: max(d["us"] for d in per[k].values())):
        ds = list(per[n].values())
        m = {c: sum(d.get(c, 0.0) for d in ds) / len(ds) for c in SQ_COUNTERS + ["us"]}
        cyc = m["GRBM_GUI_ACTIVE"] / args.xcds
        busy = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * simds) if cyc else 0.0
        mf = m["SQ_INSTS_MFMA"]
        ratio = f"{(m['SQ_INSTS_VALU'] - mf) / mf:.2f}" if mf else "no MFMA"
        w = m["SQ_WAVES"] or 1.0
        out.append(f"| `{n}` | {m['us']:.1f} | {m['SQ_WAVES']:.0f} | {busy:.3f} | {ratio} | "
                   f"{m['SQ_INSTS_VALU'] / w:.0f} | {m['SQ_INSTS_LDS'] / w:.0f} |")
        if n.startswith("attn_fwd"):
            clock = (n, m["us"], cyc / (m["us"] * 1e-6) / 1e9, busy, ratio)
    if clock:
        out += ["", f"The `{clock[0]}` launch counted here ran {clock[1] / 1e3:.2f} ms; "
                f"GRBM_GUI_ACTIVE / {args.xcds} over it is a clock of {clock[2]:.2f} GHz, so its "
                f"MFMA pipe was busy {clock[3]:.3f} of the cycles at that clock, with {clock[4]} "
                "non-MFMA VALU instructions per MFMA."]
    open(args.out, "w").write("\n".join(out) + "\n")
    print("\n".join(out))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="llama8b_bf16_L128k")
    r.add_argument("--budget", type=int, default=123997)
    r.add_argument("--path", choices=sorted(KERNEL_ARGS) + ["all"], default="fused")
    r.add_argument("--reps", type=int, default=1, help="op runs (paths fused and forward)")
    r.add_argument("--tau", type=float, default=None, help="default: the workload's first tau")
    r.set_defaults(fn=cmd_run)
    ot = sub.add_parser("op-trace")
    ot.add_argument("--trace", required=True, help="rocprofv3 --kernel-trace output dir")
    ot.add_argument("--workload", default="llama8b_bf16_L128k")
    ot.add_argument("--path", choices=["forward", "fused"], default="forward")
    ot.add_argument("--tau", type=float, default=None, help="the tau the run used")
    ot.add_argument("--command", required=True)
    ot.add_argument("--out", required=True)
    ot.set_defaults(fn=cmd_op_trace)
    s = sub.add_parser("summarize")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--workload", default="llama8b_bf16_L128k")
    s.add_argument("--budget", type=int, default=123997)
    s.add_argument("--path", choices=sorted(KERNEL_ARGS), default="fused")
    s.add_argument("--d", type=int, default=128)
    s.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    s.set_defaults(fn=cmd_summarize)
    a = sub.add_parser("summarize-all")
    a.add_argument("--fetch", required=True)
    a.add_argument("--write", required=True)
    a.add_argument("--workload", default="llama8b_bf16_L128k")
    a.add_argument("--out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    a.set_defaults(fn=cmd_summarize_all)
    t = sub.add_parser("trace-summary")
    t.add_argument("--trace", required=True, help="rocprofv3 --kernel-trace --stats output dir")
    t.add_argument("--bench", required=True, help="the bench.py output of the same run")
    t.add_argument("--workload", default="llama8b_bf16_L128k")
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    t.set_defaults(fn=cmd_trace_summary)
    f = sub.add_parser("traffic-summary")
    f.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"))
    f.add_argument("--bench", required=True, help="a bench.py output on the same workload")
    f.add_argument("--bench-label", default="", help="how the summary names that bench run")
    f.add_argument("--workload", default="llama8b_bf16_L128k")
    f.add_argument("--command", required=True)
    f.add_argument("--out", required=True)
    f.set_defaults(fn=cmd_traffic_summary)
    c = sub.add_parser("attention-counters")
    for path in ("forward", "fused", "compact"):
        c.add_argument(f"--fetch-{path}", required=True)
        c.add_argument(f"--write-{path}", required=True)
    c.add_argument("--sq", required=True)
    c.add_argument("--workload", default="llama8b_bf16_L128k")
    c.add_argument("--budget", type=int, default=123997)
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    c.set_defaults(fn=cmd_attention_counters)
    k = sub.add_parser("counter-table")
    k.add_argument("--dirs", nargs="+", required=True, help="rocprofv3 --pmc output dirs")
    k.add_argument("--kernel", required=True, help="short kernel name")
    k.add_argument("--workload", default="llama8b_bf16_L128k")
    k.add_argument("--xcds", type=int, default=8)
    k.add_argument("--note", default="")
    k.add_argument("--command", required=True)
    k.add_argument("--out", required=True)
    k.set_defaults(fn=cmd_counter_table)
    q = sub.add_parser("sq-summary")
    q.add_argument("--sq", required=True, help="rocprofv3 --pmc SQ_* output dir")
    q.add_argument("--workload", default="llama8b_bf16_L128k")
    q.add_argument("--cus", type=int, default=256)
    q.add_argument("--xcds", type=int, default=8)
    q.add_argument("--command", required=True)
    q.add_argument("--out", required=True)
    q.set_defaults(fn=cmd_sq_summary)
    args = ap.parse_args()
    args.fn(args)


if __name__ == "__main__":
    main()

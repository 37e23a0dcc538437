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
        all: tsa_forward, then the gather of Q, K and V and the scatter
          entry points on the same index sets, so that every kernel of the
          library's 128K op runs once on real data.
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
    prob = T.Problem(wl.B, wl.Hq, wl.Hkv, wl.L, wl.d, wl.w, wl.taus[0], wl.dtype)
    if args.path == "all":
        o, bud, idx = T.tsa_forward(prob, qd, kd, vd)
        s = torch.empty((wl.B, wl.Hq, wl.L), dtype=torch.float32, device=dev)
        _, rank = T.tsa_select(prob, T.tsa_score(prob, qd, kd, s), bud)
        qc, kc, vc = T.tsa_gather(prob, qd, kd, vd, idx, bud)
        del qc, kc, vc
        oc = torch.zeros_like(o)
        T.tsa_scatter(prob, oc, rank, o)
        torch.cuda.synchronize()
        print(f"ran copy of {COPY_BYTES} B, tsa_forward, score, select, gather and scatter on "
              f"{wl.name}, budget {bud.cpu().tolist()}")
        return
    if args.path in ("fused", "forward"):
        run = T.tsa_forward_fused if args.path == "fused" else T.tsa_forward
        o, bud, _ = run(prob, qd, kd, vd)
        torch.cuda.synchronize()
        print(f"ran copy of {COPY_BYTES} B and {run.__name__} on {wl.name}, "
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


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", default="llama8b_bf16_L128k")
    r.add_argument("--budget", type=int, default=123997)
    r.add_argument("--path", choices=sorted(KERNEL_ARGS) + ["all"], default="fused")
    r.set_defaults(fn=cmd_run)
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
    args = ap.parse_args()
    args.fn(args)


if __name__ == "__main__":
    main()

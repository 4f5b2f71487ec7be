"""rocprofv3 helpers: a plain copy kernel for counter calibration, and text
summaries of kernel traces and of HBM traffic counters.

    python -m sparse_moe_decode_amd.profiling copy [--mib 256] [--reps 4]
        runs torch copies of a known size (the calibration kernel for
        FETCH_SIZE / WRITE_SIZE);
    python -m sparse_moe_decode_amd.profiling trace DIR --out FILE --cmd "..."
        summarizes the *_kernel_stats.csv of a `rocprofv3 --kernel-trace
        --stats --output-format csv` run;
    python -m sparse_moe_decode_amd.profiling traffic --fetch DIR --write DIR
        --copy-fetch DIR --copy-write DIR --key KEY --kernels k1,k2,... --out FILE
        [--call-kernel NAME --launches-per-call N]
        turns two counter runs of a workload and two of the copy kernel into
        HBM bytes per call (each listed kernel once per call, or as many times
        as it was dispatched per call, the calls counted by NAME's dispatches)
        and records them, keyed by KEY and the kernel-source hash, in
        profiles/traffic.json;
    python -m sparse_moe_decode_amd.profiling counters DIR --out FILE --cmd "..."
        summarizes every counter of a `rocprofv3 --pmc` run: mean per
        dispatch, by kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def source_sha() -> str:
    """Hash of the kernel sources (names and contents of csrc/)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_decode_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _find(dirpath: str, suffix: str) -> list:
    return sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))


def _short(name: str) -> str:
    n = name.split("(")[0]
    return n.replace("void ", "").strip()


def cmd_copy(args) -> int:
    import torch
    n = args.mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for i in range(args.reps):
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[copy] {i + 1}/{args.reps}: {args.mib} MiB", flush=True)
    return 0


def cmd_trace(args) -> int:
    files = _find(args.dir, "kernel_stats.csv")
    if not files:
        print(f"no kernel_stats.csv under {args.dir}", file=sys.stderr)
        return 1
    rows = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            rows.append(r)
    out = [f"# rocprofv3 kernel statistics: {args.title}", "",
           f"command: {args.cmd}", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | total (ms) | share |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        calls = int(r["Calls"])
        avg = float(r["AverageNs"]) / 1e3
        mn = float(r["MinNs"]) / 1e3
        mx = float(r["MaxNs"]) / 1e3
        tot = float(r["TotalDurationNs"]) / 1e6
        pct = float(r.get("Percentage", 0.0))
        out.append(f"| `{_short(r['Name'])[:90]}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {tot:.2f} | "
                   f"{pct:.1f} % |")
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)
    return 0


def _counter_means(dirpath: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch, by kernel name."""
    files = _find(dirpath, "counter_collection.csv")
    if not files:
        raise SystemExit(f"no counter_collection.csv under {dirpath}")
    acc = defaultdict(lambda: [0.0, 0])
    per_dispatch = defaultdict(float)
    names = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                key = (fn, r.get("Dispatch_Id"))
                per_dispatch[key] += float(r["Counter_Value"])
                names[key] = _short(r["Kernel_Name"])
    for key, v in per_dispatch.items():
        a = acc[names[key]]
        a[0] += v
        a[1] += 1
    return {k: (s / n, n) for k, (s, n) in acc.items()}


def _copy_factor(dirpath: str, counter: str, mib: int) -> float:
    means = _counter_means(dirpath, counter)
    # the copy kernel is the one whose mean is the largest (torch's fill of
    # the source is a write-only kernel)
    best = max(means.items(), key=lambda kv: kv[1][0])
    kib = best[1][0]
    return (mib * 1024.0) / kib, best[0], kib


def cmd_traffic(args) -> int:
    kernels = [k.strip() for k in args.kernels.split(",") if k.strip()]
    fetch = _counter_means(args.fetch, "FETCH_SIZE")
    write = _counter_means(args.write, "WRITE_SIZE")
    ff, fk, fkib = _copy_factor(args.copy_fetch, "FETCH_SIZE", args.copy_mib)
    wf, wk, wkib = _copy_factor(args.copy_write, "WRITE_SIZE", args.copy_mib)
    lines = [f"# HBM traffic from rocprofv3 counters: {args.key}", "",
             f"fetch command: {args.fetch_cmd}", f"write command: {args.write_cmd}",
             f"copy calibration: {args.copy_cmd} ({args.copy_mib} MiB copied)", "",
             f"FETCH_SIZE of the copy kernel `{fk}`: {fkib:.0f} KiB per dispatch -> factor {ff:.4f}",
             f"WRITE_SIZE of the copy kernel `{wk}`: {wkib:.0f} KiB per dispatch -> factor {wf:.4f}", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched bytes (scaled) | written bytes (scaled) |",
             "|---|---|---|---|---|---|"]
    total_f = total_w = 0.0
    per = {}
    calls = None
    if args.call_kernel:
        cm = [n for n in fetch if args.call_kernel in n]
        if not cm:
            raise SystemExit(f"kernel {args.call_kernel} not found in the counter runs")
        calls = sum(fetch[n][1] for n in cm) / args.launches_per_call
    for k in kernels:
        match = [n for n in fetch if k in n]
        matchw = [n for n in write if k in n]
        if not match or not matchw:
            raise SystemExit(f"kernel {k} not found in the counter runs")
        fk_mean = sum(fetch[n][0] * fetch[n][1] for n in match) / sum(fetch[n][1] for n in match)
        wk_mean = sum(write[n][0] * write[n][1] for n in matchw) / sum(write[n][1] for n in matchw)
        nd = sum(fetch[n][1] for n in match)
        ndw = sum(write[n][1] for n in matchw)
        # dispatches of this kernel per call: 1, or counted against the calls
        pf = 1.0 if calls is None else nd / calls
        pw = 1.0 if calls is None else ndw / calls
        fb = fk_mean * 1024.0 * ff * pf
        wb = wk_mean * 1024.0 * wf * pw
        total_f += fb
        total_w += wb
        per[k] = {"fetch_bytes": round(fb), "write_bytes": round(wb), "dispatches": nd, "per_call": round(pf, 3)}
        lines.append(f"| `{k}` | {nd} | {fk_mean:.1f} | {wk_mean:.1f} | {fb:,.0f} | {wb:,.0f} |")
    how = ("each kernel once" if calls is None else
           f"dispatches per call counted against {calls:g} calls ({args.call_kernel} x {args.launches_per_call} per call)")
    lines += ["", f"per call ({how}): fetched {total_f:,.0f} B, written {total_w:,.0f} B, "
                  f"total {total_f + total_w:,.0f} B", f"kernel-source hash: {source_sha()}"]
    text = "\n".join(lines) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    print(text)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = {}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
    rec[args.key] = {"source_sha": source_sha(), "bytes_per_call": round(total_f + total_w),
                     "fetch_bytes_per_call": round(total_f), "write_bytes_per_call": round(total_w),
                     "fetch_factor": round(ff, 5), "write_factor": round(wf, 5), "kernels": per}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    return 0


def cmd_counters(args) -> int:
    files = _find(args.dir, "counter_collection.csv")
    if not files:
        print(f"no counter_collection.csv under {args.dir}", file=sys.stderr)
        return 1
    names = set()
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                names.add(r["Counter_Name"])
    names = sorted(names)
    per = {n: _counter_means(args.dir, n) for n in names}
    kernels = sorted({k for n in names for k in per[n]})
    out = [f"# rocprofv3 counters: {args.title}", "", f"command: {args.cmd}", "",
           "mean value per dispatch", "",
           "| kernel | dispatches | " + " | ".join(names) + " |",
           "|---|---|" + "---|" * len(names)]
    for k in kernels:
        n_disp = max(per[n].get(k, (0, 0))[1] for n in names)
        vals = [f"{per[n][k][0]:,.4g}" if k in per[n] else "-" for n in names]
        out.append(f"| `{k[:80]}` | {n_disp} | " + " | ".join(vals) + " |")
    text = "\n".join(out) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description="rocprofv3 helpers")
    sub = ap.add_subparsers(dest="action", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=256)
    c.add_argument("--reps", type=int, default=4)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--out", default="")
    t.add_argument("--title", default="")
    t.add_argument("--cmd", default="")
    r = sub.add_parser("traffic")
    for a in ("fetch", "write", "copy_fetch", "copy_write"):
        r.add_argument("--" + a.replace("_", "-"), dest=a, required=True)
    r.add_argument("--copy-mib", type=int, default=256)
    r.add_argument("--key", required=True)
    r.add_argument("--kernels", required=True)
    r.add_argument("--out", required=True)
    r.add_argument("--fetch-cmd", default="")
    r.add_argument("--write-cmd", default="")
    r.add_argument("--copy-cmd", default="")
    r.add_argument("--call-kernel", default="",
                   help="calls = dispatches of this kernel / --launches-per-call (default: every kernel once per call)")
    r.add_argument("--launches-per-call", type=int, default=1)
    k = sub.add_parser("counters")
    k.add_argument("dir")
    k.add_argument("--out", default="")
    k.add_argument("--title", default="")
    k.add_argument("--cmd", default="")
    args = ap.parse_args(argv)
    return {"copy": cmd_copy, "trace": cmd_trace, "traffic": cmd_traffic, "counters": cmd_counters}[args.action](args)


if __name__ == "__main__":
    sys.exit(main())

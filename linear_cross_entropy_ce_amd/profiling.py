"""rocprofv3 helpers for the figures bench.py reports.

    python -m linear_cross_entropy_ce_amd.profiling copy [--mib 1024] [--reps 3]
        Runs a plain elementwise copy of known size: ``torch.neg`` of one fp32
        buffer into another, each MIB MiB.  Profiled with ``--pmc FETCH_SIZE``
        and ``--pmc WRITE_SIZE`` it calibrates those counters: every dispatch
        reads and writes exactly MIB MiB.

    python -m linear_cross_entropy_ce_amd.profiling traffic \\
            --fetch F.csv --write W.csv --copy-fetch CF.csv --copy-write CW.csv \\
            --copy-mib 1024 --workload NAME --out profiles [--command "..."]
        Averages the per-dispatch FETCH_SIZE and WRITE_SIZE (KiB) of every
        library kernel, scales each counter by the copy's known bytes over
        its counted bytes, and writes ``<kernel>_<NAME>_traffic.json`` per
        kernel plus one markdown table.  Each JSON carries the digest of the
        kernel sources it was measured on; bench.py ignores a figure whose
        digest no longer matches.

    python -m linear_cross_entropy_ce_amd.profiling stats --csv K.csv \\
            --title "..." --command "..." --out FILE.md
        Formats a ``--kernel-trace --stats`` kernel_stats.csv as markdown with
        the library's kernel names.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")


def source_digest() -> str:
    """First 16 hex digits of a SHA-256 over the kernel sources."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_key(name: str) -> str | None:
    """Map a (mangled or demangled) kernel name to the library's timer name."""
    if "k_bwd_grad" in name:
        # template flag A_KMAJOR: false for dW (A = dZ^T), true for dX (A = dZ)
        if "Lb0E" in name or "false>" in name:
            return "bwd_dw"
        if "Lb1E" in name or "true>" in name:
            return "bwd_dx"
        return None
    for k in ("fwd_lse", "bwd_dz", "lse_merge", "loss_final", "label_scan", "fill_zero"):
        if f"k_{k}" in name:
            return k
    return None


def _rows(path):
    with open(path, newline="") as f:
        yield from csv.DictReader(f)


def per_dispatch(path: str, counter: str, key=kernel_key):
    """{kernel: [counter value per dispatch]} from a counter_collection.csv.
    Counters reported per shader engine or channel are summed per dispatch."""
    acc = defaultdict(lambda: defaultdict(float))
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        k = key(r["Kernel_Name"])
        if k is None:
            continue
        acc[k][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: list(v.values()) for k, v in acc.items()}


def _copy_kib(path: str, counter: str) -> float:
    """Average counter value over the calibration copy's dispatches."""
    d = per_dispatch(path, counter, key=lambda n: "copy" if "neg" in n else None)
    vals = d.get("copy", [])
    if not vals:
        raise SystemExit(f"{path}: no neg (copy) dispatch found")
    return sum(vals) / len(vals)


def cmd_copy(args):
    import torch

    n = args.mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"copy: {args.reps} x neg over {args.mib} MiB fp32 -> {args.mib} MiB", flush=True)


def cmd_traffic(args):
    known = args.copy_mib * (1 << 20)
    cf = known / (_copy_kib(args.copy_fetch, "FETCH_SIZE") * 1024.0)
    cw = known / (_copy_kib(args.copy_write, "WRITE_SIZE") * 1024.0)
    fetch = per_dispatch(args.fetch, "FETCH_SIZE")
    write = per_dispatch(args.write, "WRITE_SIZE")
    digest = source_digest()
    os.makedirs(args.out, exist_ok=True)
    lines = [f"# HBM traffic per dispatch, {args.workload}", "",
             f"Kernel sources digest: `{digest}`.", "",
             "Commands (on the MI355X box, from the repository root, with "
             "`cd /tmp && export TMPDIR=/tmp` first):", ""]
    lines += [f"    {c}" for c in (args.command or [])]
    lines += ["", f"Counter calibration: `torch.neg` over {args.copy_mib} MiB fp32 reads and "
              f"writes exactly {known} bytes per dispatch; FETCH_SIZE is scaled by "
              f"{cf:.4f} and WRITE_SIZE by {cw:.4f}.", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) |",
              "|:--|--:|--:|--:|--:|"]
    for k in sorted(set(fetch) & set(write)):
        f = sum(fetch[k]) / len(fetch[k])
        w = sum(write[k]) / len(write[k])
        hbm = f * 1024.0 * cf + w * 1024.0 * cw
        rec = {"kernel": k, "workload": args.workload, "source_sha256": digest,
               "dispatches": len(fetch[k]), "fetch_kib_per_dispatch": f,
               "write_kib_per_dispatch": w, "fetch_factor": cf, "write_factor": cw,
               "hbm_bytes_per_launch": round(hbm), "copy_calibration_bytes": known,
               "commands": args.command or []}
        with open(os.path.join(args.out, f"{k}_{args.workload}_traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        lines.append(f"| {k} | {len(fetch[k])} | {f:,.1f} | {w:,.1f} | {hbm:,.0f} |")
    with open(os.path.join(args.out, f"fce_kernels_{args.workload}_traffic.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_stats(args):
    rows = list(_rows(args.csv))
    out = [f"# {args.title}", "", "Command (on the MI355X box, from the repository root, with "
           "`cd /tmp && export TMPDIR=/tmp` first):", ""]
    out += [f"    {c}" for c in (args.command or [])]
    out += ["", "| kernel | calls | total ms | average us | min us | max us | % |",
            "|:--|--:|--:|--:|--:|--:|--:|"]
    def col(r, *names):
        for n in names:
            for key in r:
                if key.lower().replace("_", "") == n:
                    return r[key]
        raise SystemExit(f"{args.csv}: no column among {names}; have {list(r)}")

    for r in rows:
        name = col(r, "name", "kernelname")
        k = kernel_key(name) or name[:60]
        out.append(f"| {k} | {col(r, 'calls')} | "
                   f"{float(col(r, 'totaldurationns', 'durationns')) / 1e6:.3f} | "
                   f"{float(col(r, 'averagens')) / 1e3:.1f} | {float(col(r, 'minns')) / 1e3:.1f} | "
                   f"{float(col(r, 'maxns')) / 1e3:.1f} | {float(col(r, 'percentage')):.2f} |")
    if args.notes:
        out += [""] + args.notes
    with open(args.out, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m linear_cross_entropy_ce_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--command", action="append")
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--command", action="append")
    s.add_argument("--notes", action="append")
    args = ap.parse_args(argv)
    {"copy": cmd_copy, "traffic": cmd_traffic, "stats": cmd_stats}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())

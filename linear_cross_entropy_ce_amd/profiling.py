"""rocprofv3 helpers for the figures bench.py reports.

    python -m linear_cross_entropy_ce_amd.profiling copy [--mib 1024] [--reps 3]
        Runs a plain elementwise copy of known size: ``torch.neg`` of one fp32
        buffer into another, each MIB MiB.  Profiled with ``--pmc FETCH_SIZE``
        and ``--pmc WRITE_SIZE`` it calibrates those counters: every dispatch
        reads and writes exactly MIB MiB.

    python -m linear_cross_entropy_ce_amd.profiling ce [--n 8192 --v 128256 --reps 5]
        Runs the loss on given logits (dZ into another buffer) on seeded bf16
        logits of that shape, for a kernel trace or counter pass of its own.

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
import re
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


def _flags(name: str) -> list[bool]:
    """The bool template arguments of a kernel, in order (mangled Lb0E /
    Lb1E, or demangled false / true after the tile configuration)."""
    m = re.findall(r"Lb([01])E", name)
    if m:
        return [f == "1" for f in m]
    tail = name.split(">,", 1)[-1]
    return [w == "true" for w in re.findall(r"\b(true|false)\b", tail)]


def kernel_key(name: str) -> str | None:
    """Map a (mangled or demangled) kernel name to the library's timer name."""
    if "k_bwd_grad_pair" in name:
        # both gradient products of a logit block in one launch
        return "bwd_grad"
    if "k_bwd_grad" in name:
        # flags A_KMAJOR, FILTER, TRANS: dX has a K-major A (dZ); dW has an
        # M-major one (dZ^T), or is the transposed product X^T dZ (TRANS)
        f = _flags(name)
        if not f:
            return None
        return "bwd_dw" if (len(f) > 2 and f[2]) or not f[0] else "bwd_dx"
    if "k_transpose_x" in name:
        return "x_transpose"
    if "k_fwd_lse" in name:
        # flags SMOOTH, STORE: the storing forward is the store-logits variant's
        f = _flags(name)
        return "sl_fwd" if len(f) > 1 and f[1] else "fwd_lse"
    for k in ("bwd_dz", "lse_merge", "loss_final", "label_scan", "fill_zero", "ce_logits",
              "dx_reduce", "filter_lists"):
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


def cmd_ce(args):
    """The loss on given logits, dZ into another buffer, on seeded bf16
    logits N(0, sigma^2) of the 8192 x 128256 logit shape."""
    import torch

    import linear_cross_entropy_ce_amd as fce

    fce.load_library()
    g = torch.Generator(device="cuda")
    g.manual_seed(args.seed)
    Z = (torch.randn((args.n, args.v), generator=g, device="cuda") * args.sigma).to(torch.bfloat16)
    y = torch.randint(0, args.v, (args.n,), generator=g, device="cuda", dtype=torch.int32)
    dZ = torch.empty_like(Z)
    loss = torch.empty(1, device="cuda")
    lse = torch.empty(args.n, device="cuda")
    ws = torch.empty(fce.fce_ce_logits_workspace_size(args.n), dtype=torch.uint8, device="cuda")
    for _ in range(args.reps):
        fce.fce_ce_logits(Z, y, loss, lse, ws, dZ=dZ)
    torch.cuda.synchronize()
    print(f"ce_logits: {args.reps} calls on {args.n} x {args.v} bf16 logits, loss {loss.item():.5f}",
          flush=True)


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


def cmd_counters(args):
    """Per-kernel averages per dispatch of every counter in a
    counter_collection.csv, as markdown, with derived ratios where the
    counters for them are present."""
    names = []
    for r in _rows(args.csv):
        if r["Counter_Name"] not in names:
            names.append(r["Counter_Name"])
    per = {n: per_dispatch(args.csv, n) for n in names}
    kernels = sorted({k for d in per.values() for k in d})
    # durations of the same dispatches from a kernel trace of the same run
    dur = {}
    if getattr(args, "trace", None):
        by_id = {}
        for r in _rows(args.trace):
            by_id[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        ids = defaultdict(set)
        for r in _rows(args.csv):
            k = kernel_key(r["Kernel_Name"])
            if k is not None and r["Dispatch_Id"] in by_id:
                ids[k].add(r["Dispatch_Id"])
        for k, s_ in ids.items():
            dur[k] = sum(by_id[i] for i in s_) / len(s_)
    out = [f"# {args.title}", "", "Commands (on the MI355X box, from the repository root, with "
           "`cd /tmp && export TMPDIR=/tmp` first):", ""]
    out += [f"    {c}" for c in (args.command or [])]
    out += ["", "Average per dispatch (counters summed over shader engines).", "",
            "| kernel | dispatches | " + " | ".join(names) + " |",
            "|:--|--:|" + "--:|" * len(names)]
    derived = []
    for k in kernels:
        avg = {n: (sum(per[n][k]) / len(per[n][k]) if per[n].get(k) else float("nan"))
               for n in names}
        ndisp = max(len(per[n].get(k, [])) for n in names)
        out.append(f"| {k} | {ndisp} | " + " | ".join(f"{avg[n]:,.0f}" for n in names) + " |")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "SQ_BUSY_CYCLES" in avg:
            # SQ_BUSY_CYCLES is summed over the 32 shader engines, the MFMA
            # busy cycles over the 1024 SIMDs (32 per engine): their ratio over
            # 32 is the fraction of busy cycles each SIMD's matrix pipe worked.
            # Over a dispatch's duration, SQ_BUSY_CYCLES / 32 gives the clock.
            busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / max(32.0 * avg["SQ_BUSY_CYCLES"], 1)
            conf = (f"{avg['SQ_LDS_BANK_CONFLICT'] / max(avg.get('SQ_INSTS_LDS', 1), 1):.4f}"
                    if "SQ_LDS_BANK_CONFLICT" in avg else "")
            if k in dur:
                clk = avg["SQ_BUSY_CYCLES"] / 32.0 / dur[k] / 1e9
                derived.append(f"| {k} | {dur[k] * 1e6:,.1f} | {clk:.3f} | {busy:.3f} | "
                               f"{busy * clk / 2.4:.3f} | {conf} |")
            else:
                derived.append(f"| {k} | | | {busy:.3f} | | {conf} |")
    if derived:
        out += ["", "| kernel | duration us | clock GHz | MFMA busy fraction per SIMD | "
                "busy x clock / 2.4 GHz (fraction of dense peak) | LDS bank-conflict cycles per "
                "LDS instruction |", "|:--|--:|--:|--:|--:|--:|"] + derived
    if args.notes:
        out += [""] + args.notes
    with open(args.out, "w") as fh:
        fh.write("\n".join(out) + "\n")
    print("\n".join(out))


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
    e = sub.add_parser("ce")
    e.add_argument("--n", type=int, default=8192)
    e.add_argument("--v", type=int, default=128256)
    e.add_argument("--sigma", type=float, default=1.28)
    e.add_argument("--seed", type=int, default=7)
    e.add_argument("--reps", type=int, default=5)
    t = sub.add_parser("traffic")
    for a in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--workload", "--out"):
        t.add_argument(a, required=True)
    t.add_argument("--copy-mib", type=int, default=1024)
    t.add_argument("--command", action="append")
    n = sub.add_parser("counters")
    n.add_argument("--csv", required=True)
    n.add_argument("--title", required=True)
    n.add_argument("--out", required=True)
    n.add_argument("--command", action="append")
    n.add_argument("--notes", action="append")
    n.add_argument("--trace", help="kernel_trace.csv of the same run (durations, clock)")
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--command", action="append")
    s.add_argument("--notes", action="append")
    args = ap.parse_args(argv)
    {"copy": cmd_copy, "ce": cmd_ce, "traffic": cmd_traffic, "counters": cmd_counters,
     "stats": cmd_stats}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())

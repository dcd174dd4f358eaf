"""Benchmark of the fused linear cross-entropy forward+backward on one MI355X.

One step = one fce_fused_fwd_bwd call over one synthetic batch (label scan,
forward logit tiles with the on-chip LSE reduction, LSE merge and loss, then
the backward recompute, dW and dX products for every logit block).  Inputs
and outputs are resident in device memory before the timed region.

Besides the headline step it times, outside the headline figure: the
forward and backward entry points on their own, the same step at the other
chunk sizes and with the token-chunk schedule, and (as context) a naive
torch step that materialises the logits.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload 3]
                    [--chunk 1024] [--schedule auto] [--cpu-sample-tokens 0]
                    [--sweep-chunks 256,512] [--no-naive] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2516.6, "fp32": 157.3}  # MI355X dense MFMA TFLOP/s (256 CUs x 2.4 GHz)
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def read_traffic(kernel: str, workload: str, launches_per_step: float):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 PMC
    summary, or None when it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    from linear_cross_entropy_ce_amd.profiling import source_digest

    if rec.get("source_sha256") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


# fp64 FLOPs the CPU baseline may execute by default (about 30 s on 16 host
# cores): the whole 8192 x 4096 x 128256 workload (25.8 TFLOP) fits, larger
# workloads take their first tokens
CPU_BUDGET_FLOPS = 30e12


def cpu_tokens(wl, requested: int) -> int:
    """Tokens of the CPU baseline: ``requested`` if positive, else the whole
    workload when its 6NVH fp64 FLOPs fit CPU_BUDGET_FLOPS, else the most
    whole 256-token tiles that do."""
    if requested > 0:
        return min(requested, wl.N)
    per_token = 6.0 * wl.V * wl.H
    if per_token * wl.N <= CPU_BUDGET_FLOPS:
        return wl.N
    return max(256, int(CPU_BUDGET_FLOPS / per_token) // 256 * 256)


def cpu_baseline(wl, inp, n_tokens: int):
    """The fp64 oracle as it stands, on the first n_tokens rows of the same
    workload (full vocabulary and hidden size; all rows: one full oracle
    call)."""
    import oracle.fce_oracle as orc
    import workloads as wk

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    n = min(n_tokens, wl.N)
    X, y = inp.X[:n], inp.labels[:n]
    t0 = time.perf_counter()
    last = [t0]

    def progress(done, total):  # a line every 20 s of a long call
        now = time.perf_counter()
        if now - last[0] >= 20.0:
            last[0] = now
            log(f"  oracle: {done} of {total} valid rows, {now - t0:.0f} s")

    orc.linear_cross_entropy(X, inp.W, y, wk.IGNORE_INDEX, wl.label_smoothing, "mean",
                             progress=progress)
    dt = time.perf_counter() - t0
    what = (f"one full oracle call on all {n} tokens of {wl.name}" if n == wl.N else
            f"first {n} of {wl.N} tokens of {wl.name}")
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 2), "cpu_model": model,
            "sample": f"{what} (full V={wl.V}, H={wl.H}): loss, dX and dW in fp64 numpy on "
                      f"{model}, {6 * n * wl.V * wl.H / 1e12:.2f} TFLOP executed in {dt:.1f} s"}


def time_steps(torch, fn, steps, stream):
    """Total and per-step milliseconds of ``steps`` calls, from events on ``stream``."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[-1]), per


def naive_torch(torch, X, W, y, eps, steps):
    """Context only: logits materialised by a torch GEMM, torch's cross-entropy
    in fp32, autograd backward.  Time per step and peak bytes above the inputs."""
    import torch.nn.functional as F

    Xp = X.detach().clone().requires_grad_(True)
    Wp = W.detach().clone().requires_grad_(True)
    y64 = y.long()

    def step():
        Xp.grad = None
        Wp.grad = None
        z = Xp @ Wp.t()
        loss = F.cross_entropy(z.float(), y64, ignore_index=-100, label_smoothing=eps)
        loss.backward()

    step()
    torch.cuda.synchronize()
    Xp.grad = None
    Wp.grad = None
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    total, per = time_steps(torch, step, steps, torch.cuda.current_stream())
    peak = torch.cuda.max_memory_allocated() - base
    del Xp, Wp
    torch.cuda.empty_cache()
    return {"what": "torch GEMM X @ W^T (bf16) + F.cross_entropy on fp32 logits + autograd; context only",
            "ms_per_step": round(total / steps, 3), "steps": steps,
            "peak_bytes_above_inputs": int(peak)}


def run_side(torch, fce, wk, args, side, X, W, y, loss, lse, dX, dW, ws, step, stream, ms):
    """Measurements outside the headline figure: the forward and backward entry
    points alone, the step at other chunk sizes and with the token-chunk
    schedule, and the naive torch step (context)."""
    N, H = X.shape
    V = W.shape[0]
    chunk, sched, eps = args.chunk, args.schedule, wk.WORKLOADS[args.workload].label_smoothing
    k2 = args.side_steps
    fwd = lambda: fce.fce_forward(X, W, y, loss, lse, ws, wk.IGNORE_INDEX, eps, "mean", chunk, sched)
    bwd = lambda: fce.fce_backward(X, W, y, lse, None, dX, dW, ws, wk.IGNORE_INDEX, eps, "mean",
                                   chunk, sched)
    fwd()
    bwd()
    t_f, _ = time_steps(torch, fwd, k2, stream)
    t_b, _ = time_steps(torch, bwd, k2, stream)
    side["fce_forward"] = {"ms": round(t_f / k2, 4), "tflops_2NVH": round(2 * N * V * H / (t_f / k2 / 1e3) / 1e12, 1)}
    side["fce_backward"] = {"ms": round(t_b / k2, 4), "tflops_6NVH": round(6 * N * V * H / (t_b / k2 / 1e3) / 1e12, 1)}
    log(f"  forward alone {t_f / k2:.3f} ms, backward alone {t_b / k2:.3f} ms")
    sweep = {str(chunk) + "/" + sched: round(ms, 4)}
    variants = [(int(c), sched) for c in args.sweep_chunks.split(",") if c and int(c) != chunk]
    if sched != "token":
        variants.append((chunk, "token"))
    for c, sc in variants:
        ws_c = fce.workspace_for(N, H, V, X.dtype, c, sc)
        fn = lambda: step(ws_c, c, sc)
        fn()
        t_c, _ = time_steps(torch, fn, k2, stream)
        sweep[f"{c}/{sc}"] = round(t_c / k2, 4)
        log(f"  chunk {c} schedule {sc}: {t_c / k2:.3f} ms/step")
        del ws_c
    side["ms_per_step_by_chunk_schedule"] = sweep
    side["store_logits"] = store_logits_side(torch, fce, wk, args, X, W, y, loss, dX, dW, eps,
                                             stream)
    side["filtered"] = filtered_side(torch, fce, wk, args, X, W, y, loss, dX, dW, eps, stream)
    side["ce_logits"] = ce_logits_side(torch, fce, wk, args, X, W, y, eps, stream)
    if not args.no_naive:
        try:
            side["naive_torch"] = naive_torch(torch, X, W, y, eps, min(k2, 5))
            log(f"  naive torch: {side['naive_torch']}")
        except torch.cuda.OutOfMemoryError as e:  # pragma: no cover
            side["naive_torch"] = {"error": str(e)[:200]}
        try:
            side["vendor_gemms"] = vendor_gemms(torch, X, W, min(k2, 5))
            log(f"  vendor GEMMs: {side['vendor_gemms']}")
        except torch.cuda.OutOfMemoryError as e:  # pragma: no cover
            side["vendor_gemms"] = {"error": str(e)[:200]}


def vendor_gemms(torch, X, W, steps):
    """Context only: the step's three GEMM shapes through torch (hipBLASLt,
    bf16 in and out, no epilogue): logits X W^T (the forward, and the
    backward's recompute), dX = dZ W and dW = dZ^T X, with a stand-in dZ of
    small random values.  Their sum, with the logits GEMM twice, is what the
    vendor library takes for the step's 8NVH without any loss arithmetic."""
    N, H = X.shape
    V = W.shape[0]
    g = torch.Generator(device=X.device).manual_seed(5)
    dZ = (torch.randn(N, V, device=X.device, generator=g) * 1e-4).to(torch.bfloat16)
    dZt = dZ.t().contiguous()
    Wt = W.t().contiguous()
    out = {"what": "torch mm (hipBLASLt), bf16 in and out, same shapes; context only"}
    shapes = {"logits_XWt": lambda: torch.mm(X, Wt),
              "dX_dZW": lambda: torch.mm(dZ, W),
              "dW_dZtX": lambda: torch.mm(dZt, X)}
    stream = torch.cuda.current_stream()
    total = 0.0
    for name, fn in shapes.items():
        fn()
        t, _ = time_steps(torch, fn, steps, stream)
        ms = t / steps
        out[name] = {"ms": round(ms, 4), "tflops": round(2.0 * N * V * H / (ms / 1e3) / 1e12, 1)}
        total += ms * (2 if name == "logits_XWt" else 1)
    out["four_gemm_ms"] = round(total, 4)
    out["four_gemm_tflops_8NVH"] = round(8.0 * N * V * H / (total / 1e3) / 1e12, 1)
    del dZ, dZt, Wt
    torch.cuda.empty_cache()
    return out


def store_logits_side(torch, fce, wk, args, X, W, y, loss, dX, dW, eps, stream):
    """The store-logits variant of the fused step (each chunk's logits kept
    in the workspace and overwritten by dZ; 6NVH executed FLOPs) at two chunk
    sizes: the whole batch in one chunk, and the default chunk."""
    N, H = X.shape
    V = W.shape[0]
    k2 = args.side_steps
    res = {"what": "store-logits fused step: executed FLOPs 6NVH (no recompute); tokens/s "
                   "comparable with the headline, TFLOP/s counted on 6NVH"}
    for chunk in sorted({N, args.chunk}, reverse=True):
        opts = dict(ignore_index=wk.IGNORE_INDEX, label_smoothing=eps, chunk=chunk,
                    variant="store_logits")
        ws = fce.workspace_for(N, H, V, X.dtype, **opts)
        fn = lambda: fce.fce_fused_fwd_bwd_ex(X, W, y, loss, dX, dW, ws, **opts)
        fn()
        fce.fce_timing_enable(True)
        t, per = time_steps(torch, fn, k2, stream)
        kern = fce.fce_timing_read()
        fce.fce_timing_enable(False)
        ms = t / k2
        res[f"chunk_{chunk}"] = {
            "ms_per_step": round(ms, 4), "tokens_per_s": round(N / (ms / 1e3), 1),
            "tflops_6NVH": round(6.0 * N * V * H / (ms / 1e3) / 1e12, 1),
            "workspace_bytes": int(ws.numel()),
            "kernels_ms_per_step": {k: round(r["total_ms"] / k2, 4) for k, r in kern.items()}}
        log(f"  store-logits chunk {chunk}: {ms:.3f} ms/step, workspace {ws.numel() / 1e9:.2f} GB, "
            f"{res[f'chunk_{chunk}']['kernels_ms_per_step']}")
        del ws
        torch.cuda.empty_cache()
    return res


def filtered_side(torch, fce, wk, args, X, W, y, loss, dX, dW, eps, stream):
    """Gradient filtering (an approximation): the filtered step against the
    exact one on the same inputs, with the kept-tile fraction and the
    gradients' deviation from the exact ones.  On this workload's logits and
    on a flatter version of them (W scaled by 1/4), where most tiles hold only
    softmax values below 2^-12."""
    N, H = X.shape
    V = W.shape[0]
    k2 = args.side_steps
    res = {"what": "filtered (CCE) vs exact recompute step; error = relative L2 of the "
                   "filtered dX, dW against the exact ones on the same inputs"}
    dX2, dW2 = torch.empty_like(dX), torch.empty_like(dW)
    for name, Wc in (("workload", W), ("flat_logits_W_x0.25", W * 0.25)):
        times = {}
        for variant, gx, gw in (("recompute", dX, dW), ("filtered", dX2, dW2)):
            opts = dict(ignore_index=wk.IGNORE_INDEX, label_smoothing=eps, chunk=args.chunk,
                        variant=variant)
            ws = fce.workspace_for(N, H, V, X.dtype, **opts)
            fn = lambda: fce.fce_fused_fwd_bwd_ex(X, Wc, y, loss, gx, gw, ws, **opts)
            fn()
            fce.fce_timing_enable(True)
            t, _ = time_steps(torch, fn, k2, stream)
            kern = fce.fce_timing_read()
            fce.fce_timing_enable(False)
            times[variant] = t / k2
            if variant == "filtered":
                kept, total = fce.fce_get_filter_stats(ws)
                kms = {k: round(r["total_ms"] / k2, 4) for k, r in kern.items()}
            del ws
        ex = ((dX2.double() - dX.double()).norm() / dX.double().norm()).item()
        ew = ((dW2.double() - dW.double()).norm() / dW.double().norm()).item()
        res[name] = {"ms_exact": round(times["recompute"], 4),
                     "ms_filtered": round(times["filtered"], 4),
                     "speedup": round(times["recompute"] / times["filtered"], 3),
                     "kept_tiles": kept, "all_tiles": total, "filtered_kernels_ms": kms,
                     "dX_rel_l2_vs_exact": ex, "dW_rel_l2_vs_exact": ew}
        log(f"  filtered [{name}]: {res[name]}")
    del dX2, dW2
    torch.cuda.empty_cache()
    return res


def ce_logits_side(torch, fce, wk, args, X, W, y, eps, stream):
    """The loss on logits the caller holds (fce_ce_logits) on this workload's
    own logits Z = X W^T (made by a torch GEMM outside the timed region):
    dZ into another buffer, dZ over Z, and the loss alone.  HBM-bound; the
    algorithmic bytes are one read of Z plus, with a gradient, one write."""
    N, V = X.shape[0], W.shape[0]
    Z = X @ W.t()
    esz = Z.element_size()
    dZ = torch.empty_like(Z)
    loss = torch.empty(1, device="cuda")
    lse = torch.empty(N, device="cuda")
    ws = torch.empty(fce.fce_ce_logits_workspace_size(N), dtype=torch.uint8, device="cuda")
    k2 = args.side_steps
    res = {"what": f"loss on given {N}x{V} logits ({str(Z.dtype).split('.')[-1]}), "
                   "one workgroup per row, two streaming passes", "peak_GBps": HBM_PEAK_GBS}
    Zc = Z.clone()
    modes = {"separate_dZ": (dZ, 2), "loss_only": (None, 1), "in_place_dZ": (Zc, 2)}
    for name, (out, passes) in modes.items():
        src = Zc if name == "in_place_dZ" else Z
        fn = lambda: fce.fce_ce_logits(src, y, loss, lse, ws, dZ=out, ignore_index=wk.IGNORE_INDEX,
                                       label_smoothing=eps)
        fn()
        fce.fce_timing_enable(True)
        t, _ = time_steps(torch, fn, k2, stream)
        kt = fce.fce_timing_read().get("ce_logits")
        fce.fce_timing_enable(False)
        kms = kt["total_ms"] / kt["launches"] if kt else t / k2
        nbytes = passes * N * V * esz
        gbps = nbytes / (kms / 1e3) / 1e9
        res[name] = {"ms": round(kms, 4), "algorithmic_bytes": nbytes, "GBps": round(gbps, 1),
                     "frac": round(gbps / HBM_PEAK_GBS, 4)}
        log(f"  ce_logits {name}: {kms:.3f} ms, {gbps:.0f} GB/s ({100 * gbps / HBM_PEAK_GBS:.1f}%)")
    del Z, Zc, dZ
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--chunk", type=int, default=1024)
    ap.add_argument("--schedule", default="auto", choices=["auto", "token", "vocab"])
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens of the CPU oracle baseline (0: the whole workload if it fits "
                         "about 30 s of host time, else the first tokens that do)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-chunks", default="256,512")
    ap.add_argument("--side-steps", type=int, default=10)
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--no-side", action="store_true",
                    help="only the headline step (no forward/backward alone, sweeps or naive run)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import linear_cross_entropy_ce_amd as fce
    import workloads as wk

    fce.load_library()
    wl = wk.WORKLOADS[args.workload]
    log(f"drawing inputs for {wl.name} (N={wl.N}, H={wl.H}, V={wl.V}, {wl.dtype})")
    inp = wk.draw(wl)
    X, W, y = wk.to_torch(inp, "cuda")
    N, H, V = wl.N, wl.H, wl.V
    chunk, sched = args.chunk, args.schedule
    plan = fce.fce_plan(N, H, V, fce.FCE_BF16 if wl.dtype == "bf16" else fce.FCE_F32, chunk,
                        fce.SCHEDULES[sched])
    log(f"plan: {plan}")
    base_alloc = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ws = fce.workspace_for(N, H, V, X.dtype, chunk, sched)
    loss = torch.empty(1, device="cuda")
    lse = torch.empty(N, device="cuda")
    dX = torch.empty((N, H), device="cuda")
    dW = torch.empty((V, H), device="cuda")
    out_bytes = 4 * (1 + N + N * H + V * H)
    eps = wl.label_smoothing
    stream = torch.cuda.current_stream()

    def step(ws=ws, chunk=chunk, sched=sched):
        fce.fce_fused_fwd_bwd(X, W, y, loss, dX, dW, ws, wk.IGNORE_INDEX, eps, "mean", chunk, sched)

    # the warmup runs as the timed steps do, with the library's kernel timer
    # on (its first timed call has one-time costs); its records are dropped
    fce.fce_timing_enable(True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    fce.fce_timing_read()
    # everything the step allocated beyond inputs and outputs: the workspace only
    peak_delta = torch.cuda.max_memory_allocated() - base_alloc - out_bytes
    log(f"warmup done, loss {loss.item():.6f}")

    total_ms, per_step = time_steps(torch, step, args.steps, stream)
    kernels = fce.fce_timing_read()
    fce.fce_timing_enable(False)
    ms = total_ms / args.steps
    tokens_per_s = N / (ms / 1e3)
    flops_step = 8.0 * N * V * H
    peak = PEAK[wl.dtype]
    tflops = flops_step / (ms / 1e3) / 1e12
    srt = sorted(per_step)
    med = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2])
    log(f"{args.steps} steps: {ms:.3f} ms/step (median {med:.3f}, min {srt[0]:.3f}, "
        f"max {srt[-1]:.3f}), {tokens_per_s:,.0f} tokens/s, "
        f"{tflops:.1f} TFLOP/s = {100 * tflops / peak:.1f}% of {peak} TFLOP/s")
    log("  per step (ms): " + " ".join(f"{t:.2f}" for t in per_step))

    # dominant kernel: largest share of the timed region
    kern = {}
    for name, r in kernels.items():
        avg = r["total_ms"] / max(r["launches"], 1)
        kern[name] = {"launches_per_step": r["launches"] / args.steps,
                      "ms_per_step": r["total_ms"] / args.steps, "avg_launch_ms": avg,
                      "tflops": (r["flops"] / (r["total_ms"] / 1e3) / 1e12) if r["flops"] else None}
        log(f"  {name:12s} {r['launches'] / args.steps:6.1f} launches/step "
            f"{r['total_ms'] / args.steps:9.3f} ms/step  avg {avg * 1e3:9.1f} us"
            + (f"  {kern[name]['tflops']:8.1f} TFLOP/s" if r["flops"] else ""))
    dom = max(kern, key=lambda k: kern[k]["ms_per_step"])
    dom_r = kernels[dom]
    achieved = dom_r["flops"] / dom_r["launches"] / (dom_r["total_ms"] / dom_r["launches"] / 1e3) / 1e12
    traffic = read_traffic(dom, wl.name, kern[dom]["launches_per_step"])
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic}

    # ---- outside the headline figure
    side = {}
    k2 = args.side_steps
    if args.no_side or k2 < 1:
        side = None
    else:
        run_side(torch, fce, wk, args, side, X, W, y, loss, lse, dX, dW, ws, step, stream, ms)

    mem = {"logit_scratch_bytes": plan["scratch_bytes"],
           "workspace_bytes": plan["workspace_bytes"],
           "measured_peak_alloc_beyond_inputs_outputs": int(peak_delta),
           "naive_logits_bytes": N * V * (2 if wl.dtype == "bf16" else 4),
           "naive_3x_bytes": 3 * N * V * (2 if wl.dtype == "bf16" else 4),
           "chunk_tile_bound_bytes": chunk * V * (2 if wl.dtype == "bf16" else 4)}

    cpu = None
    if not args.no_cpu_baseline:
        n_cpu = cpu_tokens(wl, args.cpu_sample_tokens)
        log(f"timing the CPU oracle on {n_cpu} of {wl.N} tokens ...")
        cpu = cpu_baseline(wl, inp, n_cpu)
        log(f"  {cpu}")

    out = {
        "metric": "tokens/s + % bf16 MFMA peak, fused CE fwd+bwd, N=8192 H=4096 V=128256",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(med, 4),
        "ms_per_step_min": round(srt[0], 4),
        "ms_per_step_max": round(srt[-1], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name} fused CE fwd+bwd N={N} H={H} V={V}",
                   "N": N, "H": H, "V": V, "chunk": chunk, "schedule": sched,
                   "block_tokens": plan["block_tokens"], "block_vocab": plan["block_vocab"],
                   "label_smoothing": eps, "ignored_tokens": wl.n_ignored,
                   "parallelism": "single GPU"},
        "pct_peak_bf16_mfma": round(100 * tflops / peak, 2),
        "tflops_8NVH": round(tflops, 2),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kern,
        "memory": mem,
        "side": side,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the hybrid attention hot path on one MI355X.

One step = one hsa_hybrid_attn call over the whole batch of the 720P-shaped
workload (B=1, H=40, d=128, N=75600 tokens on the 21x45x80 latent grid,
padded to 75648, top-36 of 1182 tiles per row = 96.95% of tiles skipped,
rank 64, bf16): tile pooling, pooled scores, top-k selection, the linear
key/value state, block-sparse flash attention and the linear readout.  Inputs
are seeded synthetic tensors of that shape, resident in HBM before timing.

Prints one JSON line with the whole-call throughput in dense-equivalent
TFLOP/s (4 N^2 d H per call), the per-kernel split from HIP events recorded
on the launch stream, the roofline of the dominant kernel (the sparse flash
kernel against the dense matrix-core peak of the input type) and the fp64 oracle timed on this
host's cores over a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def executed_flops(nnz_tiles, d, tile=64):
    """Matrix-core work of the sparse branch: Q K^T and P V over every kept
    (query tile, key tile) pair, 2 * 64 * 64 * d FLOP each."""
    return 4.0 * tile * tile * d * nnz_tiles


def dense_equivalent_flops(n, d, heads, batch=1):
    """The same two products over every (query, key) pair of N valid tokens."""
    return 4.0 * n * n * d * heads * batch


def host_cores():
    """CPUs this process may run on, the CPU model and the BLAS thread count."""
    cpus = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max((d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"), default=1)
    except Exception:
        blas = 1
    return cpus, model, blas


def time_calls(run, steps, warmup, stream):
    """Whole-call times from HIP events recorded on the launch stream before and
    after every call (the library's per-kernel timing is off meanwhile).
    Returns (mean ms over the timed window, per-call ms)."""
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize()
    per = [e0.elapsed_time(e1) for e0, e1 in ev]
    return ev[0][0].elapsed_time(ev[-1][1]) / steps, per


def kernel_split(run, steps):
    """Average milliseconds per launch of every kernel kind over `steps` more
    calls, from the HIP events the library records on the launch stream."""
    import torch
    from block_sparse_linear_select_amd import binding as B
    B.timing_enable(steps)
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    kt = B.timing_read()
    B.timing_enable(0)
    return {k: (v[0] / v[1] if v[1] else None) for k, v in kt.items()}


def percentiles(per):
    import numpy as np
    return {"p50": float(np.percentile(per, 50)), "p95": float(np.percentile(per, 95)),
            "min": float(min(per)), "max": float(max(per))}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


ATTEND_SOURCES = ("common.hpp", "lds_dma.hpp", "readout.hpp", "attend.hpp", "k_attend.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_attend_hbm_traffic.md")


def attend_source_digest():
    """sha256 over the sources the attend kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in ATTEND_SOURCES:
        with open(os.path.join(ROOT, "block_sparse_linear_select_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attend launch from the committed counter summary, or None
    when there is none for this workload or the kernel sources changed since.
    The summary carries lines `traffic <workload> <bytes per launch> <digest>`."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    digest = attend_source_digest()
    for ln in lines:
        f = ln.strip().strip("`").split()
        if len(f) == 4 and f[0] == "traffic" and f[1] == workload and f[3] == digest:
            return float(f[2])
    return None


def head_fp64(w, inp, h):
    """(q, k, v) of head (0, h) in fp64 exactly as the kernels read them."""
    from oracle import rola as R
    from workloads.gen import fp8_codes, to_fp64
    if w.dtype == "fp8":
        return tuple(R.dequantize_tiles(fp8_codes(getattr(inp, n)[0, h]), getattr(inp, n + "_scale")[0, h].numpy())
                     for n in ("q", "k", "v"))
    return to_fp64(inp.q[0, h]), to_fp64(inp.k[0, h]), to_fp64(inp.v[0, h])


def cpu_baseline(w, inp, heads):
    """The fp64 oracle on `heads` whole heads of the workload, in the metric's unit."""
    from oracle import rola as R
    from workloads.gen import to_fp64
    cpus, model, blas = host_cores()
    t_total = 0.0
    for h in heads:
        args = (*head_fp64(w, inp, h), w.N, w.grid, to_fp64(inp.uq[h]), to_fp64(inp.uk[h]), to_fp64(inp.wo[h]))
        t0 = time.perf_counter()
        R.hybrid_head(*args, topk=w.topk, force_diag=w.force_diag, scale=w.softmax_scale, base=w.rope_base)
        t_total += time.perf_counter() - t0
        log(f"  oracle head {h}: {t_total:.1f} s so far")
    flops = dense_equivalent_flops(w.N, w.d, len(heads), 1)
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s (dense-equivalent)", "cores": int(min(cpus, blas)),
            "kind": "oracle",
            "sample": f"{len(heads)} of {w.H} heads of the workload, every query tile, full hybrid in fp64 "
                      f"({t_total:.1f} s; {t_total / len(heads) * w.H * w.B:.0f} s per whole call extrapolated)",
            "seconds_per_call_extrapolated": t_total / len(heads) * w.H * w.B,
            "cpus_available": cpus, "blas_threads": blas, "cpu_model": model}


def bench_proj(w, args, dev):
    """The W8A8 FP8 QKV projection in front of the attention, timed like the
    hybrid call: per step one row quantisation of the bf16 activations
    [B*N_pad, H*d] and one projection to FP8 q, k, v with their tile scales."""
    import torch
    from block_sparse_linear_select_amd import binding as B
    from workloads.gen import generate_proj
    t0 = time.time()
    p = generate_proj(w)
    C = w.H * w.d
    M = w.B * w.N_pad
    x = p.x.reshape(M, C).to(dev)
    wq, sw = p.wq.to(dev), p.sw.to(dev)
    log(f"  projection inputs: x [{M}, {C}] bf16, w [{3 * C}, {C}] fp8 ({time.time() - t0:.1f} s)")
    del p

    def step():
        xc, xs = B.quantize_rows_fp8(x)
        return B.qkv_proj_fp8(xc, xs, wq, sw, w.B, w.N_pad, w.H, w.d)

    ms, per = time_calls(step, args.steps, args.warmup, torch.cuda.current_stream())
    kern = kernel_split(step, args.steps)
    q_ms, p_ms = kern["quant"], kern["proj"]
    flops = 2.0 * M * C * 3 * C
    log(f"  {args.steps} projection steps: {ms:.3f} ms/step (quant {q_ms:.3f}, proj {p_ms:.3f})")
    achieved = flops / (p_ms * 1e-3) / 1e12
    return {"ms_per_step": ms, "quant_ms": q_ms, "proj_ms": p_ms, "flops": flops,
            "quant_GBps": 3.0 * M * C / (q_ms * 1e-3) / 1e9,
            "roofline": {"bound": "mfma", "kernel": "k_proj_fp8", "achieved": achieved, "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_FP8_TFLOPS}}


def bench_compl(w, cfg, d, sc, args, dev):
    """Hybrid calls with the linear branch over the complement of each row's
    kept tiles (selection inside, as the main measurement), timed the same way.
    The complement kernel gathers min(k, T - k) per-tile states per row (from
    L2 / MALL; each state is read from HBM at least once) and reads Q and
    reads + writes O."""
    import dataclasses

    import torch
    from block_sparse_linear_select_amd import binding as B

    ccfg = dataclasses.replace(cfg, linear_keys="complement")
    plan = B.HybridPlan(ccfg, dev)
    run = lambda: plan.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], sc["q_scale"], sc["k_scale"],
                           sc["v_scale"], check=False)
    ms, per = time_calls(run, args.steps, args.warmup, torch.cuda.current_stream())
    kern = kernel_split(run, args.steps)
    log(f"  {args.steps} calls, complement keys: {ms:.3f} ms/call (complement kernel {kern['compl']:.3f} ms)")
    return {"ms_per_call": ms, **{"ms_" + k: v for k, v in percentiles(per).items()}, "kernels_ms": kern,
            "compl_kernel": compl_figures(w, kern["compl"])}


def bench_backward(w, cfg, d, args, dev):
    """Backward calls (dQ, dK, dV float32 for a seeded dO) on the mask the
    hybrid call selects, timed like the forward.  The sparse part recomputes
    P and dP per kept tile pair and forms dS, dQ, dK, dV: 5 products of
    2*64*64*d FLOP per pair, the algorithmic count the roofline uses.  The
    kernels execute 8 (QK^T in each of the dQ, dV and dK kernels, dO V^T in
    the dQ and dK kernels), reported as executed_flop."""
    import torch
    from block_sparse_linear_select_amd import binding as B
    from workloads.gen import upstream_grad

    sel = B.HybridPlan(cfg, dev, export_mask=True)
    sel.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"])
    g = upstream_grad(w, seed=w.seed + 7).to(dev)
    run = lambda: B.hybrid_attn_backward(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], sel.row_ptr,
                                         sel.col_idx, g)
    steps = max(1, args.steps // 2)
    ms, per = time_calls(run, steps, max(1, args.warmup // 2), torch.cuda.current_stream())
    kern = kernel_split(run, steps)
    log(f"  {steps} backward calls: {ms:.3f} ms/call (sparse part {kern['bwd_sparse']:.3f} ms)")
    # the same gradients from the training forward's saved O_s and log-sum-exp (no sparse recompute)
    _, o_s, lse = B.hybrid_attn_train(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], row_ptr=sel.row_ptr,
                                      col_idx=sel.col_idx)
    run_saved = lambda: B.hybrid_attn_backward_saved(cfg, d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"],
                                                     sel.row_ptr, sel.col_idx, o_s, lse, g)
    ms_saved, per_saved = time_calls(run_saved, steps, max(1, args.warmup // 2), torch.cuda.current_stream())
    log(f"  {steps} backward calls on saved statistics: {ms_saved:.3f} ms/call")
    cols = sel.col_idx[:int(sel.row_ptr[-1].item())]
    pairs = int(((cols >= 0) & (cols < w.T)).sum().item())
    flops = 5 * 2.0 * 64 * 64 * w.d * pairs
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else 157.3
    ach = flops / (kern["bwd_sparse"] * 1e-3) / 1e12
    return {"ms_per_call": ms, **{"ms_" + k: v for k, v in percentiles(per).items()}, "kernels_ms": kern,
            "steps": steps,
            "saved_statistics": {"ms_per_call": ms_saved, **{"ms_" + k: v for k, v in percentiles(per_saved).items()}},
            "sparse_roofline": {"bound": "mfma", "kernel": "k_bwd_dq + k_bwd_dv + k_bwd_dk (+ transposed mask)",
                                "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
                                "flop": flops, "executed_flop": flops * 8 / 5}}


def compl_figures(w, cms):
    """Bytes of the complement kernel per call: the per-row state sums read
    min(k, T - k) tile states per row (before the reuse that four rows per
    block and the caches give), and Q, O and every tile state at least once."""
    rows = w.B * w.H * w.T
    summed = rows * min(w.topk, w.T - w.topk)            # no forced diagonal
    st_elt = 4 if w.dtype == "f32" else 2
    in_elt = 1 if w.dtype == "fp8" else (4 if w.dtype == "f32" else 2)
    state_bytes = 32 * ((w.rank + 31) // 32) * w.d * st_elt
    gathered = summed * state_bytes
    hbm = (w.B * w.H * w.N_pad * w.d * (in_elt + 2 * st_elt)   # Q read, O read and written
           + rows * state_bytes)                              # every tile state at least once
    return {"ms": cms, "states_summed": summed, "summed_bytes": gathered,
            "summed_GBps": gathered / (cms * 1e-3) / 1e9,
            "hbm_bytes_min": hbm, "hbm_GBps_min": hbm / (cms * 1e-3) / 1e9,
            "hbm_frac_min": hbm / (cms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def call_figures(w, ms, per, kern, nnz, linear_keys="all"):
    """The JSON fields of one timed workload: whole-call figures, the roofline
    of the attend kernel (executed FLOP over its average launch) and the
    linear state pass against HBM."""
    exec_flops = executed_flops(nnz, w.d)
    dense_flops = dense_equivalent_flops(w.N, w.d, w.H, w.B)
    attend_ms = kern["attend"]
    elt = 1 if w.dtype == "fp8" else (4 if w.dtype == "f32" else 2)
    peak = PEAK_FP8_TFLOPS if w.dtype == "fp8" else PEAK_BF16_TFLOPS
    achieved = exec_flops / (attend_ms * 1e-3) / 1e12
    kv_bytes = 2.0 * w.B * w.H * w.N * w.d * elt          # K and V, the linear key/value state's input
    stream_ms = kern["stream"]
    pct = percentiles(per)
    return {
        "value": dense_flops / (ms * 1e-3) / 1e12,
        "unit": "TFLOP/s (dense-equivalent, 4*N^2*d*H per call)",
        "ms_per_step": ms,
        "ms_per_call": {"mean": ms, **pct},
        "executed_tflops": exec_flops / (ms * 1e-3) / 1e12,
        "kept_tile_pairs": nnz,
        "roofline": {"bound": "mfma", "kernel": "k_attend (block-sparse flash" + (
                         " + linear readout)" if linear_keys == "all" else ")"),
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "flop_per_launch": exec_flops, "ms_per_launch": attend_ms,
                     "traffic": measured_traffic(w.name) if linear_keys == "all" else None},
        "kernels_ms": kern,
        "linear_state": {"kernel": "k_stream (key/value state)", "ms": stream_ms,
                         "kv_bytes": kv_bytes, "kv_GBps": kv_bytes / (stream_ms * 1e-3) / 1e9,
                         "kv_frac_hbm": kv_bytes / (stream_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }


def bench_locality(w, cfg, d, sc, sel, args, dev):
    """The sparse attend kernel alone (hsa_sparse_attn) on the selected mask and
    on three masks of the same size and the same k tiles per row that differ
    only in which key tiles the rows share: every row the same k tiles (they
    stay in L2), a band of k consecutive tiles around the row, and k tiles
    drawn uniformly per row.  Shows how much of the kernel's time depends on
    key tiles being re-fetched from memory."""
    import torch
    from block_sparse_linear_select_amd import binding as B
    T, k, bh = w.T, w.topk, w.B * w.H
    a = torch.arange(T)
    g = torch.Generator().manual_seed(1234)
    masks = {
        "selected": None,
        "same_tiles": torch.arange(k).repeat(T, 1),
        "band": (a - k // 2).clamp(0, T - k)[:, None] + torch.arange(k)[None, :],
        "uniform_random": torch.stack([torch.randperm(T, generator=g)[:k].sort().values for _ in range(T)]),
    }
    rp = (torch.arange(bh * T + 1, dtype=torch.int32) * k).to(dev)
    res = {}
    for name, m in masks.items():
        if m is None:
            row_ptr, col_idx = sel.row_ptr, sel.col_idx
        else:
            row_ptr, col_idx = rp, m.to(torch.int32).repeat(bh, 1).reshape(-1).contiguous().to(dev)
        run = lambda: B.sparse_attn(cfg, d["q"], d["k"], d["v"], row_ptr, col_idx, sc["q_scale"], sc["k_scale"],
                                    sc["v_scale"])
        for _ in range(args.warmup):
            run()
        kern = kernel_split(run, min(args.steps, 20))
        res[name] = {"attend_ms": kern["attend"]}
        log(f"  sparse attend on the {name} mask: {kern['attend']:.3f} ms")
    return res


def bench_second_workload(name, args, dev):
    """Another workload of the same shape (the FP8 one), timed the same way:
    whole calls with p50/p95, the kernel split, and its roofline."""
    import torch
    from block_sparse_linear_select_amd import binding as B
    from workloads import make_workload, generate
    w = make_workload(name)
    cfg = B.Config.from_workload(w)
    t0 = time.time()
    inp = generate(w)
    log(f"  {name} generated in {time.time() - t0:.1f} s")
    d = {k: getattr(inp, k).to(dev) for k in ("q", "k", "v", "uq", "uk", "wo")}
    sc = {k: (None if getattr(inp, k) is None else getattr(inp, k).to(dev)) for k in ("q_scale", "k_scale", "v_scale")}
    del inp
    plan = B.HybridPlan(cfg, dev)
    run = lambda: plan.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], sc["q_scale"], sc["k_scale"],
                           sc["v_scale"], check=False)
    ms, per = time_calls(run, args.steps, args.warmup, torch.cuda.current_stream())
    kern = kernel_split(run, args.steps)
    sel = B.HybridPlan(cfg, dev, export_mask=True)
    sel.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], sc["q_scale"], sc["k_scale"], sc["v_scale"])
    torch.cuda.synchronize()
    cols = sel.col_idx[: int(sel.row_ptr[-1].item())]
    nnz = int(((cols >= 0) & (cols < w.T)).sum().item())
    log(f"  {args.steps} {name} calls: {ms:.3f} ms/call (attend {kern['attend']:.3f} ms)")
    res = {"workload": name, "dtype": w.dtype}
    res.update(call_figures(w, ms, per, kern, nnz))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan14b_720p_bf16")
    ap.add_argument("--cpu-heads", type=int, default=8, help="heads the oracle baseline runs (0 skips it)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 leg: the same 720P shape with E4M3 inputs, timed like the main workload")
    ap.add_argument("--no-reuse", action="store_true",
                    help="skip the second measurement: calls that reuse one selected mask (no pooling, "
                         "scores or top-k), as across denoising steps")
    ap.add_argument("--no-proj", action="store_true",
                    help="skip the third measurement: the W8A8 FP8 QKV projection (activation quantisation + "
                         "projection with fused output quantisation) at the workload's shape")
    ap.add_argument("--linear-keys", choices=("all", "complement"), default="all",
                    help="keys of the linear branch in the main measurement: every valid key, or the complement "
                         "of each row's kept tiles")
    ap.add_argument("--no-compl", action="store_true",
                    help="skip the fourth measurement: hybrid calls whose linear branch sums over the complement "
                         "of each row's kept tiles")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the fifth measurement: the backward pass (dQ, dK, dV) on the selected mask")
    ap.add_argument("--no-locality", action="store_true",
                    help="skip the sparse attend kernel on masks of the same size with shared, banded and uniformly "
                         "drawn key tiles")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before warmup, run 3 launches of a plain elementwise kernel that reads and writes MIB "
                         "MiB each (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards by head, "
              "see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_linear_select_amd import binding as B
    from workloads import make_workload, generate

    w = make_workload(args.workload)
    cfg = B.Config.from_workload(w)
    if args.linear_keys != "all":
        import dataclasses
        cfg = dataclasses.replace(cfg, linear_keys=args.linear_keys)
    dev = torch.device("cuda:0")
    log(f"generating {w.name}: B={w.B} H={w.H} N={w.N} (pad {w.N_pad}) d={w.d} top-{w.topk} of {w.T}, r={w.rank}")
    t0 = time.time()
    inp = generate(w)
    log(f"  generated in {time.time() - t0:.1f} s")
    d = {k: getattr(inp, k).to(dev) for k in ("q", "k", "v", "uq", "uk", "wo")}
    sc = {k: (None if getattr(inp, k) is None else getattr(inp, k).to(dev)) for k in ("q_scale", "k_scale", "v_scale")}
    plan = B.HybridPlan(cfg, dev)
    run = lambda: plan.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], sc["q_scale"], sc["k_scale"],
                           sc["v_scale"], check=False)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        log(f"  calibration: 3 x neg over {args.calibrate_copy} MiB float32 (read and write {n * 4} bytes each)")
        del x, y
    stream = torch.cuda.current_stream()
    ms, per = time_calls(run, args.steps, args.warmup, stream)
    log(f"  {args.steps} calls: {ms:.3f} ms/call mean, p50 {percentiles(per)['p50']:.3f} ms")
    kern = kernel_split(run, args.steps)

    # kept tile pairs, counted on the mask this workload selects
    sel = B.HybridPlan(cfg, dev, export_mask=True)
    sel.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], sc["q_scale"], sc["k_scale"], sc["v_scale"])
    torch.cuda.synchronize()
    cols = sel.col_idx[: int(sel.row_ptr[-1].item())]
    nnz = int(((cols >= 0) & (cols < w.T)).sum().item())
    out = {"metric": "hybrid attn ms/call + effective TFLOP/s at N=75600,H=40; % MFMA/HBM peak",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": w.dtype, "data": "synthetic",
           "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "N_pad": w.N_pad, "d": w.d,
                      "grid": list(w.grid), "tile": 64, "topk": w.topk, "tiles_per_row": w.T,
                      "density": nnz / (w.B * w.H * w.T * w.T), "rank": w.rank, "linear_keys": args.linear_keys,
                      "parallelism": "single GPU"}}
    out.update(call_figures(w, ms, per, kern, nnz, args.linear_keys))
    # the same call captured once in a HIP graph and replayed (a serving loop's
    # way to call it: no launch gaps between the call's kernels)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    ms_g, per_g = time_calls(graph.replay, args.steps, args.warmup, stream)
    out["graph_replay"] = {"ms_per_call": ms_g, **{"ms_" + k: v for k, v in percentiles(per_g).items()},
                           "value": dense_equivalent_flops(w.N, w.d, w.H, w.B) / (ms_g * 1e-3) / 1e12}
    log(f"  {args.steps} graph replays: {ms_g:.3f} ms/call")
    del graph
    if "linear_state" in out:
        # a library read of the same K and V bytes on this GPU, for scale: torch's
        # sum over each tensor (rows past N included; FP8 codes summed as bytes)
        kv = [x.view(torch.uint8) if x.element_size() == 1 else x for x in (d["k"], d["v"])]
        rd = lambda: [x.sum(dtype=torch.int64 if x.dtype == torch.uint8 else torch.float32) for x in kv]
        ms_sum, _ = time_calls(rd, 10, 3, stream)
        nb = sum(x.numel() * x.element_size() for x in kv)
        out["linear_state"]["torch_sum_kv"] = {"bytes": nb, "ms": ms_sum, "GBps": nb / (ms_sum * 1e-3) / 1e9,
                                               "frac_hbm": nb / (ms_sum * 1e-3) / 1e9 / PEAK_HBM_GBS}
        # the read rate of a plain streaming kernel over the same two tensors
        # (the library's calibration read), the practical ceiling of the pass
        sink = torch.empty(B.READ_SINK_WORDS, dtype=torch.int32, device=dev)
        ms_rd = 0.0
        for x in (d["k"], d["v"]):  # one launch per timed call, events around it
            ms_rd += percentiles(time_calls(lambda: B.read_calibrate(x, sink), 20, 5, stream)[1])["p50"]
        ceil = nb / (ms_rd * 1e-3) / 1e9
        out["linear_state"]["read_ceiling"] = {"kernel": "hsa_attn_read_calibrate over K and V", "bytes": nb,
                                               "ms": ms_rd, "GBps": ceil, "frac_hbm": ceil / PEAK_HBM_GBS}
        out["linear_state"]["kv_frac_read_ceiling"] = out["linear_state"]["kv_GBps"] / ceil
        log(f"  read ceiling {ceil:.0f} GB/s; streaming pass {out['linear_state']['kv_GBps']:.0f} GB/s")
    if not args.no_reuse:
        # Mask reuse: select once, then run the hybrid call on that CSR (the
        # streaming pass then computes the linear state only).  Same inputs,
        # same launch configuration; timed the same way.
        reuse = lambda: plan.run(d["q"], d["k"], d["v"], d["uq"], d["uk"], d["wo"], sc["q_scale"], sc["k_scale"],
                                 sc["v_scale"], row_ptr=sel.row_ptr, col_idx=sel.col_idx, check=False)
        ms_r, per_r = time_calls(reuse, args.steps, args.warmup, stream)
        kern_r = kernel_split(reuse, args.steps)
        log(f"  {args.steps} calls on a reused mask: {ms_r:.3f} ms/call")
        out["mask_reuse"] = {"ms_per_call": ms_r, **{"ms_" + k: v for k, v in percentiles(per_r).items()},
                             "value": dense_equivalent_flops(w.N, w.d, w.H, w.B) / (ms_r * 1e-3) / 1e12,
                             "kernels_ms": kern_r}
        if "linear_state" in out:
            # on a given mask the streaming pass is the state reduction alone (no key pooling)
            ls = out["linear_state"]
            gbs = ls["kv_bytes"] / (kern_r["stream"] * 1e-3) / 1e9
            ls["state_only"] = {"kernel": "k_stream without pooling (calls on a given mask)", "ms": kern_r["stream"],
                                "kv_GBps": gbs, "kv_frac_hbm": gbs / PEAK_HBM_GBS}
            if "read_ceiling" in ls:
                ls["state_only"]["kv_frac_read_ceiling"] = gbs / ls["read_ceiling"]["GBps"]
    if not args.no_locality and args.linear_keys == "all":
        out["attend_locality"] = bench_locality(w, cfg, d, sc, sel, args, dev)
    if not args.no_proj and w.d == 128:
        out["qkv_proj"] = bench_proj(w, args, dev)
    if not args.no_bwd and w.dtype != "fp8" and args.linear_keys == "all":
        out["backward"] = bench_backward(w, cfg, d, args, dev)
    if args.linear_keys == "complement":
        out["compl_kernel"] = compl_figures(w, kern["compl"])
    elif not args.no_compl:
        out["linear_complement"] = bench_compl(w, cfg, d, sc, args, dev)
    if not args.no_fp8 and w.dtype == "bf16" and w.name == "wan14b_720p_bf16":
        # the same shape with FP8 E4M3 inputs (per-tile scales), as its own leg
        del plan, sel
        torch.cuda.empty_cache()
        out["fp8"] = bench_second_workload("wan14b_720p_fp8", args, dev)
    if args.cpu_heads > 0:
        log(f"oracle baseline on {args.cpu_heads} heads")
        heads = list(range(min(args.cpu_heads, w.H)))
        out["cpu_baseline"] = cpu_baseline(w, inp, heads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

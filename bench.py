#!/usr/bin/env python3
"""Throughput of the GPTQ layer solve on one MI355X.

One step = the whole hot path on one layer: Hessian accumulation over the
calibration tokens (H from scratch), prepare (dead columns, act-order,
damping, fp64 Cholesky and triangular inverse -> U), and the quantize sweep
(lazy block updates, packing, loss).  Inputs are synthetic, seeded, and
resident in HBM before timing starts.

Prints one JSON line.  value = weights quantized per second for the whole
step (rows * n / step time).  Also reported: Hessian TFLOP/s (algorithmic:
n(n+1) flops per token, the unique entries of the symmetric product), the
solve-only rate (prepare + quantize, H given), per-stage times, the roofline of
the Hessian kernel measured live with HIP events on its stream, and the
float64 CPU oracle timed on a bounded sample of the same workload.

The line also carries "dequant_matmul": the decode-time product with the
packed layers (one token, and a batch of 16) through every linear of a
32-block Llama-2-7B-shaped stack at 4-bit g128, replayed as a graph, with its
HBM roofline.

Usage: python bench.py [--steps K] [--warmup W] [--workload attn4096]
       python bench.py --matmul-only  (only the dequant_matmul part, for profiling)
       python bench.py --pmc-probe    (short run for rocprofv3 --pmc counter passes)
       python bench.py --matmul-only --pmc-probe   (the same for the dequant_matmul pass)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA (published)
PEAK_FP64_TFLOPS = 78.6      # MI355X fp64 (vector and MFMA, published)
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 vector and fp32 MFMA (published)
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 MFMA (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)
DTYPE = ("bf16 MFMA Hessian (fp32 chains of 256 tokens, fp64 accumulation); fp64 MFMA Cholesky + triangular "
         "inverse; fp32 column sweep with split-bf16 (3 bf16 MFMA products, fp32 accumulation) lazy-block updates")
METRIC = "GPTQ weights quantized/sec per layer (4096×4096, g128) + Hessian TFLOP/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hessian_attn4096_traffic.json")
HESSIAN_SRC = os.path.join(ROOT, "post_weight_quantization_13_amd", "csrc", "hessian.hip")
MM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dequant_matmul_decode7b_traffic.json")
MM_SRC = os.path.join(ROOT, "post_weight_quantization_13_amd", "csrc", "matmul.hip")


def _log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _sha(path) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(path=TRAFFIC_FILE, src=HESSIAN_SRC, key="bytes_per_launch"):
    """HBM bytes per launch (or per pass) from a committed counter summary, if
    it is for the current kernel source; else None."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != _sha(src):
        return None
    return t.get(key)


def layer_solve_roofline(layers, hess, stage_ms):
    """t_roof per stage of one step against the peak of the arithmetic each
    stage runs in, and t_roof / t_measured for the solve and the whole step.

    layers: [(rows, n, bits, group_size)] quantized linears; hess: [(n, tokens)]
    Hessians built (a factor shared by several linears is counted once).
      Hessian   n(n+1) flop per token (unique entries of X^T X), bf16 MFMA.
      prepare   2n^3/3 flop (Cholesky n^3/3 + triangular inverse n^3/3), fp64.
      quantize  the column sweep rows*n*B flop on the fp32 vector ALUs
                (each column updates the rest of its 128-column block);
                the lazy-block updates rows*n*(n-B) flop issued as three bf16
                MFMA products each, or their fp32 W read-modify-write per
                512-column super-block if that takes longer; and the minimal
                I/O (W bf16 in, U fp32 read, packed codes, scales and zeros,
                g_idx out) at HBM speed."""
    B, SB = 128, 512
    t_h = sum(n * (n + 1) * tok for n, tok in hess) / (PEAK_BF16_TFLOPS * 1e12)
    t_p = sum(2.0 * n ** 3 / 3 for n, _ in hess) / (PEAK_FP64_TFLOPS * 1e12)
    t_sweep = t_upd = t_io = 0.0
    for rows, n, bits, gs in layers:
        t_sweep += rows * n * B / (PEAK_FP32_TFLOPS * 1e12)
        flops = 3.0 * rows * n * max(n - B, 0)
        sbs = n // SB
        upd_bytes = 8.0 * rows * sum(max(n - (s + 2) * SB, 0) for s in range(sbs))
        t_upd += max(flops / (PEAK_BF16_TFLOPS * 1e12), upd_bytes / (PEAK_HBM_GBS * 1e9))
        G = n // gs if gs > 0 else 1
        io = 2.0 * rows * n + 4.0 * n * n + rows * n * bits / 8 + 4.0 * rows * G + 4 * n
        t_io += io / (PEAK_HBM_GBS * 1e9)
    t_q = t_sweep + t_upd + t_io
    ms = lambda t: t * 1e3
    solve_meas = stage_ms["prepare"] + stage_ms["quantize"]
    step_meas = solve_meas + stage_ms["hessian"]
    return {
        "stages": {
            "hessian": {"t_roof_ms": ms(t_h), "t_ms": stage_ms["hessian"], "frac": ms(t_h) / stage_ms["hessian"],
                        "peak": "bf16 MFMA 2500 TFLOP/s"},
            "prepare": {"t_roof_ms": ms(t_p), "t_ms": stage_ms["prepare"], "frac": ms(t_p) / stage_ms["prepare"],
                        "peak": "fp64 78.6 TFLOP/s"},
            "quantize": {"t_roof_ms": ms(t_q), "t_ms": stage_ms["quantize"], "frac": ms(t_q) / stage_ms["quantize"],
                         "parts_ms": {"sweep_fp32_valu": ms(t_sweep), "split_bf16_updates": ms(t_upd),
                                      "io_hbm": ms(t_io)},
                         "peak": "fp32 vector 157.3 TFLOP/s, bf16 MFMA 2500 TFLOP/s, HBM 8 TB/s"},
        },
        "solve": {"t_roof_ms": ms(t_p + t_q), "t_ms": solve_meas, "frac": ms(t_p + t_q) / solve_meas},
        "step": {"t_roof_ms": ms(t_h + t_p + t_q), "t_ms": step_meas, "frac": ms(t_h + t_p + t_q) / step_meas},
    }


def _host_info():
    """CPU model, the threads numpy's BLAS uses, and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas_threads, blas = 0, "unknown"
    try:
        import numpy  # noqa: F401  (loads the BLAS threadpoolctl reports on)
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas_threads = max(blas_threads, int(i.get("num_threads", 0)))
                blas = f"{i.get('internal_api')} {i.get('version')}"
    except Exception:  # pragma: no cover
        pass
    return model, blas, blas_threads, len(os.sched_getaffinity(0))


def _device_inputs(wl, torch):
    import numpy as np
    import synth
    lin = wl.linears[0]
    _log(f"generating {wl.name}: W {lin.rows}x{lin.n}, X {wl.tokens}x{lin.n} ({wl.dtype})")
    w_raw = synth.weights_raw(wl, 0)
    x_raw = synth.activations_raw(wl, lin.xset)
    if wl.dtype == "bf16":
        W = torch.from_numpy(w_raw.view(np.int16)).view(torch.bfloat16).cuda()
        X = torch.from_numpy(x_raw.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        W = torch.from_numpy(w_raw).cuda()
        X = torch.from_numpy(x_raw).cuda()
    return w_raw, x_raw, W, X


def _xset_on_device(wl, xset, torch):
    """X set ``xset`` of the workload on the GPU, its chunks generated by
    spawned worker processes (numpy only, no GPU use there)."""
    import numpy as np
    import synth
    n = wl.xsets[xset][0]
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    X = torch.empty((wl.tokens, n), dtype=dt, device="cuda")

    def put(t0, raw):
        src = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16) if wl.dtype == "bf16" \
            else torch.from_numpy(raw)
        X[t0:t0 + raw.shape[0]].copy_(src)

    synth.activations_raw_parallel(wl, xset, workers=min(16, len(os.sched_getaffinity(0))), out=put)
    return X


def _check_steps(info, loss=None):
    """Every step's prepare found a positive definite Hessian, and every
    step's loss (deterministic inputs, deterministic kernels) is the same
    finite number."""
    flags = info.cpu().tolist()
    if any(f != 0 for f in flags):
        raise RuntimeError(f"prepare reported a Hessian that is not positive definite: flags {flags}")
    if loss is not None:
        vals = loss.cpu().tolist()
        if not all(v == vals[0] for v in vals) or not (vals[0] >= 0.0 and vals[0] < float("inf")):
            raise RuntimeError(f"step losses differ or are not finite: {vals}")


def block_bench(args, wl, g, torch):
    """One step = the whole block: a Hessian from scratch and a prepare per
    activation set, then a quantize per linear (the sets' factors shared)."""
    import numpy as np
    import synth
    torch.cuda.set_device(0)
    cfg = g.Config(bits=wl.bits, group_size=wl.group_size, sym=wl.sym, desc_act=wl.desc_act,
                   damp_percent=wl.damp, block_size=wl.block_size)
    Xs = []
    for xs in range(len(wl.xsets)):
        _log(f"generating X set {xs}: {wl.tokens} x {wl.xsets[xs][0]}")
        Xs.append(_xset_on_device(wl, xs, torch))
    Ws = []
    for li, lin in enumerate(wl.linears):
        w_raw = synth.weights_raw(wl, li)
        Ws.append(torch.from_numpy(w_raw.view(np.int16)).view(torch.bfloat16).cuda() if wl.dtype == "bf16"
                  else torch.from_numpy(w_raw).cuda())
    dev = Xs[0].device
    ns = [x.shape[1] for x in Xs]
    Hs = [torch.empty((n, n), dtype=torch.float64, device=dev) for n in ns]
    Us = [torch.empty((n, n), dtype=torch.float32, device=dev) for n in ns]
    perms = [torch.empty(n, dtype=torch.int32, device=dev) for n in ns]
    deads = [torch.empty(n, dtype=torch.uint8, device=dev) for n in ns]
    ws_h = [g.hessian_workspace(n, X) for n, X in zip(ns, Xs)]
    ws_p = [g.workspace(g.gptq_prepare_workspace_bytes(n, cfg), dev) for n in ns]
    outs = [g.alloc_outputs(lin.rows, lin.n, cfg, dev) for lin in wl.linears]
    ws_q = [g.workspace(g.gptq_quantize_workspace_bytes(lin.rows, lin.n, cfg), dev) for lin in wl.linears]
    torch.cuda.synchronize()

    # stream-ordered prepare and quantize (no host round trip inside a step);
    # the flags and losses are checked after the timed steps
    nsets, nlin = len(Xs), len(wl.linears)
    info = torch.full(((args.warmup + args.steps) * nsets,), -1, dtype=torch.int32, device=dev)
    loss = torch.full(((args.warmup + args.steps), nlin), -1.0, dtype=torch.float64, device=dev)

    def step(i):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        for s in range(nsets):
            g.gptq_hessian_accumulate(Hs[s], 0, Xs[s], ws_h[s])
        ev[1].record()
        for s in range(nsets):
            g.gptq_prepare_hinv_async(Hs[s], cfg, Us[s], perms[s], deads[s], info[i * nsets + s:i * nsets + s + 1],
                                      ws_p[s])
        ev[2].record()
        for li, lin in enumerate(wl.linears):
            s = lin.xset
            qw, sc, ze, gi = outs[li]
            g.gptq_quantize_layer_async(Us[s], perms[s], deads[s], cfg, Ws[li], qw, sc, ze, gi,
                                        loss[i, li:li + 1], ws_q[li])
        ev[3].record()
        return ev

    for i in range(args.warmup):
        step(i)
        torch.cuda.synchronize()
        _log(f"warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        events.append(step(args.warmup + i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _check_steps(info)
    for li in range(nlin):
        _check_steps(info[:1], loss[:, li])
    ms_step = (t1 - t0) * 1e3 / args.steps
    st = {k: sum(e[a].elapsed_time(e[b]) for e in events) / args.steps
          for k, a, b in (("hessian", 0, 1), ("prepare", 1, 2), ("quantize", 2, 3))}
    weights = sum(lin.rows * lin.n for lin in wl.linears)
    hess_flops = float(sum(n * (n + 1) for n in ns)) * wl.tokens
    hess_tflops = hess_flops / (st["hessian"] * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": weights / (ms_step * 1e-3), "unit": "weights/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": wl.name, "linears": [(lin.name, lin.rows, lin.n, lin.xset) for lin in wl.linears],
                   "xsets": [x[0] for x in wl.xsets], "tokens": wl.tokens, "bits": wl.bits,
                   "group_size": wl.group_size, "sym": wl.sym, "desc_act": wl.desc_act, "damp": wl.damp,
                   "description": wl.description},
        "hessian_tflops": hess_tflops,
        "solve_weights_per_s": weights / ((st["prepare"] + st["quantize"]) * 1e-3),
        "stage_ms": st,
        "roofline": {"kernel": "syrk_dma_kernel<bf16> (Hessian, all sets)", "bound": "mfma",
                     "achieved": hess_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": hess_tflops / PEAK_BF16_TFLOPS, "traffic": None,
                     "layer_solve": layer_solve_roofline(
                         [(lin.rows, lin.n, wl.bits, wl.group_size) for lin in wl.linears],
                         [(n, wl.tokens) for n in ns], st)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        _log("timing the float64 oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline_block(wl)
    print(json.dumps(out), flush=True)
    return 0


def block_sequential_bench(args, wl, g, torch):
    """One step = block-sequential calibration of the whole block: the block
    forward in the library's kernels (RMSNorm, q/k/v through the dequantizing
    matmul of the just-quantized weights, RoPE, causal attention, o, residual,
    RMSNorm, gate/up, SiLU gate) with a Hessian, a prepare and the quantize
    calls of each stage on the activations that reach it."""
    import numpy as np
    import synth
    torch.cuda.set_device(0)
    cfg = g.Config(bits=wl.bits, group_size=wl.group_size, sym=wl.sym, desc_act=wl.desc_act,
                   damp_percent=wl.damp, block_size=wl.block_size)
    seq_len = 2048
    _log(f"generating the block input: {wl.tokens} x {wl.xsets[0][0]} ({wl.tokens // seq_len} sequences)")
    X0 = _xset_on_device(wl, 0, torch)
    Ws = []
    for li, lin in enumerate(wl.linears):
        w_raw = synth.weights_raw(wl, li)
        Ws.append(torch.from_numpy(w_raw.view(np.int16)).view(torch.bfloat16).cuda())
    torch.cuda.synchronize()

    def step(timings=None):
        outs, Hs, _ = g.calibrate_block_sequential(X0, Ws, cfg, seq_len=seq_len, timings=timings)
        return outs

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        _log(f"warmup step {i + 1}/{args.warmup} done")
    # HIP events around the forward's projections (the prefill dequantizing
    # matmul, with the act-order gather that precedes it in the same call) and
    # the attention, on the stream they run on, over the timed steps
    timings = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(timings)
        torch.cuda.synchronize()
        _log(f"step {i + 1}/{args.steps} done")
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    part = {}
    for name, flop, a, b in timings:
        ms, fl, k = part.get(name, (0.0, 0.0, 0))
        part[name] = (ms + a.elapsed_time(b), fl + flop, k + 1)
    mm_ms, mm_flop, mm_calls = part["matmul"]
    at_ms, at_flop, at_calls = part["attention"]
    mm_tf = mm_flop / (mm_ms * 1e-3) / 1e12
    at_tf = at_flop / (at_ms * 1e-3) / 1e12
    weights = sum(lin.rows * lin.n for lin in wl.linears)
    out = {
        "metric": "GPTQ weights quantized/sec, block-sequential calibration of one decoder block",
        "value": weights / (ms_step * 1e-3), "unit": "weights/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE + "; block forward: fp16 activations, fp16 MFMA projections with fp32 sums, fp32 MFMA attention, fp64 norms",
        "data": "synthetic",
        "config": {"workload": wl.name + "-sequential", "tokens": wl.tokens, "seq_len": seq_len,
                   "linears": [(lin.name, lin.rows, lin.n) for lin in wl.linears], "bits": wl.bits,
                   "group_size": wl.group_size, "desc_act": wl.desc_act, "damp": wl.damp},
        "stage_ms": {"forward_projections": mm_ms / args.steps, "attention": at_ms / args.steps},
        "roofline": {"kernel": "prefill_matmul_kernel (the forward's six projections, act-order gathers included)",
                     "bound": "mfma", "achieved": mm_tf, "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": mm_tf / PEAK_FP16_TFLOPS, "traffic": None,
                     "work": "2 * tokens * rows * n flop per projection, %d launches per step" % (mm_calls // args.steps),
                     "attention": {"kernel": "attention_kernel (fp32 MFMA)", "achieved": at_tf,
                                   "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s", "frac": at_tf / PEAK_FP32_TFLOPS,
                                   "work": "2 * tokens * seq_len * d flop (the causal half of QK^T and PV)"}},
    }
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_block(wl):
    """The float64 oracle on a bounded sample of the block, scaled to weights/s:
    each set's Hessian on 4096 tokens (x tokens/4096), prepare once at the
    first set's width n_0 (scaled by (n_s/n_0)^3 for each set: Cholesky and
    inverse), the sweep on 32 rows of a linear of width n_0 (scaled by rows and
    (n/n_0)^2 per linear: the column loop with its trailing updates)."""
    import numpy as np
    import oracle
    import synth
    model, blas, blas_threads, affinity = _host_info()
    cores = blas_threads or affinity
    cfg = oracle.QuantConfig(bits=wl.bits, group_size=wl.group_size, sym=wl.sym, desc_act=wl.desc_act,
                             damp=wl.damp)
    tok_s = min(wl.tokens, synth.CHUNK)
    t_h, Hs = 0.0, []
    for xs in range(len(wl.xsets)):
        x = synth.activations_chunk_raw(wl, 0, xs)[:tok_s]
        xv = synth.bf16_value(x) if wl.dtype == "bf16" else x
        t0 = time.perf_counter()
        H, _ = oracle.hessian(xv)
        t_h += (time.perf_counter() - t0) * wl.tokens / tok_s
        Hs.append(H)
    t0 = time.perf_counter()
    p0 = oracle.prepare(Hs[0], cfg.damp, cfg.desc_act)
    t_p0 = time.perf_counter() - t0
    n0 = wl.xsets[0][0]
    t_p = sum(t_p0 * (x[0] / n0) ** 3 for x in wl.xsets)
    rows_s = 32
    lin0 = next(i for i, lin in enumerate(wl.linears) if lin.n == n0)
    wv = synth.weights(wl, lin0)[:rows_s].astype(np.float64)
    t0 = time.perf_counter()
    oracle.quantize_layer(wv, p0["U"], p0["perm"], p0["dead"], cfg)
    per_row = (time.perf_counter() - t0) / rows_s
    t_s = sum(per_row * lin.rows * (lin.n / n0) ** 2 for lin in wl.linears)
    total = t_h + t_p + t_s
    weights = sum(lin.rows * lin.n for lin in wl.linears)
    return {
        "value": weights / total, "unit": "weights/s", "cores": cores, "kind": "oracle",
        "cpu_model": model, "blas": blas, "blas_threads": blas_threads, "affinity_cores": affinity,
        "sample": (f"each set's Hessian on {tok_s} of {wl.tokens} tokens (time x{wl.tokens / tok_s:g}); prepare timed "
                   f"once at n={n0} ({t_p0:.2f} s) and scaled by (n/{n0})^3 per set; sweep on {rows_s} rows of "
                   f"width {n0} ({per_row * rows_s:.2f} s), scaled by rows and (n/{n0})^2 per linear"),
        "stage_s": {"hessian": t_h, "prepare": t_p, "quantize": t_s},
    }


def cpu_baseline(wl, w_raw, x_raw):
    """The float64 oracle on a bounded sample of the same layer, scaled to weights/s."""
    import numpy as np
    import oracle
    import synth
    model, blas, blas_threads, affinity = _host_info()
    cores = blas_threads or affinity
    rows, n = wl.rows, wl.n
    tok_s = min(wl.tokens, 8192)
    rows_s = min(rows, 256)
    xv = synth.bf16_value(x_raw[:tok_s]) if wl.dtype == "bf16" else x_raw[:tok_s]
    wv = synth.bf16_value(w_raw[:rows_s]) if wl.dtype == "bf16" else w_raw[:rows_s]
    cfg = oracle.QuantConfig(bits=wl.bits, group_size=wl.group_size, sym=wl.sym, desc_act=wl.desc_act,
                             damp=wl.damp)
    t0 = time.perf_counter()
    H, _ = oracle.hessian(xv)
    t1 = time.perf_counter()
    p = oracle.prepare(H, cfg.damp, cfg.desc_act)
    t2 = time.perf_counter()
    oracle.quantize_layer(wv.astype(np.float64), p["U"], p["perm"], p["dead"], cfg)
    t3 = time.perf_counter()
    t_h = (t1 - t0) * wl.tokens / tok_s
    t_p = t2 - t1
    t_s = (t3 - t2) * rows / rows_s
    total = t_h + t_p + t_s
    return {
        "value": rows * n / total, "unit": "weights/s", "cores": cores, "kind": "oracle",
        "cpu_model": model, "blas": blas, "blas_threads": blas_threads, "affinity_cores": affinity,
        "sample": (f"Hessian on {tok_s} of {wl.tokens} tokens (time x{wl.tokens / tok_s:g}), prepare at full "
                   f"n={n}, sweep on {rows_s} of {rows} rows (time x{rows / rows_s:g}; rows are independent); "
                   f"measured {t1 - t0:.2f}+{t2 - t1:.2f}+{t3 - t2:.2f} s"),
        "stage_s": {"hessian": t_h, "prepare": t_p, "quantize": t_s},
    }


# Llama-2-7B block linears with q/k/v and gate/up fused, as a decoder serves them
MM_SHAPES = (("qkv_proj", 12288, 4096), ("o_proj", 4096, 4096), ("gate_up_proj", 22016, 4096),
             ("down_proj", 4096, 11008))
MM_BLOCKS = 32
MM_BITS, MM_GS = 4, 128


def dequant_matmul_bench(g, torch, replays: int = 20, token_counts=(1, 16), pmc_probe: bool = False):
    """Decode through all linears of MM_BLOCKS blocks (each block its own copy
    of the packed weights, 3.4 GB in all, so nothing is served from cache),
    captured once as a graph of 4 * MM_BLOCKS launches and replayed.

    pmc_probe: instead, a 1 GiB device copy (counter calibration) and one
    eager one-token pass, for rocprofv3 --pmc passes."""
    import numpy as np
    import synth
    dev = torch.device("cuda")
    base = []
    for li, (name, rows, n) in enumerate(MM_SHAPES):
        qw = torch.from_numpy(synth.random_qweight(31 + li, rows, n, MM_BITS).view(np.int32)).to(dev)
        sc, ze, gi = synth.group_params(31 + li, rows, n, MM_BITS, MM_GS)
        layer = g.PackedLayer(qw, torch.from_numpy(sc).to(dev), torch.from_numpy(ze).to(dev),
                              torch.from_numpy(gi).to(dev), MM_BITS, MM_GS)
        assert layer.col_order is None
        base.append(layer)
        del qw
    packed = [[base[li].packed if b == 0 else base[li].packed.clone() for li in range(len(MM_SHAPES))]
              for b in range(MM_BLOCKS)]
    torch.cuda.synchronize()
    weight_bytes = sum(int(p.numel()) - 256 for blk in packed for p in blk)
    out = {"workload": (f"decode through the q/k/v (fused), o, gate/up (fused) and down projections of "
                        f"{MM_BLOCKS} Llama-2-7B-shaped blocks, {MM_BITS}-bit asym g{MM_GS}, desc_act off, "
                        f"fp16 activations and outputs; one graph replay = {4 * MM_BLOCKS} launches"),
           "packed_weight_bytes": weight_bytes, "by_tokens": {}}
    if pmc_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        A = [torch.from_numpy(synth.decode_activations_raw(41 + li, 1, n).view(np.float16)).to(dev)
             for li, (_, rows, n) in enumerate(MM_SHAPES)]
        Y = [torch.empty((1, rows), dtype=torch.float16, device=dev) for (_, rows, n) in MM_SHAPES]
        for b in range(MM_BLOCKS):
            for li, (_, rows, n) in enumerate(MM_SHAPES):
                g.gptq_matmul(A[li], packed[b][li], None, rows, n, MM_BITS, MM_GS, Y[li])
        torch.cuda.synchronize()
        _log(f"pmc probe done: 1 GiB copy + {4 * MM_BLOCKS} one-token launches")
        return None
    for M in token_counts:
        A = [torch.from_numpy(synth.decode_activations_raw(41 + li, M, n).view(np.float16)).to(dev)
             for li, (_, rows, n) in enumerate(MM_SHAPES)]
        Y = [torch.empty((M, rows), dtype=torch.float16, device=dev) for (_, rows, n) in MM_SHAPES]

        def run():
            for b in range(MM_BLOCKS):
                for li, (_, rows, n) in enumerate(MM_SHAPES):
                    g.gptq_matmul(A[li], packed[b][li], None, rows, n, MM_BITS, MM_GS, Y[li])

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / replays
        act_bytes = MM_BLOCKS * sum(M * n * 2 + M * rows * 2 for (_, rows, n) in MM_SHAPES)
        gbs = (weight_bytes + act_bytes) / (ms * 1e-3) / 1e9
        out["by_tokens"][str(M)] = {"ms_per_step": ms, "tokens_per_s": M / (ms * 1e-3), "GB_per_s": gbs,
                                    "algorithmic_bytes_per_step": weight_bytes + act_bytes}
        _log(f"dequant matmul, {M} token(s): {ms:.4f} ms per pass, {gbs:.0f} GB/s")
        del graph
    one = out["by_tokens"][str(token_counts[0])]
    out["roofline"] = {"kernel": "dequant_matmul_kernel<4,1,full> (one token)", "bound": "hbm",
                       "achieved": one["GB_per_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": one["GB_per_s"] / PEAK_HBM_GBS,
                       "traffic": _traffic(MM_TRAFFIC_FILE, MM_SRC, "bytes_per_pass"),
                       "note": "achieved: algorithmic bytes (packed codes, scale/zero words, activations, outputs) "
                               "over the graph replay time, inter-kernel gaps included; traffic: HBM bytes per "
                               "one-token pass from FETCH_SIZE/WRITE_SIZE"}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="attn4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    # quantize-config overrides (default: the workload's own); e.g. the pages'
    # "maximum precision" recipe: --group-size 32 --desc-act 1 --damp 0.005
    ap.add_argument("--bits", type=int, default=None, choices=[2, 3, 4, 8])
    ap.add_argument("--group-size", type=int, default=None, choices=[32, 64, 128, -1])
    ap.add_argument("--sym", type=int, default=None, choices=[0, 1, 2])
    ap.add_argument("--desc-act", type=int, default=None, choices=[0, 1])
    ap.add_argument("--damp", type=float, default=None)
    ap.add_argument("--matmul-only", action="store_true", help="only the dequant_matmul measurement")
    ap.add_argument("--no-matmul", action="store_true", help="skip the dequant_matmul measurement")
    ap.add_argument("--sequential", action="store_true",
                    help="block workloads: block-sequential calibration (the block forward between the stages)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="copy 1 GiB (counter calibration) then 3 Hessian launches; no timing output")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); the layer solve "
              f"is not sharded across GPUs in this build.", file=sys.stderr)
        return 2

    import torch
    import post_weight_quantization_13_amd as g
    import synth

    if args.matmul_only:
        torch.cuda.set_device(0)
        res = dequant_matmul_bench(g, torch, pmc_probe=args.pmc_probe)
        if res is not None:
            print(json.dumps({"dequant_matmul": res}), flush=True)
        return 0

    wl = synth.get(args.workload)
    over = {k: v for k, v in (("bits", args.bits), ("group_size", args.group_size), ("sym", args.sym),
                              ("desc_act", None if args.desc_act is None else bool(args.desc_act)),
                              ("damp", args.damp)) if v is not None}
    if over:
        wl = dataclasses.replace(wl, **over)
    if len(wl.linears) != 1:
        if args.sequential:
            return block_sequential_bench(args, wl, g, torch)
        return block_bench(args, wl, g, torch)
    torch.cuda.set_device(0)
    w_raw, x_raw, W, X = _device_inputs(wl, torch)
    rows, n, tokens = wl.rows, wl.n, wl.tokens
    cfg = g.Config(bits=wl.bits, group_size=wl.group_size, sym=wl.sym, desc_act=wl.desc_act,
                   damp_percent=wl.damp, block_size=wl.block_size)
    dev = W.device
    H = torch.empty((n, n), dtype=torch.float64, device=dev)
    U = torch.empty((n, n), dtype=torch.float32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    dead = torch.empty(n, dtype=torch.uint8, device=dev)
    qweight, scales, zeros, g_idx = g.alloc_outputs(rows, n, cfg, dev)
    ws_h = g.hessian_workspace(n, X)
    ws_p = g.workspace(g.gptq_prepare_workspace_bytes(n, cfg), dev)
    ws_q = g.workspace(g.gptq_quantize_workspace_bytes(rows, n, cfg), dev)
    torch.cuda.synchronize()

    if args.pmc_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        for _ in range(3):
            g.gptq_hessian_accumulate(H, 0, X, ws_h)
        torch.cuda.synchronize()
        _log("pmc probe done: 1 GiB copy + 3 Hessian launches")
        return 0

    # The stream-ordered entry points queue every step's work without a host
    # round trip; each step's positive-definiteness flag and loss land in
    # device memory and are checked once the timed steps are done.
    info = torch.full((args.warmup + args.steps,), -1, dtype=torch.int32, device=dev)
    loss = torch.full((args.warmup + args.steps,), -1.0, dtype=torch.float64, device=dev)

    def step(i):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        g.gptq_hessian_accumulate(H, 0, X, ws_h)
        ev[1].record()
        g.gptq_prepare_hinv_async(H, cfg, U, perm, dead, info[i:i + 1], ws_p)
        ev[2].record()
        g.gptq_quantize_layer_async(U, perm, dead, cfg, W, qweight, scales, zeros, g_idx, loss[i:i + 1], ws_q)
        ev[3].record()
        return ev

    for i in range(args.warmup):
        step(i)
        torch.cuda.synchronize()
        _log(f"warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        events.append(step(args.warmup + i))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _log(f"timed {args.steps} steps")
    _check_steps(info, loss)
    ms_step = (t1 - t0) * 1e3 / args.steps
    st = {k: sum(e[a].elapsed_time(e[b]) for e in events) / args.steps
          for k, a, b in (("hessian", 0, 1), ("prepare", 1, 2), ("quantize", 2, 3))}
    hess_flops = float(n) * (n + 1) * tokens
    hess_tflops = hess_flops / (st["hessian"] * 1e-3) / 1e12
    # the committed counter summary is for the default layer as configured
    traffic = _traffic() if wl.name == "attn4096" and not over else None
    out = {
        "metric": METRIC,
        "value": rows * n / (ms_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": wl.name, "rows": rows, "n": n, "tokens": tokens, "bits": wl.bits,
                   "group_size": wl.group_size, "sym": wl.sym, "desc_act": wl.desc_act, "damp": wl.damp,
                   "description": wl.description},
        "hessian_tflops": hess_tflops,
        "solve_weights_per_s": rows * n / ((st["prepare"] + st["quantize"]) * 1e-3),
        "stage_ms": st,
        "roofline": {
            "kernel": "syrk_dma_kernel<bf16> (Hessian)",
            "bound": "mfma",
            "achieved": hess_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": hess_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "layer_solve": layer_solve_roofline([(rows, n, wl.bits, wl.group_size)], [(n, tokens)], st),
        },
        "cpu_baseline": None,
    }
    if not args.no_matmul:
        del X, W, H, U, ws_h, ws_p, ws_q
        torch.cuda.empty_cache()
        out["dequant_matmul"] = dequant_matmul_bench(g, torch)
    if not args.no_cpu_baseline:
        _log("timing the float64 oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl, w_raw, x_raw)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

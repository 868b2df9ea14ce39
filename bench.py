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
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E (published)
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


def cpu_baseline(wl, w_raw, x_raw):
    """The float64 oracle on a bounded sample of the same layer, scaled to weights/s."""
    import numpy as np
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] or [0])
    except Exception:  # pragma: no cover
        cores = 0
    cores = cores or len(os.sched_getaffinity(0))
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
        print("bench.py times single-layer workloads", file=sys.stderr)
        return 2
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

    def step():
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        g.gptq_hessian_accumulate(H, 0, X, ws_h)
        ev[1].record()
        g.gptq_prepare_hinv(H, cfg, U, perm, dead, ws_p)
        ev[2].record()
        loss = g.gptq_quantize_layer(U, perm, dead, cfg, W, qweight, scales, zeros, g_idx, ws_q)
        ev[3].record()
        return ev, loss

    for i in range(args.warmup):
        step()
        _log(f"warmup step {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        events.append(step()[0])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    _log(f"timed {args.steps} steps")
    ms_step = (t1 - t0) * 1e3 / args.steps
    st = {k: sum(e[a].elapsed_time(e[b]) for e in events) / args.steps
          for k, a, b in (("hessian", 0, 1), ("prepare", 1, 2), ("quantize", 2, 3))}
    hess_flops = float(n) * (n + 1) * tokens
    hess_tflops = hess_flops / (st["hessian"] * 1e-3) / 1e12
    traffic = _traffic()
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
        "dtype": "bf16 mfma (fp32/fp64 accumulate) + fp64 cholesky + fp32 sweep",
        "data": "synthetic",
        "config": {"workload": wl.name, "rows": rows, "n": n, "tokens": tokens, "bits": wl.bits,
                   "group_size": wl.group_size, "sym": wl.sym, "desc_act": wl.desc_act, "damp": wl.damp,
                   "description": wl.description},
        "hessian_tflops": hess_tflops,
        "solve_weights_per_s": rows * n / ((st["prepare"] + st["quantize"]) * 1e-3),
        "stage_ms": st,
        "roofline": {
            "kernel": "syrk_mfma_kernel<bf16> (Hessian)",
            "bound": "mfma",
            "achieved": hess_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": hess_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
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

"""Benchmark of the QLoRA quantized linear layer on one MI355X.

Step = one training pass of an 8B-shaped MLP's three QLoRA projections
(gate and up 14336x4096, down 4096x14336; NF4 + double quantisation),
2048 tokens, LoRA r=16 alpha=32: forward (u, y) and backward (dx, dA, dB)
for each projection, inputs resident in HBM.  The headline value is the
step's algorithmic TFLOP/s (4MNK + 6Mr(K+N) per projection).

In the same run (reported beside the step):
  roofline     the forward GEMM timed alone in a loop with HIP events
  rows         each step row per projection, timed through the entry points
  few_tokens   the gate projection at 17 .. 512 tokens, forward and backward
  dropout      the gate projection with LoRA dropout 0.05 against without
  formats      the gate projection in each storage variant (blocks of 64 or
               128, with or without double quantisation)
  compute_dtype  the training step with bf16 and with fp16 compute
  decode_gemv  Llama-3-8B attention projection (4096x4096) at M = 1, 4, 16,
               packed-weight GB/s, rotating over 64 weight copies so the
               256 MB Infinity Cache cannot hold them
  quantize     NF4 + double quantisation and full dequantisation of an
               8B-shaped weight set, GB/s and bits/param
  optimizer    one AdamW step over an 8B model's LoRA factors
  cpu_baseline the CPU oracle on a bounded sample of the step (host cores)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s (%MFMA peak); decode GEMV packed-weight GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ROOFLINE_KERNEL = "k_gemm_fwd<256, unsigned short, unsigned short, true>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_gemm_fwd_mlp8b_gate.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def layer_flops(M, N, K, r):
    return 4 * M * N * K + 6 * M * r * (K + N)


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("gemm.hip", "common.h"):
        with open(os.path.join(ROOT, "qlora_fine_tuning_quantize_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def timed(fn, iters, warmup):
    """Average ms per call of fn() over `iters` calls, HIP events on the
    current stream, synchronised on both sides."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true", help="only the training step")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of the step instead of direct launches")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's data-parallel sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import qlora_fine_tuning_quantize_amd as q
    import synth_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = si.MLP_8B
    M, r, alpha = c["M"], c["r"], c["alpha"]

    # ---------------- training step: gate, up, down -----------------------
    projs = []
    for pi, (name, (N, K)) in enumerate(c["projs"].items()):
        t = si.linear_inputs(c["config"], M, N, K, r, sub=pi, device=dev)
        W = q.nf4_quantize(t["W"], double_quant=True)
        del t["W"]
        p = dict(name=name, N=N, K=K, W=W, x=t["x"], dy=t["dy"], A=t["A"], B=t["B"],
                 y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                 u=torch.empty((M, r), dtype=torch.float32, device=dev),
                 dx=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                 dA=torch.empty((r, K), dtype=torch.float32, device=dev),
                 dB=torch.empty((N, r), dtype=torch.float32, device=dev),
                 wsf=q.workspace(q.QL_OP_FWD, M, N, K, r, dev),
                 wsb=q.workspace(q.QL_OP_BWD, M, N, K, r, dev))
        projs.append(p)
    torch.cuda.synchronize()
    log("inputs ready")

    def step():
        for p in projs:
            q.qlora_linear_fwd(p["x"], p["W"], p["A"], p["B"], alpha, y=p["y"], u_save=p["u"],
                               ws=p["wsf"])
            q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"], alpha, u_saved=p["u"],
                               dx=p["dx"], dA=p["dA"], dB=p["dB"], ws=p["wsb"])

    flops_step = sum(layer_flops(M, p["N"], p["K"], r) for p in projs)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_eager = timed(step, args.steps, 0)
    log(f"eager step {ms_eager:.3f} ms")

    # With --graph the step's ~27 launches are captured once into a HIP graph
    # and replayed: every kernel still runs each step, only host launch gaps
    # go away (the GPU is the bottleneck here, so the two timings agree).
    # The first replay must reproduce the eager outputs bit for bit.
    outs = ("y", "u", "dx", "dA", "dB")
    eager_out = [{k: p[k].clone() for k in outs} for p in projs]
    graph = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for p in projs:
            for k in outs:
                p[k].zero_()
        graph.replay()
        torch.cuda.synchronize()
        for p, e in zip(projs, eager_out):
            for k in outs:
                if not torch.equal(p[k], e[k]):
                    raise RuntimeError(f"graph replay differs from the eager step ({p['name']} {k})")
        log("graph replay reproduces the eager step")
    run = graph.replay if graph is not None else step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    log(f"step {ms_step:.3f} ms  {tflops:.1f} TFLOP/s  (wall {wall:.2f} s for {args.steps} steps"
        f", {'graph replay' if graph is not None else 'eager'})")
    del graph, eager_out

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "8B-shaped MLP QLoRA training step: gate+up 14336x4096, down "
                               "4096x14336, NF4 block 64 + 8-bit double quant, 2048 tokens, "
                               "LoRA r=16 alpha=32, forward + backward (dx, dA, dB)",
                   "tokens": M, "rank": r, "alpha": alpha, "flop_per_step": flops_step},
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "launch": "HIP graph replay of the whole step" if args.graph else "direct launches",
        "ms_per_step_eager": round(ms_eager, 4),
    }

    # ---------------- roofline: the forward GEMM alone ------------------------
    # qlora_linear_fwd_u is one launch of the matrix-core forward kernel (u is
    # the u_save of the step), so events on this stream bracket exactly it.
    g = projs[0]
    fwd_ms = timed(lambda: q.qlora_linear_fwd_u(g["x"], g["W"], g["u"], g["B"], alpha,
                                                y=g["y"]), 50, 5)
    fwd_flops = 2 * M * g["N"] * g["K"] + 2 * M * r * g["N"]
    ach = fwd_flops / (fwd_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_sha") == kernel_source_sha():
            traffic = tr.get("hbm_bytes_per_launch")
    result["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                          "traffic": traffic, "kernel": ROOFLINE_KERNEL,
                          "launch": "qlora_linear_fwd_u gate 2048x14336x4096 (one GEMM launch)",
                          "ms_per_launch": round(fwd_ms, 4), "flop_per_launch": fwd_flops}
    log(f"fwd gate {fwd_ms:.3f} ms {ach:.1f} TFLOP/s")

    # ---------------- every row of the path, per projection -------------------
    # Each row is timed through the entry points alone (HIP events, 30 calls):
    #   a4 u = x A^T         = qlora_linear_bwd(u recomputed, dx = NULL)
    #                          - qlora_linear_bwd(u_saved, dx = NULL)
    #                          (the same u kernels as the forward's)
    #   a5 forward GEMM      = qlora_linear_fwd - a4 (the GEMM launches, with
    #                          its split-K sum where the shape splits)
    #   a6 LoRA gradients    = qlora_linear_bwd(u_saved, dx = NULL)   (g, dB, dA)
    #   a7 input gradient    = qlora_linear_bwd(u_saved) - the above
    # against MFMA peak (a5, a7) or HBM peak (a4, a6: bytes of x / dy read).
    rows = {}
    for p in projs:
        N, K = p["N"], p["K"]
        t_fwd = timed(lambda: q.qlora_linear_fwd(p["x"], p["W"], p["A"], p["B"], alpha, y=p["y"],
                                                 u_save=p["u"], ws=p["wsf"]), 30, 3)
        t_bwd = timed(lambda: q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"], alpha,
                                                 u_saved=p["u"], dx=p["dx"], dA=p["dA"],
                                                 dB=p["dB"], ws=p["wsb"]), 30, 3)
        t_lora = timed(lambda: q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"], alpha,
                                                  u_saved=p["u"], need_dx=False, dA=p["dA"],
                                                  dB=p["dB"], ws=p["wsb"]), 30, 3)
        t_lora_u = timed(lambda: q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"],
                                                    alpha, need_dx=False, dA=p["dA"], dB=p["dB"],
                                                    ws=p["wsb"]), 30, 3)
        t_u = t_lora_u - t_lora
        a5 = 2 * M * N * K + 2 * M * r * N
        a7 = 2 * M * N * K + 2 * M * r * K
        by_x, by_dy = M * K * 2, M * N * 2
        rec = {
            "a4_u": {"us": round(t_u * 1e3, 2), "bytes": by_x},
            "a5_fwd_gemm": {"us": round((t_fwd - t_u) * 1e3, 2), "flop": a5},
            "a6_lora_grads": {"us": round(t_lora * 1e3, 2), "bytes": by_x + 2 * by_dy},
            "a7_dx_gemm": {"us": round((t_bwd - t_lora) * 1e3, 2), "flop": a7},
        }
        for k, v in rec.items():
            sec = v["us"] * 1e-6
            if "flop" in v:
                v["TFLOPs"] = round(v["flop"] / sec / 1e12, 1)
                v["frac_mfma"] = round(v["TFLOPs"] / PEAK_BF16_TFLOPS, 4)
            else:
                v["GBps"] = round(v["bytes"] / sec / 1e9, 1)
                v["frac_hbm"] = round(v["GBps"] / PEAK_HBM_GBS, 4)
        rows[p["name"]] = rec
        log(f"rows {p['name']}: " + ", ".join(f"{k} {v['us']} us" for k, v in rec.items()))
    result["rows"] = rows
    del projs, g
    torch.cuda.empty_cache()

    if not args.no_extras:
        result["few_tokens"] = bench_few_tokens(q, si, dev)
        result["dropout"] = bench_dropout(q, si, dev)
        result["formats"] = bench_formats(q, si, dev)
        result["compute_dtype"] = bench_compute_dtype(q, si, dev)
        result["decode_gemv"] = bench_decode(q, si, dev)
        result["quantize"] = bench_quantize(q, si, dev)
        result["optimizer"] = bench_adamw(q, si, dev)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(si, M, r, alpha)
    print(json.dumps(result), flush=True)


def bench_few_tokens(q, si, dev, token_counts=(17, 64, 128, 256, 512)):
    """The gate projection (14336x4096, NF4 + double quant, r=16) with few
    tokens: forward (u + y) and backward (g, dA, dB, dx) per call, eager."""
    c = si.MLP_8B
    N, K = c["projs"]["gate"]
    r, alpha = c["r"], c["alpha"]
    W = None
    out = {"workload": "gate projection 14336x4096 NF4 + double quant, r=16, alpha=32, bf16, "
                       "forward and backward per call (eager, every launch of the call)",
           "unit": "us"}
    for M in token_counts:
        t = si.linear_inputs(c["config"], M, N, K, r, device=dev)
        if W is None:
            W = q.nf4_quantize(t["W"], double_quant=True)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        u = torch.empty((M, r), dtype=torch.float32, device=dev)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        dA = torch.empty((r, K), dtype=torch.float32, device=dev)
        dB = torch.empty((N, r), dtype=torch.float32, device=dev)
        wsf = q.workspace(q.QL_OP_FWD, M, N, K, r, dev)
        wsb = q.workspace(q.QL_OP_BWD, M, N, K, r, dev)
        tf = timed(lambda: q.qlora_linear_fwd(t["x"], W, t["A"], t["B"], alpha, y=y, u_save=u,
                                              ws=wsf), 30, 3)
        tb = timed(lambda: q.qlora_linear_bwd(t["dy"], t["x"], W, t["A"], t["B"], alpha,
                                              u_saved=u, dx=dx, dA=dA, dB=dB, ws=wsb), 30, 3)
        fl = layer_flops(M, N, K, r)
        out[f"M{M}"] = {"fwd_us": round(tf * 1e3, 2), "bwd_us": round(tb * 1e3, 2),
                        "fwd_bwd_TFLOPs": round(fl / ((tf + tb) * 1e-3) / 1e12, 1),
                        "fwd_packed_weight_GBps": round(W.storage_bytes() / (tf * 1e-3) / 1e9, 1)}
        log(f"few tokens M={M}: fwd {tf * 1e3:.1f} us, bwd {tb * 1e3:.1f} us")
        del t, y, u, dx, dA, dB, wsf, wsb
    del W
    torch.cuda.empty_cache()
    return out


def bench_dropout(q, si, dev):
    """LoRA dropout (p = 0.05) on the gate projection at 2048 tokens: the
    forward + backward with dropout against the same without it."""
    c = si.MLP_8B
    N, K = c["projs"]["gate"]
    M, r, alpha = c["M"], c["r"], c["alpha"]
    t = si.linear_inputs(c["config"], M, N, K, r, device=dev)
    W = q.nf4_quantize(t["W"], double_quant=True)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    u = torch.empty((M, r), dtype=torch.float32, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    wsf = q.workspace(q.QL_OP_FWD, M, N, K, r, dev)
    wsb = q.workspace(q.QL_OP_BWD, M, N, K, r, dev)

    def plain():
        q.qlora_linear_fwd(t["x"], W, t["A"], t["B"], alpha, y=y, u_save=u, ws=wsf)
        q.qlora_linear_bwd(t["dy"], t["x"], W, t["A"], t["B"], alpha, u_saved=u, dx=dx, dA=dA,
                           dB=dB, ws=wsb)

    def dropped():
        q.qlora_linear_fwd_dropout(t["x"], W, t["A"], t["B"], alpha, 0.05, 1234, y=y, u_save=u,
                                   ws=wsf)
        q.qlora_linear_bwd_dropout(t["dy"], t["x"], W, t["A"], t["B"], alpha, 0.05, 1234,
                                   u_saved=u, dx=dx, dA=dA, dB=dB, ws=wsb)

    tp = timed(plain, 20, 3)
    td = timed(dropped, 20, 3)
    fl = layer_flops(M, N, K, r)
    out = {"workload": "gate projection 2048x14336x4096 NF4 + double quant, r=16, lora_dropout "
                       "0.05, forward + backward", "unit": "us",
           "with_dropout_us": round(td * 1e3, 2), "without_us": round(tp * 1e3, 2),
           "with_dropout_TFLOPs": round(fl / (td * 1e-3) / 1e12, 1),
           "overhead_frac": round(td / tp - 1.0, 4)}
    log(f"dropout: {td * 1e3:.1f} us with, {tp * 1e3:.1f} us without")
    del t, W, y, u, dx, dA, dB, wsf, wsb
    torch.cuda.empty_cache()
    return out


def bench_formats(q, si, dev):
    """The NF4 storage variants on the gate projection (14336x4096, 2048
    tokens, r=16): blocks of 64 or 128 weights, with or without double
    quantisation of the block constants.  Per format: bits/param, quantise
    time of the weight, and the layer's forward + backward."""
    c = si.MLP_8B
    N, K = c["projs"]["gate"]
    M, r, alpha = c["M"], c["r"], c["alpha"]
    t = si.linear_inputs(c["config"], M, N, K, r, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    u = torch.empty((M, r), dtype=torch.float32, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    wsf = q.workspace(q.QL_OP_FWD, M, N, K, r, dev)
    wsb = q.workspace(q.QL_OP_BWD, M, N, K, r, dev)
    wsq = q.workspace(q.QL_OP_QUANTIZE, 0, N, K, 0, dev)
    out = {"workload": "gate projection 2048x14336x4096, r=16, alpha=32, bf16: quantise the "
                       "weight, then forward + backward", "unit": "us"}
    fl = layer_flops(M, N, K, r)
    fmts = [(block, dq) for block in (64, 128) for dq in (True, False)]
    Ws = {}
    for block, dq in fmts:
        W = q.NF4Weight.empty(N, K, dq, dev, block=block)
        tq = timed(lambda: q.nf4_quantize(t["W"], dq, out=W, ws=wsq, block=block), 20, 3)
        Ws[(block, dq)] = (W, tq)

    def fb(W):
        q.qlora_linear_fwd(t["x"], W, t["A"], t["B"], alpha, y=y, u_save=u, ws=wsf)
        q.qlora_linear_bwd(t["dy"], t["x"], W, t["A"], t["B"], alpha, u_saved=u, dx=dx, dA=dA,
                           dB=dB, ws=wsb)
    timed(lambda: fb(Ws[fmts[0]][0]), 20, 0)  # clocks up before the first timed format
    for block, dq in fmts:
        W, tq = Ws[(block, dq)]
        tl = timed(lambda: fb(W), 10, 3)
        key = f"block{block}_{'dq' if dq else 'fp32absmax'}"
        out[key] = {"bits_per_param": round(8 * W.storage_bytes() / (N * K), 5),
                    "quantize_us": round(tq * 1e3, 2), "fwd_bwd_us": round(tl * 1e3, 2),
                    "fwd_bwd_TFLOPs": round(fl / (tl * 1e-3) / 1e12, 1)}
        log(f"format {key}: {out[key]}")
    del Ws
    del t, y, u, dx, dA, dB, wsf, wsb, wsq
    torch.cuda.empty_cache()
    return out


def bench_compute_dtype(q, si, dev, rounds=3, iters=10):
    """The 8B-MLP training step (gate, up, down; 2048 tokens, r=16) with bf16
    and with fp16 compute (activations, dequantised weight and LoRA factors
    in the dtype, fp32 accumulation).  The two are timed alternately,
    `rounds` times `iters` steps each; the median per dtype is reported."""
    c = si.MLP_8B
    M, r, alpha = c["M"], c["r"], c["alpha"]
    steps, fl = {}, 0
    for dt in (torch.bfloat16, torch.float16):
        projs = []
        for pi, (name, (N, K)) in enumerate(c["projs"].items()):
            t = si.linear_inputs(c["config"], M, N, K, r, act_dtype=dt, w_dtype=dt, lora_dtype=dt,
                                 sub=pi, device=dev)
            W = q.nf4_quantize(t["W"], double_quant=True)
            del t["W"]
            projs.append(dict(t, W=W, y=torch.empty((M, N), dtype=dt, device=dev),
                              u=torch.empty((M, r), dtype=torch.float32, device=dev),
                              dx=torch.empty((M, K), dtype=dt, device=dev),
                              dA=torch.empty((r, K), dtype=torch.float32, device=dev),
                              dB=torch.empty((N, r), dtype=torch.float32, device=dev),
                              wsf=q.workspace(q.QL_OP_FWD, M, N, K, r, dev),
                              wsb=q.workspace(q.QL_OP_BWD, M, N, K, r, dev)))
            if dt == torch.bfloat16:
                fl += layer_flops(M, N, K, r)

        def step(projs=projs):
            for p in projs:
                q.qlora_linear_fwd(p["x"], p["W"], p["A"], p["B"], alpha, y=p["y"],
                                   u_save=p["u"], ws=p["wsf"])
                q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"], alpha,
                                   u_saved=p["u"], dx=p["dx"], dA=p["dA"], dB=p["dB"],
                                   ws=p["wsb"])
        steps[dt] = step
    times = {dt: [] for dt in steps}
    for dt, fn in steps.items():
        timed(fn, 3, 2)
    for _ in range(rounds):
        for dt, fn in steps.items():
            times[dt].append(timed(fn, iters, 1))
    out = {"workload": "8B-MLP training step (gate, up, down fwd + bwd), 2048 tokens, r=16, "
                       "NF4 + double quant", "unit": "ms"}
    for dt, ts in times.items():
        ms = sorted(ts)[len(ts) // 2]
        key = "bf16" if dt == torch.bfloat16 else "fp16"
        out[key] = {"ms_per_step": round(ms, 3), "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 1)}
        log(f"compute dtype {key}: {out[key]}")
    del steps
    torch.cuda.empty_cache()
    return out


def bench_decode(q, si, dev, copies=64, iters=1000):
    c = si.DECODE
    N, K, r, alpha = c["N"], c["K"], c["r"], c["alpha"]
    t = si.linear_inputs(c["config"], 16, N, K, r, with_dy=False, device=dev)
    Ws = []
    for i in range(copies):
        w = t["W"] if i == 0 else si.normal((N, K), 0.02, si.seed_of(2, 1, i), device=dev)
        Ws.append(q.nf4_quantize(w, double_quant=True))
    del w
    packed_bytes = sum(q.nf4_sizes(N, K, True))
    out = {"workload": "Llama-3-8B attention projection 4096x4096 NF4 + double quant, r=16, "
                       "alpha=32, bf16, forward only; 64 rotating weight copies",
           "unit": "GB/s", "packed_weight_bytes": packed_bytes}
    for M in c["Ms"]:
        x = t["x"][:M].contiguous()
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = q.workspace(q.QL_OP_FWD, M, N, K, r, dev)
        state = {"i": 0}

        def call():
            W = Ws[state["i"] % copies]
            state["i"] += 1
            q.qlora_linear_fwd(x, W, t["A"], t["B"], alpha, y=y, ws=ws)

        ms_eager = timed(call, iters, 50)
        # The same launches captured once in a HIP graph (one call per weight
        # copy) and replayed: the GPU-side rate, without the Python binding's
        # per-call overhead, which is of the order of the kernel itself.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(copies):
                call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(copies):
                call()
        reps = max(1, iters // copies)
        ms = timed(g.replay, reps, 3) / copies
        del g
        gbs = packed_bytes / (ms * 1e-3) / 1e9
        out[f"M{M}"] = {"us_per_call": round(ms * 1e3, 3), "packed_GBps": round(gbs, 1),
                        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "launch": "graph replay",
                        "us_per_call_eager": round(ms_eager * 1e3, 3)}
        log(f"decode M={M}: {ms * 1e3:.2f} us/call in a graph ({gbs:.0f} GB/s packed), "
            f"{ms_eager * 1e3:.2f} us/call eager")
    del Ws
    torch.cuda.empty_cache()
    return out


def bench_adamw(q, si, dev):
    """One AdamW step over all LoRA factors of an 8B-shaped model (r = 16 on
    q, k, v, o, gate, up, down of 32 layers) kept as one flat fp32 buffer
    with fp32 moments and a bf16 copy for the layers: HBM-bound, 30 bytes per
    parameter (p, g, m, v read; p, m, v, bf16 p written)."""
    cfg = si.WEIGHTSET_8B
    r = 16
    n = 0
    for _ in range(cfg["layers"]):
        for (N, K) in cfg["shapes"].values():
            n += r * K + N * r
    n = (n + 3) // 4 * 4
    gen = torch.Generator(device=dev).manual_seed(7)
    p = torch.randn(n, device=dev, generator=gen) * 0.01
    g = torch.randn(n, device=dev, generator=gen) * 1e-3
    m = torch.zeros(n, device=dev)
    v = torch.zeros(n, device=dev)
    pb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    state = {"t": 0}

    def step():
        state["t"] += 1
        q.adamw_step(p, g, m, v, lr=2e-4, step=state["t"], param_bf16=pb)

    ms = timed(step, 50, 5)
    nbytes = 30 * n
    gbs = nbytes / (ms * 1e-3) / 1e9
    log(f"adamw {n} params: {ms * 1e3:.1f} us, {gbs:.0f} GB/s")
    out = {"workload": "AdamW step over an 8B-shaped model's LoRA factors (r=16 on q,k,v,o,gate,"
                       "up,down x 32 layers), fp32 params and moments + bf16 copy",
           "params": n, "us_per_step": round(ms * 1e3, 2), "bytes_per_step": nbytes,
           "GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    del p, g, m, v, pb
    torch.cuda.empty_cache()
    return out


def bench_quantize(q, si, dev):
    """8B-shaped weight set (32 layers x q,k,v,o,gate,up,down), bf16 N(0,0.02)
    with 0.1% outliers at 20 sigma: quantise (+ double quant) and dequantise
    every tensor once per pass."""
    cfg = si.WEIGHTSET_8B
    ws_list, q_list, out_list = [], [], []
    n_total = 0
    for layer in range(cfg["layers"]):
        for name in cfg["shapes"]:
            w = si.weightset_tensor(layer, name, device=dev)
            ws_list.append(w)
            q_list.append(q.NF4Weight.empty(w.shape[0], w.shape[1], True, dev))
            n_total += w.numel()
    maxn = max(w.numel() for w in ws_list)
    wsq = q.workspace(q.QL_OP_QUANTIZE, 0, 1, maxn, 0, dev)
    deq = torch.empty(maxn, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"weight set ready: {n_total} params")

    def quant_all():
        for w, qq in zip(ws_list, q_list):
            q.nf4_quantize(w, double_quant=True, out=qq, ws=wsq)

    def dequant_all():
        for qq in q_list:
            q.nf4_dequantize(qq, out=deq[:qq.rows * qq.cols].view(qq.rows, qq.cols))

    qms = timed(quant_all, 3, 1)
    dms = timed(dequant_all, 3, 1)
    stored = sum(qq.storage_bytes() for qq in q_list)
    q_bytes = 2 * n_total + stored
    d_bytes = stored + 2 * n_total
    out = {"workload": "8B-shaped weight set, 32 layers x {q,k,v,o,gate,up,down}, bf16 "
                       "N(0,0.02) + 0.1% outliers at 20 sigma, NF4 + double quant",
           "params": n_total, "bits_per_param": round(8 * stored / n_total, 5),
           "quantize_ms": round(qms, 3), "quantize_GBps": round(q_bytes / (qms * 1e-3) / 1e9, 1),
           "dequantize_ms": round(dms, 3),
           "dequantize_GBps": round(d_bytes / (dms * 1e-3) / 1e9, 1), "unit": "GB/s"}
    out["quantize_hbm_frac"] = round(out["quantize_GBps"] / PEAK_HBM_GBS, 4)
    out["dequantize_hbm_frac"] = round(out["dequantize_GBps"] / PEAK_HBM_GBS, 4)
    log(f"quantize {qms:.2f} ms ({out['quantize_GBps']} GB/s), dequantize {dms:.2f} ms "
        f"({out['dequantize_GBps']} GB/s), {out['bits_per_param']} bits/param")
    del ws_list, q_list, deq
    torch.cuda.empty_cache()
    return out


def cpu_baseline(si, M, r, alpha, target_s=10.0):
    """The CPU oracle on a bounded sample: the gate projection's forward and
    backward (dequantisation included) for a slice of the token batch sized
    so that the run takes about target_s seconds on this host; TFLOP/s."""
    from oracle import oracle as orc
    c = si.MLP_8B
    N, K = c["projs"]["gate"]
    bits = lambda v: v.contiguous().view(torch.int16).numpy().view("uint16")

    def run(rows):
        t = si.linear_inputs(c["config"], rows, N, K, r, sub=0)
        Wh, xh, Ah, Bh, dyh = (bits(t[k]) for k in ("W", "x", "A", "B", "dy"))
        st = orc.quantize_nf4(Wh, double_quant=True)
        t0 = time.perf_counter()
        w_hat = orc.dequantize(st).reshape(N, K)
        orc.linear_fwd(xh, w_hat, Ah, Bh, alpha, r)
        orc.linear_bwd(xh, w_hat, Ah, Bh, dyh, alpha, r)
        return time.perf_counter() - t0

    dt = run(64)
    rows = int(min(M, max(64, 64 * target_s / max(dt, 1e-3))) // 64 * 64)
    if rows > 64:
        dt = run(rows)
    flops = layer_flops(rows, N, K, r)
    log(f"cpu oracle: {dt:.2f} s for {flops / 1e9:.1f} GFLOP ({rows} tokens)")
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": orc.num_threads(),
            "kind": "oracle",
            "sample": f"gate projection 14336x4096, {rows} of the {M} tokens, forward + backward "
                      f"including dequantisation, fp64 accumulation, {dt:.1f} s"}


if __name__ == "__main__":
    main()

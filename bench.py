"""Benchmark of the QLoRA quantized linear layer on one MI355X.

Step = one training pass of a 70B-shaped MLP's three QLoRA projections
(gate and up 28672x8192, down 8192x28672; NF4 block 64 + 8-bit double
quantisation), 4096 tokens, LoRA r=64 alpha=16: forward (u, y) and backward
(dx, dA, dB) for each projection, inputs resident in HBM.  The headline value
is the step's algorithmic TFLOP/s (4MNK + 6Mr(K+N) per projection).  This is
the largest training configuration of the layer that fits one GPU.

In the same run (reported beside the step):
  roofline     the dominant kernel (the forward GEMM of the gate projection)
               timed alone with HIP events, against the bf16 matrix peak
  rows         each step row per projection, timed through the entry points
  mlp_8b       the same step on an 8B-shaped MLP (gate/up 14336x4096, down
               4096x14336, 2048 tokens, r=16, alpha=32)
  few_tokens   the 8B gate (and down) projection at 17 .. 512 tokens, forward and backward
  dropout      the 8B gate projection with LoRA dropout 0.05 against without
  formats      the 8B gate projection in each storage variant (blocks of 64
               or 128, with or without double quantisation)
  compute_dtype  the 8B training step with bf16 and with fp16 compute
  decode_gemv  Llama-3-8B attention projection (4096x4096) at M = 1, 4, 16,
               packed-weight GB/s, rotating over 64 weight copies so the
               256 MB Infinity Cache cannot hold them; per-call median and
               p10/p90; the oracle's GEMV on the host beside it; decode-sized
               calls on larger weights
  quantize     NF4 + double quantisation and full dequantisation of an
               8B-shaped weight set, GB/s and bits/param (quantised one layer
               per call, and one weight per call); the oracle's
               quantise + dequantise of layers 0 and 31 on the host beside it
  small_fp32   the fp32 256x256 layer (4 tokens, r=8) forward + backward,
               1000 calls, and the single-thread oracle beside it
  optimizer    one AdamW step over an 8B model's LoRA factors
  cpu_baseline the CPU oracle on a bounded sample of the step (host cores)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Prints exactly one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s (%MFMA peak); decode GEMV packed-weight GB/s"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
ROOFLINE_KERNEL = "k_gemm_fwd<256, unsigned short, unsigned short, true>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_k_gemm_fwd_mlp70b_gate.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace_bench_mlp70b.txt")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def layer_flops(M, N, K, r):
    return 4 * M * N * K + 6 * M * r * (K + N)


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("csrc/gemm.hip", "csrc/common.h", "build.py"):
        with open(os.path.join(ROOT, "qlora_fine_tuning_quantize_amd", f), "rb") as fh:
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


def timed_each(fn, iters, warmup):
    """ms of each of `iters` calls of fn(), each bracketed by its own HIP
    events on the current stream (sorted)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    return sorted(s.elapsed_time(e) for s, e in evs)


def pct(sorted_vals, p):
    i = min(len(sorted_vals) - 1, max(0, int(round(p / 100.0 * (len(sorted_vals) - 1)))))
    return sorted_vals[i]


def host_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "cpus_available": avail}


def trace_median_us(kernel_prefix, grid):
    """The rocprofv3 kernel-trace median of a kernel launch shape, from the
    committed summary of this benchmark (None if absent)."""
    if not os.path.exists(TRACE_FILE):
        return None
    with open(TRACE_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) >= 6 and line.startswith(kernel_prefix) and str(grid) in parts:
                try:
                    gi = parts.index(str(grid))
                    return float(parts[gi + 3])
                except (ValueError, IndexError):
                    return None
    return None


def make_projs(q, si, c, dev, act=torch.bfloat16):
    M, r = c["M"], c["r"]
    projs = []
    for pi, (name, (N, K)) in enumerate(c["projs"].items()):
        t = si.linear_inputs(c["config"], M, N, K, r, act_dtype=act, w_dtype=act, lora_dtype=act,
                             sub=pi, device=dev)
        W = q.nf4_quantize(t["W"], double_quant=True)
        del t["W"]
        projs.append(dict(name=name, N=N, K=K, W=W, x=t["x"], dy=t["dy"], A=t["A"], B=t["B"],
                          y=torch.empty((M, N), dtype=act, device=dev),
                          u=torch.empty((M, r), dtype=torch.float32, device=dev),
                          dx=torch.empty((M, K), dtype=act, device=dev),
                          dA=torch.empty((r, K), dtype=torch.float32, device=dev),
                          dB=torch.empty((N, r), dtype=torch.float32, device=dev),
                          wsf=q.workspace(q.QL_OP_FWD, M, N, K, r, dev),
                          wsb=q.workspace(q.QL_OP_BWD, M, N, K, r, dev)))
    return projs


def step_fn(q, projs, alpha):
    def step():
        for p in projs:
            q.qlora_linear_fwd(p["x"], p["W"], p["A"], p["B"], alpha, y=p["y"], u_save=p["u"],
                               ws=p["wsf"])
            q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"], alpha, u_saved=p["u"],
                               dx=p["dx"], dA=p["dA"], dB=p["dB"], ws=p["wsb"])
    return step


def row_times(q, projs, M, r, alpha, iters=20):
    """Each row of the path per projection, timed through the entry points
    alone (HIP events):
      a4 u = x A^T       = qlora_linear_bwd(u recomputed, dx = NULL)
                           - qlora_linear_bwd(u_saved, dx = NULL)
      a5 forward GEMM    = qlora_linear_fwd - a4 (with its split-K sum)
      a6 LoRA gradients  = qlora_linear_bwd(u_saved, dx = NULL)   (g, dB, dA)
      a7 input gradient  = qlora_linear_bwd(u_saved) - the above
    against MFMA peak (a5, a7) or HBM peak (a4, a6: bytes of x / dy read)."""
    rows = {}
    for p in projs:
        N, K = p["N"], p["K"]
        t_fwd = timed(lambda: q.qlora_linear_fwd(p["x"], p["W"], p["A"], p["B"], alpha, y=p["y"],
                                                 u_save=p["u"], ws=p["wsf"]), iters, 3)
        t_bwd = timed(lambda: q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"], alpha,
                                                 u_saved=p["u"], dx=p["dx"], dA=p["dA"],
                                                 dB=p["dB"], ws=p["wsb"]), iters, 3)
        t_lora = timed(lambda: q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"], alpha,
                                                  u_saved=p["u"], need_dx=False, dA=p["dA"],
                                                  dB=p["dB"], ws=p["wsb"]), iters, 3)
        t_lora_u = timed(lambda: q.qlora_linear_bwd(p["dy"], p["x"], p["W"], p["A"], p["B"],
                                                    alpha, need_dx=False, dA=p["dA"], dB=p["dB"],
                                                    ws=p["wsb"]), iters, 3)
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
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-extras", action="store_true", help="only the training step")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of a HIP graph of the step instead of direct launches")
    ap.add_argument("--only", default="",
                    help="comma-separated extras to run (default: all), e.g. decode_gemv")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's data-parallel sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import qlora_fine_tuning_quantize_amd as q
    import synth_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = si.MLP_70B
    M, r, alpha = c["M"], c["r"], c["alpha"]

    # ---------------- training step: gate, up, down -----------------------
    projs = make_projs(q, si, c, dev)
    torch.cuda.synchronize()
    log("inputs ready")
    step = step_fn(q, projs, alpha)
    flops_step = sum(layer_flops(M, p["N"], p["K"], r) for p in projs)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_eager = timed(step, args.steps, 0)
    log(f"eager step {ms_eager:.3f} ms")

    # With --graph the step's launches are captured once into a HIP graph and
    # replayed: every kernel still runs each step, only host launch gaps go
    # away.  The first replay must reproduce the eager outputs bit for bit.
    outs = ("y", "u", "dx", "dA", "dB")
    graph = None
    if args.graph:
        eager_out = [{k: p[k].clone() for k in outs} for p in projs]
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
        del eager_out
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
    del graph

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "70B-shaped MLP QLoRA training step: gate+up 28672x8192, down "
                               "8192x28672, NF4 block 64 + 8-bit double quant, 4096 tokens, "
                               "LoRA r=64 alpha=16, forward + backward (dx, dA, dB)",
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
                                                y=g["y"]), 20, 3)
    fwd_flops = 2 * M * g["N"] * g["K"] + 2 * M * r * g["N"]
    ach = fwd_flops / (fwd_ms * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_sha") == kernel_source_sha():
            traffic = tr.get("hbm_bytes_per_launch")
    grid = ((M + 255) // 256) * ((g["N"] + 255) // 256) * 512
    prof_us = trace_median_us("qlora::k_gemm_fwd<256, unsigned short, unsigned short, true>",
                              grid)
    result["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                          "traffic": traffic, "kernel": ROOFLINE_KERNEL,
                          "launch": f"qlora_linear_fwd_u gate {M}x{g['N']}x{g['K']} r={r} "
                                    "(one GEMM launch)",
                          "ms_per_launch": round(fwd_ms, 4), "flop_per_launch": fwd_flops,
                          "profile_median_us": prof_us,
                          "profile_ratio": (round(fwd_ms * 1e3 / prof_us, 4)
                                            if prof_us else None)}
    log(f"fwd gate {fwd_ms:.3f} ms {ach:.1f} TFLOP/s (profile median {prof_us} us)")
    result["rows"] = row_times(q, projs, M, r, alpha, iters=10)
    del projs, g
    torch.cuda.empty_cache()

    if not args.no_extras:
        cpu = not args.no_cpu
        extras = {
            "mlp_8b": lambda: bench_mlp8b(q, si, dev, args.steps, args.warmup),
            "few_tokens": lambda: bench_few_tokens(q, si, dev),
            "dropout": lambda: bench_dropout(q, si, dev),
            "formats": lambda: bench_formats(q, si, dev),
            "compute_dtype": lambda: bench_compute_dtype(q, si, dev),
            "decode_gemv": lambda: bench_decode(q, si, dev, with_cpu=cpu),
            "quantize": lambda: bench_quantize(q, si, dev, with_cpu=cpu),
            "small_fp32": lambda: bench_small_fp32(q, si, dev, with_cpu=cpu),
            "optimizer": lambda: bench_adamw(q, si, dev),
        }
        only = [e for e in args.only.split(",") if e]
        for name, fn in extras.items():
            if not only or name in only:
                result[name] = fn()
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(si, c)
    print(json.dumps(result), flush=True)


def bench_mlp8b(q, si, dev, steps, warmup):
    """The training step on the 8B-shaped MLP (gate/up 14336x4096, down
    4096x14336, 2048 tokens, r=16, alpha=32), with its rows."""
    c = si.MLP_8B
    M, r, alpha = c["M"], c["r"], c["alpha"]
    projs = make_projs(q, si, c, dev)
    step = step_fn(q, projs, alpha)
    fl = sum(layer_flops(M, p["N"], p["K"], r) for p in projs)
    ms = timed(step, steps, warmup)
    g = projs[0]
    fwd_ms = timed(lambda: q.qlora_linear_fwd_u(g["x"], g["W"], g["u"], g["B"], alpha,
                                                y=g["y"]), 30, 3)
    fwd_flops = 2 * M * g["N"] * g["K"] + 2 * M * r * g["N"]
    out = {"workload": "8B-shaped MLP QLoRA training step: gate+up 14336x4096, down 4096x14336, "
                       "NF4 block 64 + 8-bit double quant, 2048 tokens, LoRA r=16 alpha=32, "
                       "forward + backward (dx, dA, dB)",
           "ms_per_step": round(ms, 4), "TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2),
           "flop_per_step": fl,
           "fwd_gemm_gate": {"ms_per_launch": round(fwd_ms, 4),
                             "TFLOPs": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 1)},
           "rows": row_times(q, projs, M, r, alpha, iters=20)}
    log(f"8B step {ms:.3f} ms {out['TFLOPs']} TFLOP/s")
    del projs
    torch.cuda.empty_cache()
    return out


def bench_few_tokens(q, si, dev, token_counts=(17, 64, 128, 256, 512)):
    """The gate projection (14336x4096, NF4 + double quant, r=16) with few
    tokens: forward (u + y) and backward (g, dA, dB, dx) per call, eager;
    the down projection (4096x14336, the long contraction) under "down"."""
    c = si.MLP_8B
    r, alpha = c["r"], c["alpha"]
    out = {"workload": "gate projection 14336x4096 NF4 + double quant, r=16, alpha=32, bf16, "
                       "forward and backward per call (eager, every launch of the call); "
                       "down: the down projection 4096x14336, the same calls",
           "unit": "us"}
    for proj in ("gate", "down"):
        N, K = c["projs"][proj]
        dst = out if proj == "gate" else out.setdefault("down", {})
        W = None
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
            dst[f"M{M}"] = {"fwd_us": round(tf * 1e3, 2), "bwd_us": round(tb * 1e3, 2),
                            "fwd_bwd_TFLOPs": round(fl / ((tf + tb) * 1e-3) / 1e12, 1),
                            "fwd_packed_weight_GBps": round(W.storage_bytes() / (tf * 1e-3) / 1e9,
                                                            1)}
            log(f"few tokens {proj} M={M}: fwd {tf * 1e3:.1f} us, bwd {tb * 1e3:.1f} us")
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
    steps, keep = {}, []
    fl = 0
    for dt in (torch.bfloat16, torch.float16):
        projs = make_projs(q, si, c, dev, act=dt)
        keep.append(projs)
        if dt == torch.bfloat16:
            fl = sum(layer_flops(M, p["N"], p["K"], r) for p in projs)
        steps[dt] = step_fn(q, projs, alpha)
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
    del steps, keep
    torch.cuda.empty_cache()
    return out


def _decode_rate(q, si, dev, N, K, r, alpha, Ms, copies, replays, cfg, tag):
    """Forward calls at decode token counts on `copies` distinct quantised
    N x K weights, rotated so that the 256 MB Infinity Cache cannot hold
    them: one graph of `copies` calls (one per weight) is replayed
    `replays` times, each replay timed with its own HIP events; per-call
    figures are replay time / copies.  Returns {M: record}."""
    t = si.linear_inputs(cfg, max(Ms), N, K, r, with_dy=False, device=dev)
    Ws = []
    for i in range(copies):
        w = t["W"] if i == 0 else si.normal((N, K), 0.02, si.seed_of(cfg, 1, 1000 + i), device=dev)
        Ws.append(q.nf4_quantize(w, double_quant=True))
        del w
    del t["W"]
    packed_bytes = sum(q.nf4_sizes(N, K, True))
    out = {}
    for M in Ms:
        x = t["x"][:M].contiguous()
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        u = torch.empty((M, r), dtype=torch.float32, device=dev)
        ws = q.workspace(q.QL_OP_FWD, M, N, K, r, dev)
        state = {"i": 0}

        def call():
            W = Ws[state["i"] % copies]
            state["i"] += 1
            q.qlora_linear_fwd(x, W, t["A"], t["B"], alpha, y=y, u_save=u, ws=ws)

        ms_eager = timed(call, max(copies, 200), 20)
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
        each = [v / copies for v in timed_each(g.replay, replays, 3)]
        del g
        med = pct(each, 50)
        gbs = packed_bytes / (med * 1e-3) / 1e9
        out[f"M{M}"] = {"us_per_call": round(med * 1e3, 3),
                        "us_per_call_p10": round(pct(each, 10) * 1e3, 3),
                        "us_per_call_p90": round(pct(each, 90) * 1e3, 3),
                        "packed_GBps": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                        "launch": f"graph replay of {copies} calls, median over {replays} replays",
                        "us_per_call_eager": round(ms_eager * 1e3, 3)}
        log(f"decode {tag} M={M}: {med * 1e3:.2f} us/call in a graph ({gbs:.0f} GB/s packed; "
            f"p10 {pct(each, 10) * 1e3:.2f} p90 {pct(each, 90) * 1e3:.2f}), "
            f"{ms_eager * 1e3:.2f} us/call eager")
    del Ws
    torch.cuda.empty_cache()
    return out, packed_bytes


def bench_decode(q, si, dev, with_cpu=True):
    c = si.DECODE
    N, K, r, alpha = c["N"], c["K"], c["r"], c["alpha"]
    res, packed_bytes = _decode_rate(q, si, dev, N, K, r, alpha, c["Ms"], 64, 40, c["config"],
                                     "4096x4096")
    out = {"workload": "Llama-3-8B attention projection 4096x4096 NF4 + double quant, r=16, "
                       "alpha=32, bf16, forward only (u, y); 64 rotating weight copies",
           "unit": "GB/s", "packed_weight_bytes": packed_bytes}
    out.update(res)
    # decode-sized forwards on the MLP weights of the 8B and 70B shapes
    large = {}
    for (N2, K2, r2, cp) in ((14336, 4096, 16, 17), (8192, 28672, 64, 3)):
        res2, pb2 = _decode_rate(q, si, dev, N2, K2, r2, 16.0 if r2 == 64 else 32.0, (1,), cp, 20,
                                 c["config"], f"{N2}x{K2}")
        large[f"{N2}x{K2}_r{r2}"] = dict(res2["M1"], packed_weight_bytes=pb2, copies=cp)
    out["large_weights"] = large
    if with_cpu:
        out["cpu_oracle"] = cpu_decode(si, c)
    return out


def cpu_decode(si, c):
    """The oracle's GEMV (dequantise + fp64 forward, all host threads) at the
    decode config, per call."""
    from oracle import oracle as orc
    N, K, r, alpha = c["N"], c["K"], c["r"], c["alpha"]
    t = si.linear_inputs(c["config"], max(c["Ms"]), N, K, r, with_dy=False)
    bits = lambda v: v.contiguous().view(torch.int16).numpy().view("uint16")
    st = orc.quantize_nf4(bits(t["W"]), double_quant=True)
    out = {"threads": orc.num_threads(), "kind": "oracle"}
    for M in c["Ms"]:
        xh = bits(t["x"][:M])
        reps, t0 = 0, time.perf_counter()
        while True:
            w_hat = orc.dequantize(st).reshape(N, K)
            orc.linear_fwd(xh, w_hat, bits(t["A"]), bits(t["B"]), alpha, r)
            reps += 1
            if time.perf_counter() - t0 > 1.0:
                break
        dt = (time.perf_counter() - t0) / reps
        out[f"M{M}"] = {"ms_per_call": round(dt * 1e3, 2),
                        "packed_GBps": round(sum((st["packed"].nbytes, st["absmax_q"].nbytes,
                                                  st["absmax_scale"].nbytes, 4)) / dt / 1e9, 3)}
        log(f"cpu oracle decode M={M}: {dt * 1e3:.1f} ms/call")
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


def bench_quantize(q, si, dev, with_cpu=True):
    """8B-shaped weight set (32 layers x q,k,v,o,gate,up,down), bf16 N(0,0.02)
    with 0.1% outliers at 20 sigma: quantise (+ double quant) and dequantise
    every tensor once per pass."""
    cfg = si.WEIGHTSET_8B
    ws_list, q_list = [], []
    n_total = 0
    for layer in range(cfg["layers"]):
        for name in cfg["shapes"]:
            w = si.weightset_tensor(layer, name, device=dev)
            ws_list.append(w)
            q_list.append(q.NF4Weight.empty(w.shape[0], w.shape[1], True, dev))
            n_total += w.numel()
    maxn = max(w.numel() for w in ws_list)
    wsq = q.workspace(q.QL_OP_QUANTIZE, 0, 1, maxn, 0, dev)
    per_layer = len(cfg["shapes"])
    wsm = torch.empty(q.quantize_many_workspace_bytes([w.shape for w in ws_list[:per_layer]]),
                      dtype=torch.uint8, device=dev)
    deq = torch.empty(maxn, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"weight set ready: {n_total} params")

    def quant_all():  # one nf4_quantize_many call per layer (its 7 weights)
        for i in range(0, len(ws_list), per_layer):
            q.nf4_quantize_many(ws_list[i:i + per_layer], double_quant=True,
                                out=q_list[i:i + per_layer], ws=wsm)

    def quant_each():  # one nf4_quantize call per weight
        for w, qq in zip(ws_list, q_list):
            q.nf4_quantize(w, double_quant=True, out=qq, ws=wsq)

    def dequant_all():
        for qq in q_list:
            q.nf4_dequantize(qq, out=deq[:qq.rows * qq.cols].view(qq.rows, qq.cols))

    qms_eager = timed(quant_all, 3, 1)
    q1ms_eager = timed(quant_each, 3, 1)
    dms_eager = timed(dequant_all, 3, 1)
    # the same passes replayed from HIP graphs (no per-call host work: 224
    # launches of a few microseconds each would otherwise be host-bound)
    graphs = []
    for fn in (quant_all, dequant_all, quant_each):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs.append(g)
    qms = timed(graphs[0].replay, 5, 1)
    dms = timed(graphs[1].replay, 5, 1)
    q1ms = timed(graphs[2].replay, 5, 1)
    del graphs
    stored = sum(qq.storage_bytes() for qq in q_list)
    q_bytes = 2 * n_total + stored
    d_bytes = stored + 2 * n_total
    out = {"workload": "8B-shaped weight set, 32 layers x {q,k,v,o,gate,up,down}, bf16 "
                       "N(0,0.02) + 0.1% outliers at 20 sigma, NF4 + double quant",
           "params": n_total, "bits_per_param": round(8 * stored / n_total, 5),
           "quantize_ms": round(qms, 3), "quantize_GBps": round(q_bytes / (qms * 1e-3) / 1e9, 1),
           "dequantize_ms": round(dms, 3),
           "dequantize_GBps": round(d_bytes / (dms * 1e-3) / 1e9, 1), "unit": "GB/s",
           "launch": "HIP graph replay of each pass: quantise as 32 nf4_quantize_many calls "
                     "(one per layer, 64 launches), dequantise as 224 calls",
           "quantize_per_tensor_ms": round(q1ms, 3),
           "quantize_per_tensor_GBps": round(q_bytes / (q1ms * 1e-3) / 1e9, 1),
           "quantize_ms_eager": round(qms_eager, 3),
           "quantize_per_tensor_ms_eager": round(q1ms_eager, 3),
           "dequantize_ms_eager": round(dms_eager, 3)}
    out["quantize_hbm_frac"] = round(out["quantize_GBps"] / PEAK_HBM_GBS, 4)
    out["dequantize_hbm_frac"] = round(out["dequantize_GBps"] / PEAK_HBM_GBS, 4)
    log(f"quantize {qms:.2f} ms ({out['quantize_GBps']} GB/s; one call per weight {q1ms:.2f} ms, "
        f"{out['quantize_per_tensor_GBps']} GB/s), dequantize {dms:.2f} ms "
        f"({out['dequantize_GBps']} GB/s) in graphs; eager {qms_eager:.2f} / {dms_eager:.2f} ms; "
        f"{out['bits_per_param']} bits/param")
    del ws_list, q_list, deq
    torch.cuda.empty_cache()
    if with_cpu:
        out["cpu_oracle"] = cpu_quantize(si)
    return out


def cpu_quantize(si):
    """The oracle's quantise (+ double quant) and dequantise of the weight
    set's layers 0 and 31 (14 tensors), all host threads: GB/s of the same
    algorithmic bytes as the GPU figure."""
    from oracle import oracle as orc
    cfg = si.WEIGHTSET_8B
    bits = lambda v: v.contiguous().view(torch.int16).numpy().view("uint16")
    tq = td = 0.0
    n = stored = 0
    for layer in (0, cfg["layers"] - 1):
        for name in cfg["shapes"]:
            wh = bits(si.weightset_tensor(layer, name))
            t0 = time.perf_counter()
            st = orc.quantize_nf4(wh, double_quant=True)
            t1 = time.perf_counter()
            orc.dequantize(st)
            t2 = time.perf_counter()
            tq += t1 - t0
            td += t2 - t1
            n += wh.size
            stored += (st["packed"].nbytes + st["absmax_q"].nbytes + st["absmax_scale"].nbytes + 4)
    by = 2 * n + stored
    out = {"sample": "layers 0 and 31 (14 tensors)", "params": n, "threads": orc.num_threads(),
           "kind": "oracle", "quantize_s": round(tq, 3), "quantize_GBps": round(by / tq / 1e9, 3),
           "dequantize_s": round(td, 3), "dequantize_GBps": round(by / td / 1e9, 3)}
    log(f"cpu oracle quantize {tq:.2f} s, dequantize {td:.2f} s over {n} params")
    return out


def bench_small_fp32(q, si, dev, with_cpu=True, calls=1000):
    """The fp32 layer of the small configuration (W 256x256 NF4 block 64, fp32
    absmax; x 4x256; r=8, alpha=16): forward + backward, `calls` calls timed
    with HIP events (latency-bound), and the oracle on one host thread."""
    c = si.SMALL_FP32
    M, N, K, r, alpha = c["M"], c["N"], c["K"], c["r"], c["alpha"]
    t = si.linear_inputs(c["config"], M, N, K, r, act_dtype=torch.float32,
                         w_dtype=torch.float32, lora_dtype=torch.float32)
    d = {k: v.to(dev) for k, v in t.items()}
    W = q.nf4_quantize(d["W"], double_quant=False)
    y = torch.empty((M, N), dtype=torch.float32, device=dev)
    u = torch.empty((M, r), dtype=torch.float32, device=dev)
    dx = torch.empty((M, K), dtype=torch.float32, device=dev)
    dA = torch.empty((r, K), dtype=torch.float32, device=dev)
    dB = torch.empty((N, r), dtype=torch.float32, device=dev)
    wsf = q.workspace(q.QL_OP_FWD, M, N, K, r, dev)
    wsb = q.workspace(q.QL_OP_BWD, M, N, K, r, dev)

    def call():
        q.qlora_linear_fwd(d["x"], W, d["A"], d["B"], alpha, y=y, u_save=u, ws=wsf)
        q.qlora_linear_bwd(d["dy"], d["x"], W, d["A"], d["B"], alpha, u_saved=u, dx=dx, dA=dA,
                           dB=dB, ws=wsb)

    ms = timed(call, calls, 50)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    ms_graph = timed(g.replay, calls, 50)
    del g
    fl = layer_flops(M, N, K, r)
    out = {"workload": "fp32 QLoRA linear W 256x256 NF4 block 64 fp32 absmax, x 4x256, r=8 "
                       "alpha=16, forward + backward (dx, dA, dB)",
           "flop": fl, "us_per_call_eager": round(ms * 1e3, 2),
           "us_per_call_graph": round(ms_graph * 1e3, 2), "calls": calls}
    log(f"small fp32: {ms * 1e3:.1f} us/call eager, {ms_graph * 1e3:.1f} us/call graph")
    if with_cpu:
        from oracle import oracle as orc
        nt = orc.num_threads()
        orc.set_num_threads(1)
        try:
            Wh, xh, Ah, Bh, dyh = (t[k].numpy() for k in ("W", "x", "A", "B", "dy"))
            st = orc.quantize_nf4(Wh, double_quant=False)
            reps, t0 = 0, time.perf_counter()
            while reps < 20 or time.perf_counter() - t0 < 1.0:
                w_hat = orc.dequantize(st).reshape(N, K)
                orc.linear_fwd(xh, w_hat, Ah, Bh, alpha, r)
                orc.linear_bwd(xh, w_hat, Ah, Bh, dyh, alpha, r)
                reps += 1
            dt = (time.perf_counter() - t0) / reps
        finally:
            orc.set_num_threads(nt)
        out["cpu_oracle"] = {"us_per_call": round(dt * 1e6, 1), "threads": 1, "kind": "oracle",
                             "sample": "dequantise + fp64 forward + backward, whole call"}
        log(f"small fp32 oracle: {dt * 1e6:.0f} us/call on one thread")
    return out


def _cpu_sample(si, c, rows, M_grad, bits, orc):
    """The oracle on the gate projection of config c: dequantise the weight,
    then y and dx for `rows` sampled token rows and dA / dB over the first
    M_grad tokens.  Returns (seconds, flop counted)."""
    N, K = c["projs"]["gate"]
    r, alpha = c["r"], c["alpha"]
    t = si.linear_inputs(c["config"], M_grad, N, K, r, sub=0)
    Wh, xh, Ah, Bh, dyh = (bits(t[k]) for k in ("W", "x", "A", "B", "dy"))
    st = orc.quantize_nf4(Wh, double_quant=True)
    sel = sorted({int(round(i * (M_grad - 1) / max(1, rows - 1))) for i in range(rows)})
    t0 = time.perf_counter()
    w_hat = orc.dequantize(st).reshape(N, K)
    orc.linear_fwd(xh[sel], w_hat, Ah, Bh, alpha, r)
    orc.linear_bwd(xh, w_hat, Ah, Bh, dyh, alpha, r, rows=sel)
    dt = time.perf_counter() - t0
    R = len(sel)
    flop = (2 * R * N * K + 2 * R * r * (K + N)            # y rows (+ their u)
            + 2 * M_grad * r * (K + N)                      # u, g for every token
            + 2 * N * r * M_grad + 2 * r * K * M_grad       # dB, dA
            + 2 * R * N * K + 2 * R * r * K)                # dx rows
    return dt, flop


def cpu_baseline(si, c):
    """The CPU oracle on a bounded sample of the step: the gate projection's
    dequantisation, y and dx on 32 sampled token rows and dA / dB over all
    tokens, fp64 accumulation, all host threads (TFLOP/s of the flop it
    performs); beside it the same on one thread over a smaller sample."""
    from oracle import oracle as orc
    bits = lambda v: v.contiguous().view(torch.int16).numpy().view("uint16")
    M = c["M"]
    N, K = c["projs"]["gate"]
    # the sample is run several times so that the timed CPU work is ~10 s
    reps, reps1 = 6, 4
    dt = fl = 0.0
    for _ in range(reps):
        d_, f_ = _cpu_sample(si, c, 32, M, bits, orc)
        dt, fl = dt + d_, fl + f_
    log(f"cpu oracle: {dt:.2f} s for {fl / 1e9:.1f} GFLOP ({reps} x (32 rows, {M} tokens for dA/dB))")
    nt = orc.num_threads()
    orc.set_num_threads(1)
    dt1 = fl1 = 0.0
    try:
        for _ in range(reps1):
            d_, f_ = _cpu_sample(si, c, 2, 128, bits, orc)
            dt1, fl1 = dt1 + d_, fl1 + f_
    finally:
        orc.set_num_threads(nt)
    log(f"cpu oracle 1 thread: {dt1:.2f} s for {fl1 / 1e9:.1f} GFLOP")
    out = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": nt, "kind": "oracle",
           "sample": f"gate projection {N}x{K} r={c['r']}: dequantise, y and dx on 32 sampled "
                     f"token rows, dA and dB over all {M} tokens, fp64 accumulation; run "
                     f"{reps} times, {dt:.1f} s in all",
           "one_thread": {"value": round(fl1 / dt1 / 1e12, 6), "unit": "TFLOP/s",
                          "sample": "same projection, y and dx on 2 rows, dA and dB over 128 "
                                    f"tokens; run {reps1} times, {dt1:.1f} s in all"}}
    out.update(host_info())
    return out


if __name__ == "__main__":
    main()

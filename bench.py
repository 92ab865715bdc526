"""Benchmark of the MoE block forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one moe_layer_forward (router, dispatch, gate/up GEMM, down GEMM,
combine, load-balance statistics) over one batch of seeded synthetic input that
is already resident in HBM. Prints ONE JSON line with throughput (tokens/s), the
roofline of the dominant kernel (the gate/up grouped GEMM, timed on its own with
HIP events on the stream it runs on) and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec on 1 MI355X + % of bf16 MFMA peak / % HBM BW"
# MI355X published peaks: dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk), HBM3E.
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gate_up_algorithmic(cfg, counts: np.ndarray):
    """Algorithmic FLOPs and bytes of one gate/up launch: 2 GEMMs of
    2*H*I FLOP per routed pair; bytes = gate+up weights of the touched experts
    + the x rows read + h written."""
    eb = 2 if cfg.dtype == "bf16" else 4
    touched = int((counts > 0).sum())
    flops = 4.0 * cfg.H * cfg.I * cfg.P
    bytes_ = touched * 2.0 * cfg.I * cfg.H * eb + cfg.T * cfg.H * eb + cfg.P * cfg.I * eb
    return flops, bytes_, touched


def layer_algorithmic(cfg, counts: np.ndarray):
    eb = 2 if cfg.dtype == "bf16" else 4
    touched = int((counts > 0).sum())
    flops = cfg.T * (2.0 * cfg.H * cfg.E + 6.0 * cfg.H * cfg.I * cfg.k)
    bytes_ = touched * 3.0 * cfg.H * cfg.I * eb + cfg.E * cfg.H * eb + 2.0 * cfg.T * cfg.H * eb
    return flops, bytes_


def cpu_baseline(cfg, inp, budget_s: float):
    """The oracle as it stands on a bounded sample of tokens of the same
    workload; returns tokens/s, cores used and the sample description."""
    from oracle import oracle
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    cores = int(os.environ["OMP_NUM_THREADS"])
    n = 8
    t0 = time.perf_counter()
    oracle.forward_tokens(inp, cfg, tokens=np.arange(n, dtype=np.int32))
    dt = time.perf_counter() - t0
    # scale the sample to about `budget_s` seconds
    n2 = int(max(n, min(cfg.T, n * budget_s / max(dt, 1e-3))))
    n2 = min(n2, cfg.T)
    if n2 > n:
        tok = np.linspace(0, cfg.T - 1, n2).astype(np.int32)
        t0 = time.perf_counter()
        oracle.forward_tokens(inp, cfg, tokens=tok)
        dt = time.perf_counter() - t0
        n = n2
    return {"value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {cfg.T} tokens of {cfg.name} (full block forward per token, "
                      f"fp64 scalar loops), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill128_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(no sharding, no collectives); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_mixture_experts_40_amd import binding
    from sparse_mixture_experts_40_amd.configs import WORKLOADS
    from sparse_mixture_experts_40_amd.inputs import make_inputs

    cfg = WORKLOADS[args.workload]
    if args.seed != cfg.seed:
        cfg = type(cfg)(**{**cfg.__dict__, "seed": args.seed})
    binding.load()
    torch.cuda.init()
    log(f"workload {cfg}")
    t0 = time.perf_counter()
    inp = make_inputs(cfg)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    blk = binding.MoEBlock(cfg, inp)
    x = binding.to_device(inp["x"])
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        blk.forward(x)
    torch.cuda.synchronize()

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        blk.forward(x)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    log(f"layer: {ms_step:.4f} ms/step (events), wall {wall * 1e3 / args.steps:.4f} ms/step")

    # dominant kernel: gate/up grouped GEMM on its own, same inputs, same stream
    c = blk.c
    T, E, k = cfg.T, cfg.E, cfg.k
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    wts = torch.empty(T, k, dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    h = torch.empty(T * k, cfg.I, dtype=binding.TORCH_DTYPE[cfg.dtype], device="cuda")
    binding.router_topk(c, x, blk.w_router, blk.logit_bias, None, idx, wts)
    binding.dispatch(c, idx, counts, offsets, sp, pp, blk.ws)
    for _ in range(2):
        binding.expert_gate_up(c, x, sp, offsets, blk.w_gate, blk.w_up, h)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        binding.expert_gate_up(c, x, sp, offsets, blk.w_gate, blk.w_up, h)
    ev1.record(stream)
    torch.cuda.synchronize()
    gu_ms = ev0.elapsed_time(ev1) / args.steps
    cnt = counts.cpu().numpy()
    gflops, gbytes, touched = gate_up_algorithmic(cfg, cnt)
    lflops, lbytes = layer_algorithmic(cfg, cnt)
    log(f"gate/up kernel: {gu_ms:.4f} ms/launch, touched experts {touched}/{E}")

    decode = cfg.P <= 4 * cfg.E  # weight-streaming regime: bound by HBM
    if decode:
        achieved = gbytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": None}
    else:
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
        achieved = gflops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": None}
    roof["kernel"] = "grouped_gemm_bf16 gate/up (SiLU*mul epilogue)" if cfg.dtype == "bf16" \
        else "gate_up_f32"
    roof["kernel_ms"] = gu_ms

    value = T / (ms_step * 1e-3)
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": cfg.H, "E": E, "k": k, "I": cfg.I,
                   "norm_topk_prob": cfg.norm, "zipf_s": cfg.zipf_s, "seed": cfg.seed},
        "roofline": roof,
        "layer": {"tflops": lflops / (ms_step * 1e-3) / 1e12,
                  "mfma_frac": lflops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                  "hbm_gbs_min_bytes": lbytes / (ms_step * 1e-3) / 1e9,
                  "touched_experts": touched, "wall_ms_per_step": wall * 1e3 / args.steps},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

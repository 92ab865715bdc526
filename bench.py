"""Benchmark of the MoE block forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--capacity-factor CF]   # capacity-limited dispatch, C = ceil(T*k*CF/E)
                    [--router noise|bias|noise+bias]   # router variants (seeded inputs)
                    [--dynamic-k-min KMIN]   # entropy-driven k in [KMIN, k]
                    [--w4]                   # 4-bit group-quantised expert weights
    python bench.py --copy-calibration     # plain 1 GiB device copy, for counter scaling

A step is one moe_layer_forward (router, dispatch, gate/up GEMM, down GEMM,
combine, load-balance statistics) over one batch of seeded synthetic input that
is already resident in HBM. Prints ONE JSON line with throughput (tokens/s), the
roofline of the dominant kernel (the gate/up grouped GEMM, timed on its own with
HIP events on the stream it runs on) and the CPU oracle timed on a bounded
sample of the same workload. Also in the line: the per-step distribution
(median, p10, p90 from one event per step), each stage timed on its own, the
shader clock sampled from sysfs during the timed steps, and for weight-streaming
workloads the same steps (and the gate/up launch) with 512 MB of other data
touched between them, outside the timed events: read (no weight byte can then
come from the 256 MB MALL) and, separately, written (the MALL is then full of
dirty lines that the next kernel's reads evict with write-backs).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec on 1 MI355X + % of bf16 MFMA peak / % HBM BW"
# MI355X published peaks: dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk), HBM3E.
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0

# HBM traffic of the gate/up kernel per launch, from rocprofv3 --pmc FETCH_SIZE
# and WRITE_SIZE passes over this script (KiB per dispatch, averaged), scaled by
# what the same counters read for a plain 1 GiB device copy (bench.py
# --copy-calibration): FETCH_SIZE reported 524303 KiB for 1 GiB read (x2.0),
# WRITE_SIZE 1048576 KiB for 1 GiB written (x1.0). Valid only for the kernel
# sources they were taken on (sha256 below); otherwise traffic is null.
TRAFFIC_SOURCES = ("sparse_mixture_experts_40_amd/csrc/expert_gemm.hip",
                   "sparse_mixture_experts_40_amd/csrc/moe_internal.h")
FETCH_SCALE = 1048576.0 / 524302.4
WRITE_SCALE = 1048576.0 / 1048576.0
MEASURED_TRAFFIC = {
    # workload: (sources sha256, FETCH_SIZE KiB, WRITE_SIZE KiB) per gate/up launch
    "prefill128_bf16": ("f569da93d9a4ba92e69975a45e9acfe54e18d7da914d8fe90a12ae8c27feacb0",
                        3798049.5, 394143.9),
    "decode128_bf16": ("f569da93d9a4ba92e69975a45e9acfe54e18d7da914d8fe90a12ae8c27feacb0",
                       542903.0, 1561.8),
}


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per gate/up launch, or None if not measured on these sources."""
    m = MEASURED_TRAFFIC.get(workload)
    if m is None or m[0] != kernel_sources_sha256():
        return None
    return m[1] * 1024.0 * FETCH_SCALE + m[2] * 1024.0 * WRITE_SCALE


def uses_decode_kernel(cfg) -> bool:
    """The library's choice between the weight-streaming (decode) and the tiled
    grouped GEMM for bf16: few pairs per expert and H, I multiples of 256."""
    return cfg.dtype == "bf16" and cfg.P <= 16 * cfg.E and cfg.H % 256 == 0 and cfg.I % 256 == 0


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def weight_bytes_per_element(cfg, w4: bool) -> float:
    """Bytes one weight element costs in HBM: 2 / 4 for bf16 / fp32; 4-bit codes
    are 0.5 byte plus a 4-byte (scale, bias) pair per group of 128."""
    if w4:
        return 0.5 + 4.0 / 128.0
    return 2.0 if cfg.dtype == "bf16" else 4.0


def gate_up_algorithmic(cfg, counts: np.ndarray, rows: int, w4: bool = False):
    """Algorithmic FLOPs and bytes of one gate/up launch over `rows` routed
    (kept) pairs: 2 GEMMs of 2*H*I FLOP per pair; bytes = gate+up weights of
    the touched experts + the x rows read + h written."""
    eb = 2 if cfg.dtype == "bf16" else 4
    wb = weight_bytes_per_element(cfg, w4)
    touched = int((counts > 0).sum())
    flops = 4.0 * cfg.H * cfg.I * rows
    bytes_ = touched * 2.0 * cfg.I * cfg.H * wb + cfg.T * cfg.H * eb + rows * cfg.I * eb
    return flops, bytes_, touched


def layer_algorithmic(cfg, counts: np.ndarray, rows: int, w4: bool = False):
    eb = 2 if cfg.dtype == "bf16" else 4
    wb = weight_bytes_per_element(cfg, w4)
    touched = int((counts > 0).sum())
    flops = cfg.T * 2.0 * cfg.H * cfg.E + 6.0 * cfg.H * cfg.I * rows
    bytes_ = touched * 3.0 * cfg.H * cfg.I * wb + cfg.E * cfg.H * eb + 2.0 * cfg.T * cfg.H * eb
    return flops, bytes_


def cpu_baseline(cfg, inp, budget_s: float, w4=None):
    """The oracle as it stands on a bounded sample of tokens of the same
    workload (4-bit weights: its 4-bit forward); returns tokens/s, cores used
    and the sample description."""
    from oracle import oracle
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    cores = int(os.environ["OMP_NUM_THREADS"])

    def forward(tokens):
        if w4 is None:
            oracle.forward_tokens(inp, cfg, tokens=tokens)
        else:
            oracle.forward_w4(inp, w4, cfg, tokens=tokens)

    n = 8
    t0 = time.perf_counter()
    forward(np.arange(n, dtype=np.int32))
    dt = time.perf_counter() - t0
    # scale the sample to about `budget_s` seconds
    want = int(max(n, n * budget_s / max(dt, 1e-3)))
    n2, passes = min(want, cfg.T), 1
    if want > cfg.T:  # the whole workload is cheaper than the budget: repeat it
        passes = max(1, min(50, want // cfg.T))
    if n2 > n or passes > 1:
        tok = np.linspace(0, cfg.T - 1, n2).astype(np.int32)
        t0 = time.perf_counter()
        for _ in range(passes):
            forward(tok)
        dt = time.perf_counter() - t0
        n = n2 * passes
    what = (f"{n2} of {cfg.T} tokens" if passes == 1 else
            f"all {cfg.T} tokens x {passes} passes")
    return {"value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} of {cfg.name} (full block forward per token, "
                      f"fp64 scalar loops), {dt:.1f} s"}


def pct(v, q):
    return float(np.percentile(np.asarray(v, dtype=np.float64), q))


def dist(v):
    return {"median_ms": pct(v, 50), "p10_ms": pct(v, 10), "p90_ms": pct(v, 90)}


def clock_files(torch):
    """sysfs file with the shader clock levels of device 0 (amdgpu pp_dpm_sclk,
    the current level marked with '*'), found through its PCI address."""
    try:
        pr = torch.cuda.get_device_properties(0)
        bdf = "%04x:%02x:%02x.0" % (getattr(pr, "pci_domain_id", 0), pr.pci_bus_id,
                                    pr.pci_device_id)
    except Exception:
        return []
    return glob.glob(f"/sys/bus/pci/devices/{bdf}/pp_dpm_sclk")


def read_sclk_mhz(fn):
    with open(fn) as f:
        for ln in f:
            if ln.rstrip().endswith("*"):
                return float(ln.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
    return None


class ClockSampler:
    """Reads the current shader clock from sysfs every 20 ms on a host thread."""

    def __init__(self, files):
        self.files, self.samples, self._stop = files, [], threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            for fn in self.files:
                try:
                    v = read_sclk_mhz(fn)
                    if v is not None:
                        self.samples.append(v)
                except (OSError, ValueError, IndexError):
                    pass
            self._stop.wait(0.02)

    def __enter__(self):
        if self.files:
            self._t.start()
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self.files:
            self._t.join()

    def summary(self):
        if not self.samples:
            return None
        return {"source": "sysfs pp_dpm_sclk (current level)", "samples": len(self.samples),
                "median_mhz": pct(self.samples, 50), "min_mhz": min(self.samples),
                "max_mhz": max(self.samples)}


def time_per_call(torch, stream, fn, reps):
    """Per-call times (ms) of fn from one HIP event before each call."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        ev[i].record(stream)
        fn()
    ev[reps].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill128_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--capacity-factor", type=float, default=0.0,
                    help="> 0: capacity-limited dispatch with C = ceil(T*k*CF/E)")
    ap.add_argument("--router", default="plain", choices=["plain", "noise", "bias", "noise+bias"],
                    help="router variant: noisy top-k and/or selection-only bias")
    ap.add_argument("--dynamic-k-min", type=int, default=0,
                    help="> 0: entropy-driven number of experts per token in [KMIN, k]")
    ap.add_argument("--w4", action="store_true",
                    help="4-bit group-quantised expert weights (codes + per-128 scale/bias)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 1 GiB, 3 times: the "
                         "reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(no sharding, no collectives); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 1 << 28  # float32 elements: 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 4 * n, "copies": 3}), flush=True)
        return

    from sparse_mixture_experts_40_amd import binding
    from sparse_mixture_experts_40_amd.configs import WORKLOADS
    from sparse_mixture_experts_40_amd.inputs import (make_inputs, make_router_variant_inputs,
                                                      make_w4_inputs)

    cfg = WORKLOADS[args.workload]
    if args.seed != cfg.seed:
        cfg = type(cfg)(**{**cfg.__dict__, "seed": args.seed})
    binding.load()
    torch.cuda.init()
    log(f"workload {cfg}")
    t0 = time.perf_counter()
    inp = make_inputs(cfg, weights=not args.w4)
    w4 = make_w4_inputs(cfg) if args.w4 else None
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    cap = binding.capacity(binding.make_config(cfg), args.capacity_factor) \
        if args.capacity_factor > 0 else 0
    var = make_router_variant_inputs(cfg) if args.router != "plain" else {}
    blk = binding.MoEBlock(cfg, inp, capacity=cap,
                           noise=var.get("noise") if "noise" in args.router else None,
                           w_noise=var.get("w_noise") if "noise" in args.router else None,
                           select_bias=var.get("select_bias") if "bias" in args.router else None,
                           dynamic_k_min=args.dynamic_k_min, w4=w4)
    x = binding.to_device(inp["x"])
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        blk.forward(x)
    torch.cuda.synchronize()

    # the K timed steps, one event before each (and one after the last)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    with ClockSampler(clock_files(torch)) as clk:
        w0 = time.perf_counter()
        for i in range(args.steps):
            evs[i].record(stream)
            blk.forward(x)
        evs[args.steps].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
    ms_step = evs[0].elapsed_time(evs[args.steps]) / args.steps
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    log(f"layer: {ms_step:.4f} ms/step (events), wall {wall * 1e3 / args.steps:.4f} ms/step")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    streaming = uses_decode_kernel(cfg) or args.w4
    scrub = torch.ones(1 << 27, dtype=torch.float32, device="cuda") if streaming else None
    scrubs = {"read": lambda i: scrub.sum(), "write": lambda i: scrub.fill_(float(i))}

    def scrubbed_times(fn, how):
        """Per-call times of fn with 512 MB of other data read or written before
        each call (outside the events)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            scrubs[how](i)
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    scrubbed = None
    if streaming:
        scrubbed = {"scrub_bytes": 4 << 27}
        for how in ("read", "write"):
            sm = scrubbed_times(lambda: blk.forward(x), how)
            scrubbed[f"after_{how}"] = {**dist(sm), "tokens_per_s": cfg.T / (pct(sm, 50) * 1e-3)}

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
    # the same router (variants included) as the timed block
    binding.router_topk_ex(c, blk.opts, x, blk.w_router, blk.logit_bias, None, idx, wts, blk.ws)
    if cap:
        binding.dispatch_capacity(c, idx, cap, counts, offsets, sp, pp, blk.ws)
    else:
        binding.dispatch(c, idx, counts, offsets, sp, pp, blk.ws)
    def gate_up():
        if args.w4:
            binding.expert_gate_up_w4(c, x, sp, offsets, blk.w4_struct, h)
        else:
            binding.expert_gate_up(c, x, sp, offsets, blk.w_gate, blk.w_up, h)

    for _ in range(2):
        gate_up()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        gate_up()
    ev1.record(stream)
    torch.cuda.synchronize()
    gu_ms = ev0.elapsed_time(ev1) / args.steps
    gu_scrubbed = {}
    if streaming:
        for how in ("read", "write"):
            gu_scrubbed[how] = pct(scrubbed_times(gate_up, how), 50)
    # every stage on its own, same inputs and stream (median of per-call times)
    y = torch.empty(T * k, cfg.H, dtype=torch.float32, device="cuda")
    out = torch.empty(T, cfg.H, dtype=binding.TORCH_DTYPE[cfg.dtype], device="cuda")
    lg = torch.empty(T, E, dtype=torch.float32, device="cuda")
    binding.router_topk_ex(c, blk.opts, x, blk.w_router, blk.logit_bias, lg, idx, wts, blk.ws)
    def down():
        if args.w4:
            binding.expert_down_w4(c, h, offsets, blk.w4_struct, y)
        else:
            binding.expert_down(c, h, offsets, blk.w_down, y)
    def disp():
        if cap:
            binding.dispatch_capacity(c, idx, cap, counts, offsets, sp, pp, blk.ws)
        else:
            binding.dispatch(c, idx, counts, offsets, sp, pp, blk.ws)
    stage_fns = [
        ("router", lambda: binding.router_topk_ex(c, blk.opts, x, blk.w_router, blk.logit_bias,
                                                  None, idx, wts, blk.ws)),
        ("dispatch", disp),
        ("gate_up", gate_up),
        ("down", down),
        ("combine", lambda: binding.combine(c, y, pp, wts, out)),
        ("aux_stats_from_logits", lambda: binding.aux_stats(c, lg, idx, blk.ws, counts=counts,
                                                            f=blk.f, P=blk.P, aux=blk.aux)),
    ]
    stages = {n: pct(time_per_call(torch, stream, fn, max(10, args.steps)), 50)
              for n, fn in stage_fns}
    disp()  # counts / offsets of the router's selection again
    torch.cuda.synchronize()
    cnt = counts.cpu().numpy()
    rows = int(offsets[E].item())  # kept pairs (all of them without a capacity)
    gflops, gbytes, touched = gate_up_algorithmic(cfg, cnt, rows, args.w4)
    lflops, lbytes = layer_algorithmic(cfg, cnt, rows, args.w4)
    log(f"gate/up kernel: {gu_ms:.4f} ms/launch, touched experts {touched}/{E}")

    decode = cfg.P <= 4 * cfg.E  # weight-streaming regime: bound by HBM
    traffic = measured_traffic(cfg.name) if not (cap or args.w4) else None
    if decode:
        achieved = gbytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}
    else:
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
        achieved = gflops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": traffic}
    if args.w4:
        roof["kernel"] = "decode_w4_kernel<true> (gate/up, 4-bit weights, SiLU*mul epilogue)"
    elif cfg.dtype != "bf16":
        roof["kernel"] = "gate_up_f32_kernel"
    elif uses_decode_kernel(cfg):
        roof["kernel"] = "decode_gemm_bf16_kernel<true> (gate/up, SiLU*mul epilogue)"
    else:
        roof["kernel"] = "grouped_gemm_bf16_kernel<true,...> (gate/up, SiLU*mul epilogue)"
    roof["kernel_ms"] = gu_ms
    for how, ms in gu_scrubbed.items():  # same algorithmic bytes, 512 MB touched before
        ach = gbytes / (ms * 1e-3) / 1e9
        roof[f"after_{how}_512mb"] = {"kernel_ms": ms, "achieved": ach,
                                      "frac": ach / PEAK_HBM_GBS}
    roof["algorithmic"] = {"flops": gflops, "bytes": gbytes}
    roof["traffic_unit"] = "HBM bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)"

    value = T / (ms_step * 1e-3)
    if cap:
        line_cap = {"capacity_factor": args.capacity_factor, "capacity": cap,
                    "dropped_pairs": int(blk.dropped.item()), "kept_pairs": rows}
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "T": T, "H": cfg.H, "E": E, "k": k, "I": cfg.I,
                   "norm_topk_prob": cfg.norm, "zipf_s": cfg.zipf_s, "seed": cfg.seed},
        "roofline": roof,
        "step_ms": dist(step_ms),
        "stages_ms": stages,
        "gpu_clock": clk.summary(),
        "layer": {"tflops": lflops / (ms_step * 1e-3) / 1e12,
                  "mfma_frac": lflops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                  "hbm_gbs_min_bytes": lbytes / (ms_step * 1e-3) / 1e9,
                  "touched_experts": touched, "wall_ms_per_step": wall * 1e3 / args.steps},
    }
    if scrubbed:
        line["mall_scrubbed"] = scrubbed
    if cap:
        line["config"].update(line_cap)
    if args.router != "plain":
        line["config"]["router"] = args.router
    if args.w4:
        line["config"]["weights"] = "w4 (group 128, bf16 scale/bias)"
    if args.dynamic_k_min:
        kt = blk.k_per_token.cpu().numpy()
        line["config"].update({"dynamic_k_min": args.dynamic_k_min,
                               "mean_k": float(kt.mean()), "routed_pairs": int(kt.sum())})
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget, w4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

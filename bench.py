"""Benchmark of the MoE block forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--decode-workload NAME|none] [--decode-steps N]
                    [--capacity-factor CF]   # capacity-limited dispatch, C = ceil(T*k*CF/E)
                    [--capacity-fallback-min M]  # with CF: least-loaded fallback to M slots
                    [--router noise|bias|noise+bias]   # router variants (seeded inputs)
                    [--dynamic-k-min KMIN]   # entropy-driven k in [KMIN, k]
                    [--w4]                   # 4-bit group-quantised expert weights
    python bench.py --copy-calibration     # plain 1 GiB device copy, for counter scaling
    python bench.py ... --rocprof stats|traffic|mops [--rocprof-dir D]
                                           # the same command under rocprofv3, + summary.md

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

Each workload is also timed as one step captured in a HIP graph and replayed
(`graph_replay`, launch overhead removed; `value` stays the eager step's).
The default run also times the 64-token, 128-expert decode workload after the
main one, and reports it as the line's "decode" object (ms/step, tokens/s, the
layer's fraction of HBM bandwidth, the gate/up roofline, stages, and the
MALL-scrubbed variants); `value` and the rest of the line stay the main
workload's.

The CPU-oracle leg also compares, outside its timed calls, the oracle's
outputs on its sample tokens with the timed block's output and selection
(plain routing, bf16 or 4-bit weights): the line's "parity" object holds the
number of tokens whose selection differs (recomputed by the oracle with the
GPU's selection), the largest |d| over RMS(ref), and the largest share of the
element tolerance used.
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
# and WRITE_SIZE passes over the layer's own steps (bench.py --workload W
# --steps 3 --warmup 1 --rocprof traffic; KiB per dispatch, averaged over the
# timed steps), scaled by what the same counters read for a plain 1 GiB device
# copy (bench.py --copy-calibration): FETCH_SIZE reported 524304.8 KiB for
# 1 GiB read (x2.0), WRITE_SIZE 1048576 KiB for 1 GiB written (x1.0). Valid only
# for the sources they were taken on (sha256 below: the kernel, its dispatch
# input order and the build flags); otherwise traffic is null.
TRAFFIC_SOURCES = ("sparse_mixture_experts_40_amd/csrc/expert_gemm.hip",
                   "sparse_mixture_experts_40_amd/csrc/moe_internal.h",
                   "sparse_mixture_experts_40_amd/csrc/dispatch.hip",
                   "sparse_mixture_experts_40_amd/build.py")
FETCH_SCALE = 1048576.0 / 524304.8
WRITE_SCALE = 1048576.0 / 1048576.0
MEASURED_TRAFFIC = {
    # workload: (sources sha256, FETCH_SIZE KiB, WRITE_SIZE KiB) per gate/up launch
    "prefill128_bf16": ("b4d81da6824de0e0b6f68dc276a530695be055012a8f348e97d73be92cc231ee",
                        3856735.1, 393996.8),
    "decode128_bf16": ("b4d81da6824de0e0b6f68dc276a530695be055012a8f348e97d73be92cc231ee",
                       542915.6, 1564.6),
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


def cpu_baseline(cfg, inp, budget_s: float, w4=None, gpu=None):
    """The oracle as it stands on a bounded sample of tokens of the same
    workload (4-bit weights: its 4-bit forward); returns (tokens/s, cores used
    and the sample description; parity of the GPU's block output on the
    sample, or None). `gpu` holds the timed block's output [T,H] and
    selection [T,k] on the host (None: no parity figures). The comparison
    runs after the timed oracle calls, outside their time."""
    from oracle import oracle
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    cores = int(os.environ["OMP_NUM_THREADS"])

    def forward(tokens, forced_idx=None):
        if w4 is None:
            return oracle.forward_tokens(inp, cfg, tokens=tokens, forced_idx=forced_idx)
        return oracle.forward_w4(inp, w4, cfg, tokens=tokens, forced_idx=forced_idx)

    n = 8
    tok = np.arange(n, dtype=np.int32)
    t0 = time.perf_counter()
    ref = forward(tok)
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
            ref = forward(tok)
        dt = time.perf_counter() - t0
        n = n2 * passes
    else:
        n2 = n
    what = (f"{n2} of {cfg.T} tokens" if passes == 1 else
            f"all {cfg.T} tokens x {passes} passes")
    base = {"value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{what} of {cfg.name} (full block forward per token, "
                      f"fp64 scalar loops), {dt:.1f} s"}
    return base, (sample_parity(cfg, tok, ref, gpu, forward) if gpu is not None else None)


def sample_parity(cfg, tok, ref, gpu, forward):
    """The GPU block's output and selection on the oracle's sample tokens.

    A token whose selection (experts or their slot order) differs from the
    oracle's is counted, its k-th/(k+1)-th logit gap recorded, and its oracle
    output recomputed with the GPU's selection (forced routing) before the
    outputs are compared. Tolerance: bf16, |d| <= 2e-2 * RMS(ref) + 2^-8 |ref|
    per element (the second term is the rounding of a bf16 output); fp32,
    |d| <= 1e-4. `allowance_used` is the largest |d| over its allowance."""
    gidx = np.asarray(gpu["idx"])[tok]
    mism = np.flatnonzero((gidx != ref["idx"]).any(1))
    sets = sum(set(gidx[i].tolist()) != set(ref["idx"][i].tolist()) for i in mism)
    gaps = []
    for i in mism:
        s_ = np.sort(ref["logits"][i].astype(np.float64))[::-1]
        gaps.append(float(s_[cfg.k - 1] - s_[cfg.k]) if cfg.k < cfg.E else float("inf"))
    out = np.array(ref["out"], dtype=np.float64)
    if len(mism):
        out[mism] = forward(tok[mism], forced_idx=np.ascontiguousarray(gidx[mism]))["out"]
    got = np.asarray(gpu["out"])[tok].astype(np.float64)
    d = np.abs(got - out)
    rms = float(np.sqrt((out ** 2).mean()))
    if cfg.dtype == "bf16":
        allow = 2e-2 * rms + 2.0 ** -8 * np.abs(out)
        tol = "|d| <= 2e-2*RMS(ref) + 2^-8*|ref| per element"
    else:
        allow = np.full_like(out, 1e-4)
        tol = "|d| <= 1e-4 per element"
    used = float((d / np.maximum(allow, 1e-300)).max())
    return {"sample_tokens": int(len(tok)), "index_mismatch_tokens": int(len(mism)),
            "expert_set_mismatch_tokens": int(sets),
            "max_kth_gap_of_mismatches": max(gaps) if gaps else None,
            "max_d_over_rms": float(d.max() / rms), "rms_d_over_rms":
            float(np.sqrt((d ** 2).mean()) / rms),
            "max_ref_over_rms": float(np.abs(out).max() / rms), "allowance_used": used,
            "within_tolerance": bool(used <= 1.0), "tolerance": tol,
            "reference": "oracle (fp64), mismatched selections recomputed with the GPU's"}


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


def graph_replay_ms(torch, fn, steps):
    """The step fn captured once in a HIP graph (torch.cuda.CUDAGraph, after
    one eager call on a side stream) and replayed `steps` times back to back:
    ms per replay from HIP events around the replays."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    return ms


def measure(torch, binding, cfg, args, steps, w4=False, cap_factor=0.0, router="plain",
            dynamic_k_min=0, fallback_min=0):
    """Everything the JSON line reports about one workload, except the CPU
    baseline: the timed steps, the dominant kernel's roofline, the stages,
    the clock, and for weight-streaming workloads the MALL-scrubbed variants.
    Returns (report dict, inputs, 4-bit inputs or None)."""
    from sparse_mixture_experts_40_amd.inputs import (make_inputs, make_router_variant_inputs,
                                                      make_w4_inputs)
    log(f"workload {cfg}")
    t0 = time.perf_counter()
    inp = make_inputs(cfg, weights=not w4)
    w4in = make_w4_inputs(cfg) if w4 else None
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    cap = binding.capacity(binding.make_config(cfg), cap_factor) if cap_factor > 0 else 0
    var = make_router_variant_inputs(cfg) if router != "plain" else {}
    blk = binding.MoEBlock(cfg, inp, capacity=cap,
                           noise=var.get("noise") if "noise" in router else None,
                           w_noise=var.get("w_noise") if "noise" in router else None,
                           select_bias=var.get("select_bias") if "bias" in router else None,
                           dynamic_k_min=dynamic_k_min, w4=w4in, fallback_min=fallback_min)
    x = binding.to_device(inp["x"])
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        blk.forward(x)
    torch.cuda.synchronize()

    # the timed steps, one event before each (and one after the last)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    with ClockSampler(clock_files(torch)) as clk:
        w0 = time.perf_counter()
        for i in range(steps):
            evs[i].record(stream)
            blk.forward(x)
        evs[steps].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
    ms_step = evs[0].elapsed_time(evs[steps]) / steps
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    log(f"{cfg.name}: {ms_step:.4f} ms/step (events), wall {wall * 1e3 / steps:.4f} ms/step")
    if args.layer_only:  # profiling: nothing but the warm-up and the timed steps
        return {"ms_per_step": ms_step, "value": cfg.T / (ms_step * 1e-3),
                "step_ms": dist(step_ms)}, inp, w4in
    g_ms = graph_replay_ms(torch, lambda: blk.forward(x), steps)
    graph = {"ms_per_step": g_ms, "tokens_per_s": cfg.T / (g_ms * 1e-3), "replays": steps}
    log(f"{cfg.name}: {g_ms:.4f} ms/step replayed from a HIP graph")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    streaming = uses_decode_kernel(cfg) or w4
    scrub = torch.ones(1 << 27, dtype=torch.float32, device="cuda") if streaming else None
    scrubs = {"read": lambda i: scrub.sum(), "write": lambda i: scrub.fill_(float(i))}

    def scrubbed_times(fn, how):
        """Per-call times of fn with 512 MB of other data read or written before
        each call (outside the events)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
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
    # the routing after a capacity limit with the least-loaded fallback
    idx2 = torch.empty(T, k, dtype=torch.int32, device="cuda") if fallback_min else None
    w2 = torch.empty(T, k, dtype=torch.float32, device="cuda") if fallback_min else None
    counts2 = torch.empty(E, dtype=torch.int32, device="cuda")
    binding.router_topk_ex(c, blk.opts, x, blk.w_router, blk.logit_bias, None, idx, wts, blk.ws)

    def disp():
        if cap and fallback_min:  # dropless dispatch, the fallback routing, its dispatch
            binding.dispatch(c, idx, counts, offsets, sp, pp, blk.ws)
            binding.capacity_fallback(c, idx, wts, cap, fallback_min, offsets, sp, pp, idx2, w2)
            binding.dispatch(c, idx2, counts2, offsets, sp, pp, blk.ws)
        elif cap:
            binding.dispatch_capacity(c, idx, cap, counts, offsets, sp, pp, blk.ws)
        else:
            binding.dispatch(c, idx, counts, offsets, sp, pp, blk.ws)

    disp()

    def gate_up():
        if w4:
            binding.expert_gate_up_w4(c, x, sp, offsets, blk.w4_struct, h)
        else:
            binding.expert_gate_up(c, x, sp, offsets, blk.w_gate, blk.w_up, h)

    for _ in range(2):
        gate_up()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(steps):
        gate_up()
    ev1.record(stream)
    torch.cuda.synchronize()
    gu_ms = ev0.elapsed_time(ev1) / steps
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
        if w4:
            binding.expert_down_w4(c, h, offsets, blk.w4_struct, y)
        else:
            binding.expert_down(c, h, offsets, blk.w_down, y)

    wc = w2 if fallback_min else wts  # the combine's weights
    stage_fns = [
        ("router", lambda: binding.router_topk_ex(c, blk.opts, x, blk.w_router, blk.logit_bias,
                                                  None, idx, wts, blk.ws)),
        ("dispatch", disp),
        ("gate_up", gate_up),
        ("down", down),
        ("combine", lambda: binding.combine(c, y, pp, wc, out)),
        ("aux_stats_from_logits", lambda: binding.aux_stats(c, lg, idx, blk.ws, counts=counts,
                                                            f=blk.f, P=blk.P, aux=blk.aux)),
    ]
    stages = {n: pct(time_per_call(torch, stream, fn, max(10, steps)), 50)
              for n, fn in stage_fns}
    disp()  # counts / offsets of the router's selection again
    torch.cuda.synchronize()
    # rows per expert of the routing the experts ran (with the fallback, its own)
    cnt = (counts2 if cap and fallback_min else counts).cpu().numpy()
    rows = int(offsets[E].item())  # kept pairs (all of them without a capacity)
    gflops, gbytes, touched = gate_up_algorithmic(cfg, cnt, rows, w4)
    lflops, lbytes = layer_algorithmic(cfg, cnt, rows, w4)
    log(f"{cfg.name} gate/up kernel: {gu_ms:.4f} ms/launch, touched experts {touched}/{E}")

    decode = cfg.P <= 4 * cfg.E  # weight-streaming regime: bound by HBM
    traffic = measured_traffic(cfg.name) if not (cap or w4) else None
    if decode:
        achieved = gbytes / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}
    else:
        peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS
        achieved = gflops / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": traffic}
    if w4:
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

    config = {"workload": cfg.name, "T": T, "H": cfg.H, "E": E, "k": k, "I": cfg.I,
              "norm_topk_prob": cfg.norm, "zipf_s": cfg.zipf_s, "seed": cfg.seed}
    if cap:
        config.update({"capacity_factor": cap_factor, "capacity": cap,
                       "dropped_pairs": int(blk.dropped.item()), "kept_pairs": rows})
        if fallback_min:
            config["capacity_fallback_min"] = fallback_min
    if router != "plain":
        config["router"] = router
    if w4:
        config["weights"] = "w4 (group 128, bf16 scale/bias)"
    if dynamic_k_min:
        kt = blk.k_per_token.cpu().numpy()
        config.update({"dynamic_k_min": dynamic_k_min, "mean_k": float(kt.mean()),
                       "routed_pairs": int(kt.sum())})
    rep = {
        "ms_per_step": ms_step, "value": T / (ms_step * 1e-3), "config": config,
        "graph_replay": graph,
        "roofline": roof, "step_ms": dist(step_ms), "stages_ms": stages,
        "gpu_clock": clk.summary(),
        "layer": {"tflops": lflops / (ms_step * 1e-3) / 1e12,
                  "mfma_frac": lflops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                  "hbm_gbs_min_bytes": lbytes / (ms_step * 1e-3) / 1e9,
                  "hbm_frac_min_bytes": lbytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "min_bytes": lbytes, "touched_experts": touched,
                  "wall_ms_per_step": wall * 1e3 / steps},
    }
    if scrubbed:
        rep["mall_scrubbed"] = scrubbed
    # the timed block's last output and selection, for the parity figures
    plain = not (cap or router != "plain" or dynamic_k_min)
    gpu = None
    if plain:
        blk.forward(x)
        torch.cuda.synchronize()
        gpu = {"out": blk.out.float().cpu().numpy(), "idx": blk.topk_idx.cpu().numpy()}
    rep["_gpu"] = gpu
    del blk, h, y
    return rep, inp, w4in


def decode_summary(rep):
    """The weight-streaming workload's figures as the "decode" object of the
    line: ms/step, tokens/s, the layer's fraction of HBM bandwidth (touched
    expert weights + router matrix + x + out over the step time), the gate/up
    roofline and the MALL-scrubbed variants."""
    lay = rep["layer"]
    return {"workload": rep["config"]["workload"], "config": rep["config"],
            "ms_per_step": rep["ms_per_step"], "tokens_per_s": rep["value"],
            "step_ms": rep["step_ms"], "layer_hbm_frac": lay["hbm_frac_min_bytes"],
            "layer_hbm_gbs": lay["hbm_gbs_min_bytes"], "layer_min_bytes": lay["min_bytes"],
            "touched_experts": lay["touched_experts"], "roofline": rep["roofline"],
            "graph_replay": rep.get("graph_replay"),
            "stages_ms": rep["stages_ms"], "mall_scrubbed": rep.get("mall_scrubbed"),
            "gpu_clock": rep["gpu_clock"]}


# ---- --rocprof: this command under rocprofv3, with a summary --------------
#
# The profiler runs bench.py again as a child process (the parent touches no
# GPU), and the summary tables are written from its CSV output, so every
# profile summary comes from committed code and names the commands behind it.

ROCPROF_PMC = {  # counter passes of each mode (one pass per inner list)
    "traffic": [["FETCH_SIZE"], ["WRITE_SIZE"]],
    "mops": [["SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE"]],
}


def rocprof_child_args(argv):
    """argv without the --rocprof and --rocprof-dir options."""
    out, skip = [], False
    for a in argv:
        if skip:
            skip = False
        elif a in ("--rocprof", "--rocprof-dir"):
            skip = True
        elif not a.startswith(("--rocprof=", "--rocprof-dir=")):
            out.append(a)
    return out


def short_kernel_name(name: str) -> str:
    """Kernel name without the namespace and the argument list."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("moe::(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def stats_table(path: str):
    """Markdown rows of a rocprofv3 kernel_stats.csv (durations in us)."""
    import csv
    out = ["| kernel | calls | average us | min us | max us | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(path)):
        out.append(f"| `{short_kernel_name(r['Name'])}` | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |")
    return out


def counter_per_kernel(path: str, counter: str, skip_first: bool):
    """Values of one counter per kernel, in dispatch order; with skip_first the
    first dispatch of each kernel (the warm-up step) is left out when there
    are more."""
    import csv
    acc = {}
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
    for r in rows:
        if r["Counter_Name"] == counter:
            acc.setdefault(short_kernel_name(r["Kernel_Name"]), []).append(
                float(r["Counter_Value"]))
    if skip_first:
        acc = {k: (v[1:] if len(v) > 1 else v) for k, v in acc.items()}
    return acc


def rocprof(mode: str, child: list, outdir: str, timeout_s: int = 240) -> int:
    """Runs `bench.py <child>` under rocprofv3 (mode stats: kernel trace and
    statistics; traffic: FETCH_SIZE and WRITE_SIZE passes over --layer-only
    steps plus the same counters on the 1 GiB copy calibration; mops: the
    bf16 MFMA ops counter over --layer-only steps) and writes
    <outdir>/summary.md. Returns 0, or the failing pass's status."""
    import subprocess
    os.makedirs(outdir, exist_ok=True)
    env = {**os.environ, "TMPDIR": os.environ.get("TMPDIR", "/tmp")}
    py = [sys.executable, os.path.join(ROOT, "bench.py")]
    layer = child + ([] if "--layer-only" in child else ["--layer-only"])
    passes = []  # (directory name, command, csv file)
    if mode == "stats":
        passes.append(("stats", ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv",
                                 "-d", f"{outdir}/stats", "-o", "run", "--", *py, *child],
                       "run_kernel_stats.csv"))
    else:
        runs = [(cs, layer, cs[0]) for cs in ROCPROF_PMC[mode]]
        if mode == "traffic":
            runs += [([c], ["--copy-calibration"], f"copy-{c}") for c in ("FETCH_SIZE", "WRITE_SIZE")]
        for cs, args_, name in runs:
            passes.append((name, ["timeout", "-s", "KILL", str(timeout_s), "rocprofv3", "--pmc", *cs,
                                  "--output-format", "csv", "-d", f"{outdir}/{name}", "-o", "run",
                                  "--", *py, *args_], "run_counter_collection.csv"))
    for name, cmd, csvname in passes:
        log(f"rocprof pass {name}: {' '.join(cmd)}")
        r = subprocess.run(cmd, cwd=ROOT, env=env)
        # rocprofv3 itself may exit non-zero after a complete run: the CSV decides
        if not os.path.exists(os.path.join(outdir, name, csvname)):
            log(f"rocprof pass {name} left no {csvname} (status {r.returncode})")
            return r.returncode or 1
    path = rocprof_summary(mode, child, outdir, [cmd for _, cmd, _ in passes])
    print(json.dumps({"rocprof": mode, "summary": path}), flush=True)
    return 0


def rocprof_summary(mode: str, child: list, outdir: str, commands: list) -> str:
    """Writes <outdir>/summary.md from the CSV output of the passes of
    rocprof() (`commands`: their command lines) and returns its path."""
    layer = child + ([] if "--layer-only" in child else ["--layer-only"])

    def shown(cmd):
        return " ".join("python3" if c == sys.executable else
                        (os.path.relpath(c, ROOT) if c.startswith(ROOT) else c) for c in cmd)

    head = ["Command (repo root, one MI355X):", "",
            f"    python3 bench.py {' '.join(child)} --rocprof {mode} --rocprof-dir {outdir}", "",
            "which runs:", ""] + [f"    {shown(cmd)}" for cmd in commands] + [""]
    if mode == "stats":
        lines = [f"# rocprofv3 kernel statistics: bench.py {' '.join(child)}", "", *head,
                 "Durations in microseconds; the grouped GEMM template arguments are <GATEUP, BM, "
                 "BK, stages, waves, blocks per CU, non-temporal weights>.", "",
                 *stats_table(f"{outdir}/stats/run_kernel_stats.csv")]
    elif mode == "traffic":
        fe = counter_per_kernel(f"{outdir}/FETCH_SIZE/run_counter_collection.csv", "FETCH_SIZE", True)
        wr = counter_per_kernel(f"{outdir}/WRITE_SIZE/run_counter_collection.csv", "WRITE_SIZE", True)
        cf = counter_per_kernel(f"{outdir}/copy-FETCH_SIZE/run_counter_collection.csv", "FETCH_SIZE",
                                False)
        cw = counter_per_kernel(f"{outdir}/copy-WRITE_SIZE/run_counter_collection.csv", "WRITE_SIZE",
                                False)
        ck = [k for k in cf if "copyBuffer" in k][0]
        cfa, cwa = float(np.mean(cf[ck])), float(np.mean(cw[ck]))
        fs, ws = 1048576.0 / cfa, 1048576.0 / cwa
        lines = [f"# HBM traffic per kernel launch: bench.py {' '.join(layer)}", "", *head,
                 "One counter per pass, over the layer's own steps (`--layer-only`); values per "
                 "launch are the mean over the timed steps (the warm-up step's dispatches are left "
                 "out), scaled by what the same counters read for a plain copy of 1 GiB:", "",
                 "| copy kernel | FETCH_SIZE KiB | WRITE_SIZE KiB |", "|---|---|---|",
                 f"| `{ck}` (1 GiB read, 1 GiB written) | {cfa:.1f} | {cwa:.1f} |", "",
                 f"Scale factors: read bytes = FETCH_SIZE x {fs:.4f}; written bytes = "
                 f"WRITE_SIZE x {ws:.4f}.", "",
                 "| kernel | launches averaged | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB "
                 "(scaled) | HBM written MB (scaled) |", "|---|---|---|---|---|---|"]
        for k, v in fe.items():
            if "at::native" in k or "rocclr" in k:
                continue
            f, w = float(np.mean(v)), float(np.mean(wr.get(k, [0.0])))
            lines.append(f"| `{k}` | {len(v)} | {f:.1f} | {w:.1f} | {f * 1024 * fs / 1e6:.1f} | "
                         f"{w * 1024 * ws / 1e6:.1f} |")
        lines += ["", f"Sources sha256 (the stamp of measured traffic): {kernel_sources_sha256()}"]
    else:
        mo = counter_per_kernel(f"{outdir}/{ROCPROF_PMC['mops'][0][0]}/run_counter_collection.csv",
                                "SQ_INSTS_VALU_MFMA_MOPS_BF16", True)
        lines = [f"# bf16 MFMA work per kernel launch: bench.py {' '.join(layer)}", "", *head,
                 "Executed FLOP per launch = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (mean over the "
                 "timed steps; the warm-up step's dispatches are left out).", "",
                 "| kernel | launches averaged | MOPS per launch | executed TFLOP per launch |",
                 "|---|---|---|---|"]
        for k, v in mo.items():
            m = float(np.mean(v))
            if m > 0:
                lines.append(f"| `{k}` | {len(v)} | {m:.6g} | {m * 512 / 1e12:.4f} |")
    path = os.path.join(outdir, "summary.md")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill128_bf16")
    ap.add_argument("--decode-workload", default="decode128_bf16",
                    help="weight-streaming workload timed after the main one (the line's "
                         "\"decode\" object); 'none' to skip")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--capacity-factor", type=float, default=0.0,
                    help="> 0: capacity-limited dispatch with C = ceil(T*k*CF/E)")
    ap.add_argument("--capacity-fallback-min", type=int, default=0,
                    help="with --capacity-factor: a token keeping fewer than this many of its "
                         "slots gets the least-loaded experts in its dropped slots")
    ap.add_argument("--router", default="plain", choices=["plain", "noise", "bias", "noise+bias"],
                    help="router variant: noisy top-k and/or selection-only bias")
    ap.add_argument("--dynamic-k-min", type=int, default=0,
                    help="> 0: entropy-driven number of experts per token in [KMIN, k]")
    ap.add_argument("--w4", action="store_true",
                    help="4-bit group-quantised expert weights (codes + per-128 scale/bias)")
    ap.add_argument("--layer-only", action="store_true",
                    help="profiling: run only the warm-up and the timed layer steps, print "
                         "their time and exit (no kernel legs, stages or CPU baseline)")
    ap.add_argument("--rocprof", choices=["stats", "traffic", "mops"],
                    help="run this same command under rocprofv3 (child processes) and write "
                         "a summary: kernel statistics, HBM traffic per launch (with the copy "
                         "calibration) or bf16 MFMA work per launch")
    ap.add_argument("--rocprof-dir", default="rocprof_out",
                    help="where --rocprof puts the profiler output and summary.md")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of 1 GiB, 3 times: the "
                         "reference kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(no sharding, no collectives); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.rocprof:  # before anything touches the GPU
        sys.exit(rocprof(args.rocprof, rocprof_child_args(sys.argv[1:]), args.rocprof_dir))

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

    def workload(name):
        cfg = WORKLOADS[name]
        if args.seed != cfg.seed:
            cfg = type(cfg)(**{**cfg.__dict__, "seed": args.seed})
        return cfg

    cfg = workload(args.workload)
    binding.load()
    torch.cuda.init()
    rep, inp, w4in = measure(torch, binding, cfg, args, args.steps, w4=args.w4,
                             cap_factor=args.capacity_factor, router=args.router,
                             fallback_min=args.capacity_fallback_min,
                             dynamic_k_min=args.dynamic_k_min)
    if args.layer_only:
        print(json.dumps({"layer_only": True, "workload": cfg.name, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": rep["ms_per_step"],
                          "tokens_per_s": rep["value"], "step_ms": rep["step_ms"]}), flush=True)
        return
    line = {
        "metric": METRIC, "value": rep["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rep["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic", "config": rep["config"], "roofline": rep["roofline"],
        "step_ms": rep["step_ms"], "stages_ms": rep["stages_ms"], "gpu_clock": rep["gpu_clock"],
        "layer": rep["layer"], "graph_replay": rep.get("graph_replay"),
    }
    if "mall_scrubbed" in rep:
        line["mall_scrubbed"] = rep["mall_scrubbed"]
    plain = not (args.w4 or args.capacity_factor > 0 or args.router != "plain"
                 or args.dynamic_k_min)
    if plain and args.decode_workload != "none" and args.decode_workload != cfg.name:
        torch.cuda.empty_cache()
        drep, _, _ = measure(torch, binding, workload(args.decode_workload), args,
                             max(args.steps, args.decode_steps))
        line["decode"] = decode_summary(drep)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        line["cpu_baseline"], par = cpu_baseline(cfg, inp, args.cpu_budget, w4in,
                                                 gpu=rep.get("_gpu"))
        if par is not None:
            line["parity"] = par
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

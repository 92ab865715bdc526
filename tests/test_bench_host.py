"""Host-side checks of bench.py: the algorithmic costs behind the roofline
object, the kernel choice it reports, the traffic bookkeeping and the
one-GPU contract. No GPU is touched."""
import os
import re
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_mixture_experts_40_amd.configs import WORKLOADS  # noqa: E402


def test_prefill_gate_up_algorithmic_cost():
    cfg = WORKLOADS["prefill128_bf16"]
    counts = np.full(cfg.E, cfg.P // cfg.E)
    flops, nbytes, touched = bench.gate_up_algorithmic(cfg, counts, cfg.P)
    # 2 GEMMs (gate, up) of 2*H*I FLOP per routed pair
    assert flops == 4.0 * 4096 * 1536 * 131072
    assert touched == 128
    # gate + up weights of every expert, x read once, h written once (bf16)
    assert nbytes == 128 * 2 * 1536 * 4096 * 2 + 16384 * 4096 * 2 + 131072 * 1536 * 2


def test_decode_counts_only_touched_experts():
    cfg = WORKLOADS["decode128_bf16"]
    counts = np.zeros(cfg.E, np.int64)
    counts[:3] = [500, 10, 2]
    _, nbytes, touched = bench.gate_up_algorithmic(cfg, counts, int(counts.sum()))
    assert touched == 3
    assert nbytes == 3 * 2 * cfg.I * cfg.H * 2 + cfg.T * cfg.H * 2 + 512 * cfg.I * 2
    # 4-bit weights: half a byte per element plus a 4-byte pair per group of 128
    _, nbytes4, _ = bench.gate_up_algorithmic(cfg, counts, 512, w4=True)
    assert nbytes4 == 3 * 2 * cfg.I * cfg.H * (0.5 + 4 / 128) + cfg.T * cfg.H * 2 + 512 * cfg.I * 2


def test_kernel_choice_matches_workloads():
    assert not bench.uses_decode_kernel(WORKLOADS["prefill128_bf16"])
    assert bench.uses_decode_kernel(WORKLOADS["decode128_bf16"])
    assert not bench.uses_decode_kernel(WORKLOADS["tiny_f32"])


def test_traffic_bookkeeping():
    assert re.fullmatch(r"[0-9a-f]{64}", bench.kernel_sources_sha256())
    assert bench.measured_traffic("no_such_workload") is None
    t = bench.measured_traffic("prefill128_bf16")
    # either measured on these sources (then above the algorithmic bytes) or null
    assert t is None or t > 3.7e9


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr

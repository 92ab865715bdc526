"""Seeded synthetic inputs for the MoE block (shared by the GPU path's tests and
the oracle's; holds none of the block's arithmetic).

Recipe (every tensor, chunk by chunk, so generation is parallel and
reproducible on any machine):
  * tensor ids: x=0, w_router=1, w_gate=2, w_up=3, w_down=4;
  * the flattened tensor is cut into chunks of 2**22 elements; chunk c of
    tensor i draws standard normals (float32) from numpy's Philox bit generator
    seeded with SeedSequence(seed, spawn_key=(i, c));
  * values are scaled by 1/sqrt(fan_in) in float32 (fan_in = H for the router,
    gate and up projections, I for the down projection; x is unscaled), so the
    router logits have std ~1 and expert loads come out near-uniform;
  * bf16 workloads round every value to bf16 (round to nearest even); arrays
    are then the uint16 bit patterns;
  * skewed workloads (zipf_s > 0) add the per-expert logit bias
    log(Zipf_s(rank = e + 1)) = -s ln(e+1) - ln(sum_{r=1..E} r^-s);
  * router variants (make_router_variant_inputs): w_noise [E,H] like the
    router (scale 1/sqrt(H), bf16 for bf16 workloads), noise [T,E] float32
    standard normals, select_bias [E] float32 normals times 0.5;
  * 4-bit expert weights (make_w4_inputs): uniform random code bytes, and per
    group of 128 a bf16 scale s = |1 + 0.2 n1| / (4.6 sqrt(fan_in)) and bias
    b = -s (7.5 + 0.5 n2) (n1, n2 standard normals), so that s q + b with q
    uniform in 0..15 has mean ~0 and standard deviation ~1/sqrt(fan_in).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import MoEConfig

CHUNK = 1 << 22
TENSOR_IDS = {"x": 0, "w_router": 1, "w_gate": 2, "w_up": 3, "w_down": 4, "w_noise": 5,
              "noise": 6, "select_bias": 7, "gate_q": 8, "up_q": 9, "down_q": 10, "gate_s": 11,
              "up_s": 12, "down_s": 13, "gate_b": 14, "up_b": 15, "down_b": 16}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    """Exact float32 view of an input array (float32 or bf16 bits)."""
    return bf16_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


def normal_tensor(shape, seed: int, tensor_id: int, scale: float, bf16: bool) -> np.ndarray:
    """Chunked Philox standard normals times `scale`, optionally as bf16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16 if bf16 else np.float32)
    sc = np.float32(scale)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        ss = np.random.SeedSequence(seed, spawn_key=(tensor_id, c))
        z = np.random.Generator(np.random.Philox(ss)).standard_normal(hi - lo, dtype=np.float32)
        if sc != np.float32(1.0):
            z *= sc
        out[lo:hi] = bf16_bits(z) if bf16 else z

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def zipf_logit_bias(E: int, s: float) -> np.ndarray:
    """log of the Zipf(s) probability of rank e+1, as float32 [E]."""
    norm = math.log(sum(r ** (-s) for r in range(1, E + 1)))
    return np.array([-s * math.log(e + 1) - norm for e in range(E)], dtype=np.float32)


def make_inputs(cfg: MoEConfig, seed: int | None = None, tokens: int | None = None,
                weights: bool = True) -> dict:
    """Inputs of one workload: x [T,H], w_router [E,H], w_gate/w_up [E,I,H],
    w_down [E,H,I] (float32, or uint16 bf16 bits) and logit_bias (float32 [E]
    or None). `tokens` overrides T (x is a prefix-independent draw of its own
    size); weights=False skips the expert weights."""
    seed = cfg.seed if seed is None else seed
    bf = cfg.dtype == "bf16"
    T = cfg.T if tokens is None else tokens
    H, E, I = cfg.H, cfg.E, cfg.I
    d = {
        "x": normal_tensor((T, H), seed, TENSOR_IDS["x"], 1.0, bf),
        "w_router": normal_tensor((E, H), seed, TENSOR_IDS["w_router"], 1.0 / math.sqrt(H), bf),
        "logit_bias": zipf_logit_bias(E, cfg.zipf_s) if cfg.zipf_s > 0 else None,
    }
    if weights:
        d["w_gate"] = normal_tensor((E, I, H), seed, TENSOR_IDS["w_gate"], 1.0 / math.sqrt(H), bf)
        d["w_up"] = normal_tensor((E, I, H), seed, TENSOR_IDS["w_up"], 1.0 / math.sqrt(H), bf)
        d["w_down"] = normal_tensor((E, H, I), seed, TENSOR_IDS["w_down"], 1.0 / math.sqrt(I), bf)
    return d


def make_router_variant_inputs(cfg: MoEConfig, seed: int | None = None,
                               tokens: int | None = None) -> dict:
    """Inputs of the router variants: w_noise [E,H] (dtype of the workload),
    noise [T,E] float32 draws, select_bias [E] float32."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if tokens is None else tokens
    H, E = cfg.H, cfg.E
    return {
        "w_noise": normal_tensor((E, H), seed, TENSOR_IDS["w_noise"], 1.0 / math.sqrt(H),
                                 cfg.dtype == "bf16"),
        "noise": normal_tensor((T, E), seed, TENSOR_IDS["noise"], 1.0, False),
        "select_bias": normal_tensor((E,), seed, TENSOR_IDS["select_bias"], 0.5, False),
    }


def uniform_bytes(shape, seed: int, tensor_id: int) -> np.ndarray:
    """Chunked Philox uniform bytes (0..255), the same chunk seeding as
    normal_tensor."""
    n = int(np.prod(shape))
    out = np.empty(n, np.uint8)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c: int):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        ss = np.random.SeedSequence(seed, spawn_key=(tensor_id, c))
        out[lo:hi] = np.random.Generator(np.random.Philox(ss)).integers(0, 256, hi - lo,
                                                                        dtype=np.uint8)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def make_w4_inputs(cfg: MoEConfig, seed: int | None = None) -> dict:
    """4-bit expert weights in the tiled layout of moe.h: codes uint8
    [E,N/32,K/64,32,32] (gate/up N = I, K = H; down N = H, K = I) and *_sb
    uint16 bf16 bits [E,N/32,K/128,32,2] = (scale, bias) per row and group of
    128 consecutive K. The codes are uniform random bytes."""
    seed = cfg.seed if seed is None else seed
    H, E, I = cfg.H, cfg.E, cfg.I
    d = {}
    for name, N, K in (("gate", I, H), ("up", I, H), ("down", H, I)):
        d[name] = uniform_bytes((E, N, K // 2), seed, TENSOR_IDS[name + "_q"]).reshape(
            E, N // 32, K // 64, 32, 32)
        G = K // 128
        n1 = normal_tensor((E, N, G), seed, TENSOR_IDS[name + "_s"], 1.0, False)
        n2 = normal_tensor((E, N, G), seed, TENSOR_IDS[name + "_b"], 1.0, False)
        scale = (np.abs(1.0 + 0.2 * n1) / (4.6 * math.sqrt(K))).astype(np.float32)
        bias = (-scale * (7.5 + 0.5 * n2)).astype(np.float32)
        sbn = np.stack([bf16_bits(scale), bf16_bits(bias)], axis=-1)  # [E,N,G,2]
        d[name + "_sb"] = np.ascontiguousarray(
            sbn.reshape(E, N // 32, 32, G, 2).transpose(0, 1, 3, 2, 4))
    return d

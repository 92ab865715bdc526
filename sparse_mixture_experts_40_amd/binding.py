"""Thin ctypes binding over ``libmoe.so`` (C ABI in include/moe.h).

Argument marshalling only: every step of the block runs in the HIP kernels of
the library. Tensors are torch CUDA (HIP) tensors; calls are enqueued on
``torch.cuda.current_stream()``. There is no fallback: if the library is missing
or a call fails, this module raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import torch

from .configs import MoEConfig

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_DTYPE = {"f32": 0, "bf16": 1}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}

# public entry points of include/moe.h
EXPORTS = ("moe_workspace_size", "moe_status_string", "moe_router_topk", "moe_router_topk_ex",
           "moe_dispatch",
           "moe_capacity", "moe_dispatch_capacity", "moe_capacity_fallback",
           "moe_expert_gate_up", "moe_expert_down",
           "moe_expert_swiglu", "moe_combine", "moe_aux_stats", "moe_z_loss", "moe_layer_forward",
           "moe_layer_forward_ex", "moe_expert_gate_up_w4", "moe_expert_down_w4",
           "moe_layer_forward_w4", "moe_layer_forward_noalloc", "moe_w4_from_mlx")

# bytes of the library-owned scratch of moe_layer_forward_noalloc (moe.h)
NOALLOC_SCRATCH_BYTES = 32 << 20


class moe_config(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class moe_options(ctypes.Structure):
    _fields_ = [("capacity", ctypes.c_int32), ("dropped", ctypes.c_void_p),
                ("noise", ctypes.c_void_p), ("w_noise", ctypes.c_void_p),
                ("select_bias", ctypes.c_void_p), ("dynamic_k_min", ctypes.c_int32),
                ("k_per_token", ctypes.c_void_p), ("z_loss", ctypes.c_void_p),
                ("capacity_fallback_min", ctypes.c_int32)]


class moe_w4_weights(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_sb", ctypes.c_void_p), ("up_sb", ctypes.c_void_p),
                ("down_sb", ctypes.c_void_p)]


class moe_aux_out(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("f", ctypes.c_void_p), ("P", ctypes.c_void_p),
                ("aux", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_mixture_experts_40_amd.build`")
    lib = ctypes.CDLL(path)
    V, S, C = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(moe_config)
    st = ctypes.c_int
    lib.moe_workspace_size.argtypes, lib.moe_workspace_size.restype = [C], S
    lib.moe_status_string.argtypes, lib.moe_status_string.restype = [st], ctypes.c_char_p
    lib.moe_capacity.argtypes, lib.moe_capacity.restype = [C, ctypes.c_float], ctypes.c_int32
    sig = {
        "moe_router_topk": [C, V, V, V, V, V, V, V],
        "moe_router_topk_ex": [C, ctypes.POINTER(moe_options), V, V, V, V, V, V, V, S, V],
        "moe_dispatch": [C, V, V, V, V, V, V, S, V],
        "moe_dispatch_capacity": [C, V, ctypes.c_int32, V, V, V, V, V, V, S, V],
        "moe_capacity_fallback": [C, V, V, ctypes.c_int32, ctypes.c_int32, V, V, V, V, V, V, V],
        "moe_expert_gate_up": [C, V, V, V, V, V, V, V, S, V],
        "moe_expert_down": [C, V, V, V, V, V, S, V],
        "moe_expert_swiglu": [C, V, V, V, V, V, V, V, V, S, V],
        "moe_combine": [C, V, V, V, V, V],
        "moe_aux_stats": [C, V, V, moe_aux_out, V, S, V],
        "moe_z_loss": [C, V, V, V, S, V],
        "moe_layer_forward": [C, V, V, V, V, V, V, V, V, V, V, moe_aux_out, V, S, V],
        "moe_layer_forward_ex": [C, ctypes.POINTER(moe_options), V, V, V, V, V, V, V, V, V, V,
                                 moe_aux_out, V, S, V],
        "moe_expert_gate_up_w4": [C, V, V, V, ctypes.POINTER(moe_w4_weights), V, V],
        "moe_expert_down_w4": [C, V, V, ctypes.POINTER(moe_w4_weights), V, V],
        "moe_layer_forward_noalloc": [C, V, V, V, V, V, V, V, V, V, V, moe_aux_out, V],
        "moe_layer_forward_w4": [C, ctypes.POINTER(moe_options), V, V, V,
                                 ctypes.POINTER(moe_w4_weights), V, V, V, V, moe_aux_out, V, S,
                                 V],
        "moe_w4_from_mlx": [st, st, st, V, V, V, V, V],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes, f.restype = args, st
    _lib = lib
    return lib


def make_config(cfg: MoEConfig, T: int | None = None) -> moe_config:
    return moe_config(cfg.T if T is None else T, cfg.H, cfg.E, cfg.k, cfg.I, int(cfg.norm),
                      MOE_DTYPE[cfg.dtype])


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, name: str):
    if status != 0:
        msg = load().moe_status_string(status).decode()
        raise RuntimeError(f"{name} failed: {msg} ({status})")


def workspace_size(c: moe_config) -> int:
    return int(load().moe_workspace_size(ctypes.byref(c)))


def alloc_workspace(c: moe_config, device="cuda") -> torch.Tensor:
    n = workspace_size(c)
    if n == 0:
        raise ValueError("invalid MoE configuration")
    return torch.empty(n, dtype=torch.uint8, device=device)


def router_topk(c: moe_config, x, w_router, logit_bias, logits, topk_idx, topk_w):
    _check(load().moe_router_topk(ctypes.byref(c), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                  _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _stream()),
           "moe_router_topk")


def options(capacity: int = 0, dropped=None, noise=None, w_noise=None, select_bias=None,
            dynamic_k_min: int = 0, k_per_token=None, z_loss=None,
            fallback_min: int = 0) -> moe_options:
    """moe_options from tensors (the tensors must outlive the calls)."""
    return moe_options(int(capacity), _ptr(dropped), _ptr(noise), _ptr(w_noise),
                       _ptr(select_bias), int(dynamic_k_min), _ptr(k_per_token), _ptr(z_loss),
                       int(fallback_min))


def router_topk_ex(c: moe_config, opts: moe_options | None, x, w_router, logit_bias, logits,
                   topk_idx, topk_w, ws=None):
    _check(load().moe_router_topk_ex(ctypes.byref(c), None if opts is None else ctypes.byref(opts),
                                     _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(logits),
                                     _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream()),
           "moe_router_topk_ex")


def dispatch(c: moe_config, topk_idx, counts, offsets, sorted_pair, pair_pos, ws):
    _check(load().moe_dispatch(ctypes.byref(c), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                               _ptr(sorted_pair), _ptr(pair_pos), _ptr(ws), ws.numel(),
                               _stream()), "moe_dispatch")


def capacity(c: moe_config, capacity_factor: float) -> int:
    n = int(load().moe_capacity(ctypes.byref(c), float(capacity_factor)))
    if n <= 0:
        raise ValueError("invalid configuration or capacity factor")
    return n


def dispatch_capacity(c: moe_config, topk_idx, cap: int, counts, offsets, sorted_pair, pair_pos,
                      ws, dropped=None):
    _check(load().moe_dispatch_capacity(ctypes.byref(c), _ptr(topk_idx), int(cap), _ptr(counts),
                                        _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos),
                                        _ptr(dropped), _ptr(ws), ws.numel(), _stream()),
           "moe_dispatch_capacity")


def capacity_fallback(c: moe_config, topk_idx, topk_w, cap: int, fallback_min: int, offsets,
                      sorted_pair, pair_pos, idx_out, w_out, dropped=None):
    _check(load().moe_capacity_fallback(ctypes.byref(c), _ptr(topk_idx), _ptr(topk_w), int(cap),
                                        int(fallback_min), _ptr(offsets), _ptr(sorted_pair),
                                        _ptr(pair_pos), _ptr(idx_out), _ptr(w_out), _ptr(dropped),
                                        _stream()),
           "moe_capacity_fallback")


def expert_gate_up(c: moe_config, x, sorted_pair, offsets, w_gate, w_up, h, ws=None):
    _check(load().moe_expert_gate_up(ctypes.byref(c), _ptr(x), _ptr(sorted_pair), _ptr(offsets),
                                     _ptr(w_gate), _ptr(w_up), _ptr(h), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream()),
           "moe_expert_gate_up")


def expert_down(c: moe_config, h, offsets, w_down, y_sorted, ws=None):
    _check(load().moe_expert_down(ctypes.byref(c), _ptr(h), _ptr(offsets), _ptr(w_down),
                                  _ptr(y_sorted), _ptr(ws), 0 if ws is None else ws.numel(),
                                  _stream()), "moe_expert_down")


def expert_swiglu(c: moe_config, x, sorted_pair, offsets, w_gate, w_up, w_down, y_sorted, ws):
    _check(load().moe_expert_swiglu(ctypes.byref(c), _ptr(x), _ptr(sorted_pair), _ptr(offsets),
                                    _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(y_sorted),
                                    _ptr(ws), ws.numel(), _stream()), "moe_expert_swiglu")


def combine(c: moe_config, y_sorted, pair_pos, topk_w, out):
    _check(load().moe_combine(ctypes.byref(c), _ptr(y_sorted), _ptr(pair_pos), _ptr(topk_w),
                              _ptr(out), _stream()), "moe_combine")


def _aux(counts=None, f=None, P=None, aux=None) -> moe_aux_out:
    return moe_aux_out(_ptr(counts), _ptr(f), _ptr(P), _ptr(aux))


def aux_stats(c: moe_config, logits, topk_idx, ws, counts=None, f=None, P=None, aux=None,
              z_loss=None):
    """moe_aux_stats, and moe_z_loss when z_loss is given."""
    _check(load().moe_aux_stats(ctypes.byref(c), _ptr(logits), _ptr(topk_idx),
                                _aux(counts, f, P, aux), _ptr(ws), ws.numel(), _stream()),
           "moe_aux_stats")
    if z_loss is not None:
        z_loss_stat(c, logits, z_loss, ws)


def z_loss_stat(c: moe_config, logits, z_loss, ws):
    _check(load().moe_z_loss(ctypes.byref(c), _ptr(logits), _ptr(z_loss), _ptr(ws), ws.numel(),
                             _stream()), "moe_z_loss")


def layer_forward(c: moe_config, x, w_router, logit_bias, w_gate, w_up, w_down, out, ws,
                  router_logits=None, topk_idx=None, topk_w=None, counts=None, f=None, P=None,
                  aux=None):
    _check(load().moe_layer_forward(ctypes.byref(c), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                    _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out),
                                    _ptr(router_logits), _ptr(topk_idx), _ptr(topk_w),
                                    _aux(counts, f, P, aux), _ptr(ws), ws.numel(), _stream()),
           "moe_layer_forward")


def layer_forward_noalloc(c: moe_config, x, w_router, logit_bias, w_gate, w_up, w_down, out,
                          router_logits=None, topk_idx=None, topk_w=None, counts=None, f=None,
                          P=None, aux=None):
    """moe_layer_forward without a workspace (the library's own scratch array)."""
    _check(load().moe_layer_forward_noalloc(ctypes.byref(c), _ptr(x), _ptr(w_router),
                                            _ptr(logit_bias), _ptr(w_gate), _ptr(w_up),
                                            _ptr(w_down), _ptr(out), _ptr(router_logits),
                                            _ptr(topk_idx), _ptr(topk_w), _aux(counts, f, P, aux),
                                            _stream()),
           "moe_layer_forward_noalloc")


def w4_from_mlx(mlx_w, mlx_scales, mlx_biases) -> tuple:
    """moe_w4_from_mlx on host arrays: mlx_w uint32 [E,N,K/8], scales and
    biases uint16 (bf16 bits) [E,N,K/128] -> (codes uint8 [E,N/32,K/64,32,32],
    sb uint16 [E,N/32,K/128,32,2])."""
    w = np.ascontiguousarray(mlx_w, dtype=np.uint32)
    sc = np.ascontiguousarray(mlx_scales, dtype=np.uint16)
    bi = np.ascontiguousarray(mlx_biases, dtype=np.uint16)
    E, N, K8 = w.shape
    K = 8 * K8
    if sc.shape != (E, N, K // 128) or bi.shape != sc.shape:
        raise ValueError(f"scales/biases must be [E, N, K/128] = {(E, N, K // 128)}")
    codes = np.empty((E, N // 32, K // 64, 32, 32), np.uint8)
    sb = np.empty((E, N // 32, K // 128, 32, 2), np.uint16)
    _check(load().moe_w4_from_mlx(E, N, K, w.ctypes.data, sc.ctypes.data, bi.ctypes.data,
                                  codes.ctypes.data, sb.ctypes.data), "moe_w4_from_mlx")
    return codes, sb


def _with_z_loss(opts: moe_options | None, z_loss) -> moe_options | None:
    """opts with its z_loss output set to z_loss (a copy; opts is unchanged)."""
    if z_loss is None:
        return opts
    o = moe_options()
    if opts is not None:
        ctypes.pointer(o)[0] = opts
    o.z_loss = _ptr(z_loss)
    return o


def layer_forward_ex(c: moe_config, opts: moe_options | None, x, w_router, logit_bias, w_gate,
                     w_up, w_down, out, ws, router_logits=None, topk_idx=None, topk_w=None,
                     counts=None, f=None, P=None, aux=None, z_loss=None):
    opts = _with_z_loss(opts, z_loss)
    _check(load().moe_layer_forward_ex(ctypes.byref(c), None if opts is None else ctypes.byref(opts),
                                       _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(w_gate),
                                       _ptr(w_up), _ptr(w_down), _ptr(out), _ptr(router_logits),
                                       _ptr(topk_idx), _ptr(topk_w), _aux(counts, f, P, aux),
                                       _ptr(ws), ws.numel(), _stream()),
           "moe_layer_forward_ex")


def w4_weights(t: dict) -> moe_w4_weights:
    """moe_w4_weights from a dict of device tensors gate/up/down (uint8 codes)
    and gate_sb/up_sb/down_sb (bf16 (scale, bias) pairs)."""
    return moe_w4_weights(*(_ptr(t[n]) for n in ("gate", "up", "down", "gate_sb", "up_sb",
                                                  "down_sb")))


def w4_to_device(w4: dict, device="cuda") -> dict:
    """numpy 4-bit weights (make_w4_inputs layout) -> device tensors."""
    import numpy as np
    out = {}
    for n, a in w4.items():
        if a.dtype == np.uint16:
            out[n] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(device)
        else:
            out[n] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out


def expert_gate_up_w4(c: moe_config, x, sorted_pair, offsets, w4: moe_w4_weights, h):
    _check(load().moe_expert_gate_up_w4(ctypes.byref(c), _ptr(x), _ptr(sorted_pair),
                                        _ptr(offsets), ctypes.byref(w4), _ptr(h), _stream()),
           "moe_expert_gate_up_w4")


def expert_down_w4(c: moe_config, h, offsets, w4: moe_w4_weights, y_sorted):
    _check(load().moe_expert_down_w4(ctypes.byref(c), _ptr(h), _ptr(offsets), ctypes.byref(w4),
                                     _ptr(y_sorted), _stream()), "moe_expert_down_w4")


def layer_forward_w4(c: moe_config, opts: moe_options | None, x, w_router, logit_bias,
                     w4: moe_w4_weights, out, ws, router_logits=None, topk_idx=None, topk_w=None,
                     counts=None, f=None, P=None, aux=None, z_loss=None):
    opts = _with_z_loss(opts, z_loss)
    _check(load().moe_layer_forward_w4(ctypes.byref(c), None if opts is None else ctypes.byref(opts),
                                       _ptr(x), _ptr(w_router), _ptr(logit_bias), ctypes.byref(w4),
                                       _ptr(out), _ptr(router_logits), _ptr(topk_idx),
                                       _ptr(topk_w), _aux(counts, f, P, aux), _ptr(ws),
                                       ws.numel(), _stream()),
           "moe_layer_forward_w4")


def to_device(a, device="cuda") -> torch.Tensor:
    """numpy input array (float32, or uint16 bf16 bits) -> GPU tensor of the
    matching torch dtype (bf16 bits are reinterpreted, not converted)."""
    import numpy as np
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def _as_tensor(a, device):
    if a is None or isinstance(a, torch.Tensor):
        return a
    return to_device(a, device)


class MoEBlock:
    """Device-resident block: holds the weights and a workspace, runs the
    whole forward with one library call per step."""

    def __init__(self, cfg: MoEConfig, inputs: dict, device="cuda", capacity: int = 0,
                 noise=None, w_noise=None, select_bias=None, dynamic_k_min: int = 0, w4=None,
                 fallback_min: int = 0):
        """capacity > 0: capacity-limited dispatch (see moe_capacity), with
        fallback_min > 0 the least-loaded fallback (moe_capacity_fallback); noise
        [T,E] fp32 + w_noise [E,H]: noisy top-k; select_bias [E] fp32:
        selection-only bias (numpy arrays or tensors); dynamic_k_min > 0:
        entropy-driven k in [dynamic_k_min, k]; w4: 4-bit expert weights
        (make_w4_inputs layout) used instead of inputs' w_gate/w_up/w_down."""
        self.cfg = cfg
        self.c = make_config(cfg)
        self.dropped = torch.zeros(1, dtype=torch.int32, device=device)
        self.noise = _as_tensor(noise, device)
        self.w_noise = _as_tensor(w_noise, device)
        self.select_bias = _as_tensor(select_bias, device)
        self.k_per_token = torch.empty(cfg.T, dtype=torch.int32, device=device)
        variant = capacity or noise is not None or select_bias is not None or dynamic_k_min
        self.opts = options(capacity, self.dropped, self.noise, self.w_noise, self.select_bias,
                            dynamic_k_min, self.k_per_token,
                            fallback_min=fallback_min) if variant else None
        self.w_router = to_device(inputs["w_router"], device)
        self.w4 = w4_to_device(w4, device) if w4 is not None else None
        self.w4_struct = w4_weights(self.w4) if w4 is not None else None
        if w4 is None:
            self.w_gate = to_device(inputs["w_gate"], device)
            self.w_up = to_device(inputs["w_up"], device)
            self.w_down = to_device(inputs["w_down"], device)
        self.logit_bias = to_device(inputs.get("logit_bias"), device)
        self.ws = alloc_workspace(self.c, device)
        T, E, k = cfg.T, cfg.E, cfg.k
        self.out = torch.empty(T, cfg.H, dtype=TORCH_DTYPE[cfg.dtype], device=device)
        self.logits = torch.empty(T, E, dtype=torch.float32, device=device)
        self.topk_idx = torch.empty(T, k, dtype=torch.int32, device=device)
        self.topk_w = torch.empty(T, k, dtype=torch.float32, device=device)
        self.counts = torch.empty(E, dtype=torch.int32, device=device)
        self.f = torch.empty(E, dtype=torch.float32, device=device)
        self.P = torch.empty(E, dtype=torch.float32, device=device)
        self.aux = torch.empty(1, dtype=torch.float32, device=device)
        self.z_loss = torch.empty(1, dtype=torch.float32, device=device)

    def forward(self, x: torch.Tensor, outputs: bool = True):
        """outputs=False: only `out` (logits, selection and statistics stay in
        the workspace / are not computed)."""
        if self.w4 is not None:
            extra = (self.logits, self.topk_idx, self.topk_w, self.counts, self.f, self.P,
                     self.aux, self.z_loss) if outputs else ()
            layer_forward_w4(self.c, self.opts, x, self.w_router, self.logit_bias,
                             self.w4_struct, self.out, self.ws, *extra)
        elif outputs:
            layer_forward_ex(self.c, self.opts, x, self.w_router, self.logit_bias, self.w_gate,
                             self.w_up, self.w_down, self.out, self.ws, self.logits,
                             self.topk_idx, self.topk_w, self.counts, self.f, self.P, self.aux,
                             self.z_loss)
        else:
            layer_forward_ex(self.c, self.opts, x, self.w_router, self.logit_bias, self.w_gate,
                             self.w_up, self.w_down, self.out, self.ws)
        return self.out

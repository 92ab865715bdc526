"""Python view of the plain CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The GPU product path
never calls it and shares no code with it.

Arrays are numpy: fp32 configs pass float32 arrays, bf16 configs pass the bf16
bit patterns as uint16 arrays (the C side widens them exactly). Outputs that the
definition computes in double (weights, probabilities, expert outputs, the block
output) come back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.orc_logits.argtypes = [i, i, i, i, P, P, P, P]
        lib.orc_route.argtypes = [i, i, i, i, P, P, P, P, P]
        lib.orc_route_sel.argtypes = [i, i, i, i, P, P, P, P, P, P]
        lib.orc_noisy_logits.argtypes = [i, i, P, P, P, P]
        lib.orc_z_loss.argtypes = [i, i, P, P]
        lib.orc_route_dynamic.argtypes = [i, i, i, i, i, P, P, P, P, P]
        lib.orc_dequant_w4.argtypes = [i, i, i, P, P, P]
        lib.orc_expert_rows_w4.argtypes = [i, i, i, P, P, P, P, P, P, P, i, P, P, i, P]
        lib.orc_expert_rows_f64w.argtypes = [i, i, i, P, P, P, P, i, P, P, P]
        lib.orc_dispatch.argtypes = [i, i, i, P, P, P, P, P]
        lib.orc_expert_rows.argtypes = [i, i, i, P, P, P, P, i, P, P, i, P]
        lib.orc_combine.argtypes = [i, i, i, P, P, P]
        lib.orc_combine_kept.argtypes = [i, i, i, P, P, P, P]
        lib.orc_capacity.argtypes = [i, i, i, ctypes.c_double]
        lib.orc_dispatch_capacity.argtypes = [i, i, i, i, P, P, P, P, P, P]
        lib.orc_aux.argtypes = [i, i, i, P, P, P, P, P]
        lib.orc_capacity_fallback.argtypes = [i, i, i, i, i, P, P, P, P, P]
        lib.orc_forward_tokens.argtypes = [i, i, i, i, i, i, i, P, P, P, P, P, P, i, P, P, P, i,
                                           P, P, P, P]
        for f in (lib.orc_logits, lib.orc_route, lib.orc_dispatch, lib.orc_expert_rows,
                  lib.orc_combine, lib.orc_combine_kept, lib.orc_capacity,
                  lib.orc_dispatch_capacity, lib.orc_aux, lib.orc_forward_tokens,
                  lib.orc_route_sel, lib.orc_noisy_logits, lib.orc_z_loss,
                  lib.orc_route_dynamic, lib.orc_dequant_w4, lib.orc_expert_rows_w4,
                  lib.orc_expert_rows_f64w, lib.orc_capacity_fallback):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"oracle {name}: bad argument")


def logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """Router logits [T,E] fp32 (fp64 sum, one rounding)."""
    x, w_router = _c(x), _c(w_router)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = w_router.shape[0]
    assert w_router.shape == (E, H) and x.dtype == w_router.dtype
    out = np.empty((T, E), np.float32)
    _check(_load().orc_logits(T, H, E, _dtype_code(x), _p(x), _p(w_router), _p(bias), _p(out)),
           "logits")
    return out


def route(lg: np.ndarray, k: int, norm: bool, forced_idx: np.ndarray | None = None,
          sel_bias: np.ndarray | None = None):
    """Softmax + top-k (+ renormalisation); sel_bias [E] (optional) moves only
    the selection. Returns (idx int32 [T,k], w float64 [T,k], probs float64 [T,E])."""
    lg = _c(lg, np.float32)
    T, E = lg.shape
    forced_idx = _c(forced_idx, np.int32)
    sel_bias = _c(sel_bias, np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    probs = np.empty((T, E), np.float64)
    _check(_load().orc_route_sel(T, E, k, int(bool(norm)), _p(lg), _p(sel_bias), _p(forced_idx),
                                 _p(idx), _p(w), _p(probs)), "route")
    return idx, w, probs


def route_dynamic(lg: np.ndarray, k_max: int, k_min: int, norm: bool):
    """Entropy-driven k per token. Returns (idx int32 [T,k_max] (-1 past k_t),
    w float64 [T,k_max] (0 past k_t), kt int32 [T], x float64 [T] (unfloored))."""
    lg = _c(lg, np.float32)
    T, E = lg.shape
    idx = np.empty((T, k_max), np.int32)
    w = np.empty((T, k_max), np.float64)
    kt = np.empty(T, np.int32)
    x = np.empty(T, np.float64)
    _check(_load().orc_route_dynamic(T, E, k_max, k_min, int(bool(norm)), _p(lg), _p(idx), _p(w),
                                     _p(kt), _p(x)), "route_dynamic")
    return idx, w, kt, x


def noisy_logits(lg: np.ndarray, nlg: np.ndarray, noise: np.ndarray) -> np.ndarray:
    """fp32( l + noise * softplus(nl) ) [T,E]."""
    lg, nlg, noise = _c(lg, np.float32), _c(nlg, np.float32), _c(noise, np.float32)
    T, E = lg.shape
    assert nlg.shape == (T, E) and noise.shape == (T, E)
    out = np.empty((T, E), np.float32)
    _check(_load().orc_noisy_logits(T, E, _p(lg), _p(nlg), _p(noise), _p(out)), "noisy_logits")
    return out


def z_loss(lg: np.ndarray) -> float:
    """(1/T) sum_t logsumexp(l_t)^2."""
    lg = _c(lg, np.float32)
    T, E = lg.shape
    z = np.empty(1, np.float64)
    _check(_load().orc_z_loss(T, E, _p(lg), _p(z)), "z_loss")
    return float(z[0])


def dispatch(idx: np.ndarray, E: int):
    """Counting sort of the pairs by expert. Returns (counts [E],
    offsets [E+1], sorted_pair [P], pair_pos [P]), all int32."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    pp = np.empty(T * k, np.int32)
    _check(_load().orc_dispatch(T, E, k, _p(idx), _p(counts), _p(offsets), _p(sp), _p(pp)),
           "dispatch")
    return counts, offsets, sp, pp


def capacity(T: int, E: int, k: int, cf: float) -> int:
    """Expert capacity ceil(T*k*cf/E) (at least 1, at most T*k)."""
    c = _load().orc_capacity(T, E, k, float(cf))
    _check(0 if c > 0 else -1, "capacity")
    return c


def dispatch_capacity(idx: np.ndarray, E: int, cap: int):
    """Capacity-limited dispatch. Returns (counts [E] before the limit,
    offsets [E+1] of the kept pairs, sorted_pair [P] (first offsets[E] valid),
    pair_pos [P] (-1 = dropped), dropped)."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sp = np.full(T * k, -1, np.int32)
    pp = np.empty(T * k, np.int32)
    dropped = np.zeros(1, np.int32)
    _check(_load().orc_dispatch_capacity(T, E, k, int(cap), _p(idx), _p(counts), _p(offsets),
                                         _p(sp), _p(pp), _p(dropped)), "dispatch_capacity")
    return counts, offsets, sp, pp, int(dropped[0])


def capacity_fallback(idx: np.ndarray, w: np.ndarray, E: int, cap: int, fallback_min: int):
    """Capacity-limited routing with the least-loaded fallback ([T,k] idx with
    -1 for empty slots, [T,k] float32 weights). Returns (idx_out [T,k] int32,
    -1 where no expert; w_out [T,k] float32; dropped slots left over)."""
    idx = _c(idx, np.int32)
    w = _c(w, np.float32)
    T, k = idx.shape
    io = np.empty((T, k), np.int32)
    wo = np.empty((T, k), np.float32)
    dropped = np.zeros(1, np.int32)
    _check(_load().orc_capacity_fallback(T, E, k, int(cap), int(fallback_min), _p(idx), _p(w),
                                         _p(io), _p(wo), _p(dropped)), "capacity_fallback")
    return io, wo, int(dropped[0])


def forward_routed(inp: dict, cfg, idx: np.ndarray, w: np.ndarray, tokens=None,
                   round_h: bool = False, w4: dict | None = None) -> np.ndarray:
    """Block output of the listed tokens for a given routing: idx [n,k]
    (-1 = no expert in that slot) and weights w [n,k]: out[t] = sum over the
    slots with an expert of w * MLP_e(x_t), with the 4-bit experts when w4 is
    given (dequantised element by element). Returns float64 [n,H]."""
    x = _c(inp["x"])
    T = x.shape[0]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = _c(tokens, np.int32)
    idx = _c(idx, np.int32)
    n, k = idx.shape
    live = idx >= 0
    tok = np.repeat(tokens, k).reshape(n, k)[live]
    y = np.zeros((n * k, x.shape[1]), np.float64)
    if live.any() and w4 is not None:
        y[live.ravel()] = expert_rows_w4(x, w4, tok, idx[live], round_h=round_h)
    elif live.any():
        y[live.ravel()] = expert_rows(x, inp["w_gate"], inp["w_up"], inp["w_down"], tok,
                                      idx[live], round_h=round_h)
    return combine(np.asarray(w, np.float64), y, keep=live.astype(np.int8))


def expert_rows(x, w_gate, w_up, w_down, tok, ex, round_h: bool = False) -> np.ndarray:
    """SwiGLU expert output (float64 [n,H]) for rows (token tok[r], expert ex[r])."""
    x, w_gate, w_up, w_down = _c(x), _c(w_gate), _c(w_up), _c(w_down)
    tok, ex = _c(tok, np.int32), _c(ex, np.int32)
    H = x.shape[1]
    E, I, H2 = w_gate.shape
    assert H2 == H and w_up.shape == (E, I, H) and w_down.shape == (E, H, I)
    assert len({a.dtype for a in (x, w_gate, w_up, w_down)}) == 1
    n = tok.shape[0]
    y = np.empty((n, H), np.float64)
    _check(_load().orc_expert_rows(H, I, _dtype_code(x), _p(x), _p(w_gate), _p(w_up),
                                   _p(w_down), n, _p(tok), _p(ex), int(round_h), _p(y)),
           "expert_rows")
    return y


def combine(w: np.ndarray, y_pair: np.ndarray, keep: np.ndarray | None = None) -> np.ndarray:
    """out[t] = sum_j w[t,j] * y_pair[t*k+j] over the kept slots (float64)."""
    w = _c(w, np.float64)
    y_pair = _c(y_pair, np.float64)
    T, k = w.shape
    H = y_pair.shape[1]
    out = np.empty((T, H), np.float64)
    if keep is None:
        _check(_load().orc_combine(T, H, k, _p(w), _p(y_pair), _p(out)), "combine")
    else:
        keep = _c(keep, np.int8)
        _check(_load().orc_combine_kept(T, H, k, _p(w), _p(y_pair), _p(keep), _p(out)),
               "combine")
    return out


def aux(counts: np.ndarray, probs: np.ndarray, k: int):
    """Returns (f [E], P [E], aux) in float64."""
    counts = _c(counts, np.int32)
    probs = _c(probs, np.float64)
    T, E = probs.shape
    f = np.empty(E, np.float64)
    P = np.empty(E, np.float64)
    a = np.empty(1, np.float64)
    _check(_load().orc_aux(T, E, k, _p(counts), _p(probs), _p(f), _p(P), _p(a)), "aux")
    return f, P, float(a[0])


def forward_tokens(inp: dict, cfg, tokens=None, forced_idx=None, round_h: bool = False,
                   keep=None):
    """Block forward for the listed tokens (all when None); keep [n,k] (None:
    all kept) marks the slots a capacity limit kept.

    inp: dict with x, w_router, w_gate, w_up, w_down, logit_bias (None or
    float32 [E]); cfg: an object with T, H, E, k, I, norm.
    Returns dict(logits fp32 [n,E], idx [n,k], w [n,k] f64, out [n,H] f64)."""
    x = _c(inp["x"])
    wr, wg, wu, wd = (_c(inp[n]) for n in ("w_router", "w_gate", "w_up", "w_down"))
    bias = _c(inp.get("logit_bias"), np.float32)
    T, H = x.shape
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = _c(tokens, np.int32)
    n = tokens.shape[0]
    forced_idx = _c(forced_idx, np.int32)
    keep = _c(keep, np.int8)
    k = cfg.k
    lg = np.empty((n, cfg.E), np.float32)
    idx = np.empty((n, k), np.int32)
    w = np.empty((n, k), np.float64)
    out = np.empty((n, H), np.float64)
    _check(_load().orc_forward_tokens(T, H, cfg.E, k, cfg.I, int(bool(cfg.norm)),
                                      _dtype_code(x), _p(x), _p(wr), _p(bias), _p(wg), _p(wu),
                                      _p(wd), n, _p(tokens), _p(forced_idx), _p(keep),
                                      int(round_h),
                                      _p(lg), _p(idx), _p(w), _p(out)), "forward_tokens")
    return {"logits": lg, "idx": idx, "w": w, "out": out}


def forward_variant(inp: dict, cfg, tokens=None, noise=None, w_noise=None, sel_bias=None,
                    keep=None, round_h: bool = False, k_min: int = 0, forced_idx=None):
    """Block forward of the listed tokens with the router variants, composed
    from the steps above: logits (+ bias), noisy logits if `noise` [T,E] and
    `w_noise` [E,H] are given (the noise rows of the listed tokens are used),
    selection with the optional selection-only bias, experts, combine over
    the kept slots. forced_idx [n,k] (optional) replaces the selection (with
    k_min: negative ids are the empty slots). Returns dict(logits (the ones
    the softmax saw), idx, w, out)."""
    x = _c(inp["x"])
    T = x.shape[0]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = _c(tokens, np.int32)
    xs = np.ascontiguousarray(x[tokens])
    lg = logits(xs, inp["w_router"], inp.get("logit_bias"))
    if noise is not None:
        nlg = logits(xs, w_noise)
        lg = noisy_logits(lg, nlg, np.asarray(noise, np.float32)[tokens])
    kt = None
    if forced_idx is not None:
        idx, w, _ = route(lg, cfg.k, cfg.norm, forced_idx=forced_idx)
        live = idx >= 0
        keep = live if keep is None else (np.asarray(keep, bool) & live)
        kt = live.sum(1).astype(np.int32)
    elif k_min:  # entropy-driven k (no selection bias with it)
        assert sel_bias is None
        idx, w, kt, _ = route_dynamic(lg, cfg.k, k_min, cfg.norm)
        live = idx >= 0
        keep = live if keep is None else (np.asarray(keep, bool) & live)
    else:
        idx, w, _ = route(lg, cfg.k, cfg.norm, sel_bias=sel_bias)
    n = tokens.shape[0]
    tok = np.repeat(np.arange(n, dtype=np.int32), cfg.k)
    ex = np.where(idx >= 0, idx, 0).ravel().astype(np.int32)  # empty slots: any row, not kept
    y = expert_rows(xs, inp["w_gate"], inp["w_up"], inp["w_down"], tok, ex, round_h=round_h)
    out = combine(w, y, keep)
    return {"logits": lg, "idx": idx, "w": w, "out": out, "kt": kt}


def dequant_w4(codes: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """codes uint8 [E,N/32,K/64,32,32], sb uint16 (bf16 bits) [E,N/32,K/128,32,2]
    (the tiled layout of moe.h) -> float64 [E,N,K]."""
    codes = _c(codes, np.uint8)
    sb = _c(sb, np.uint16)
    E, NB, KC, r32, b32 = codes.shape
    assert (r32, b32) == (32, 32)
    N, K = 32 * NB, 64 * KC
    assert sb.shape == (E, NB, K // 128, 32, 2)
    w = np.empty((E, N, K), np.float64)
    _check(_load().orc_dequant_w4(E, N, K, _p(codes), _p(sb), _p(w)), "dequant_w4")
    return w


def expert_rows_w4(x, w4: dict, tok, ex, round_h: bool = False) -> np.ndarray:
    """SwiGLU expert output (float64 [n,H]) with 4-bit weights w4 = dict of
    gate/up/down codes and gate_sb/up_sb/down_sb."""
    x = _c(x)
    tok, ex = _c(tok, np.int32), _c(ex, np.int32)
    H = x.shape[1]
    E, I = w4["gate"].shape[0], 32 * w4["gate"].shape[1]
    arrs = [_c(w4[n], np.uint8 if "sb" not in n else np.uint16)
            for n in ("gate", "gate_sb", "up", "up_sb", "down", "down_sb")]
    n = tok.shape[0]
    y = np.empty((n, H), np.float64)
    _check(_load().orc_expert_rows_w4(H, I, _dtype_code(x), _p(x), *(_p(a) for a in arrs), n,
                                      _p(tok), _p(ex), int(round_h), _p(y)), "expert_rows_w4")
    return y


def expert_rows_f64w(x, wg, wu, wd, tok, ex) -> np.ndarray:
    """SwiGLU expert output with float64 weight arrays (dequantised-first check)."""
    x = _c(x)
    wg, wu, wd = (_c(a, np.float64) for a in (wg, wu, wd))
    tok, ex = _c(tok, np.int32), _c(ex, np.int32)
    H = x.shape[1]
    I = wg.shape[1]
    n = tok.shape[0]
    y = np.empty((n, H), np.float64)
    _check(_load().orc_expert_rows_f64w(H, I, _dtype_code(x), _p(x), _p(wg), _p(wu), _p(wd), n,
                                        _p(tok), _p(ex), _p(y)), "expert_rows_f64w")
    return y


def forward_w4(inp: dict, w4: dict, cfg, tokens=None, round_h: bool = False, keep=None,
               forced_idx=None):
    """Block forward of the listed tokens with 4-bit expert weights (router as
    forward_variant, experts dequantised element by element); forced_idx
    [n,k] (optional) replaces the selection."""
    x = _c(inp["x"])
    T = x.shape[0]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = _c(tokens, np.int32)
    xs = np.ascontiguousarray(x[tokens])
    lg = logits(xs, inp["w_router"], inp.get("logit_bias"))
    idx, w, _ = route(lg, cfg.k, cfg.norm, forced_idx=forced_idx)
    n = tokens.shape[0]
    tok = np.repeat(np.arange(n, dtype=np.int32), cfg.k)
    y = expert_rows_w4(xs, w4, tok, idx.ravel(), round_h=round_h)
    out = combine(w, y, keep)
    return {"logits": lg, "idx": idx, "w": w, "out": out}

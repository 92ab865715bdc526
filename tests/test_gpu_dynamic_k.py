"""GPU parity of entropy-driven dynamic k (each token keeps k_t in
[k_min, k] experts; the other slots are empty) against the CPU oracle: the
router on given logits, the dispatch with empty slots, and the whole block.
k_t is an integer decided by floating point: the GPU and the oracle may
differ only where the oracle's unfloored k_min + (k - k_min) H / ln E lies
within KT_GAP of an integer. All calls go through the C ABI."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_40_amd import binding
from sparse_mixture_experts_40_amd.configs import MoEConfig, WORKLOADS
from sparse_mixture_experts_40_amd.inputs import make_inputs, make_router_variant_inputs

from gpu_common import check_output, check_selection_row, dev, host, sample_tokens

pytestmark = pytest.mark.gpu

KT_GAP = 1e-4


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _kt_ok(g_kt, o_kt, x):
    """Tokens whose k_t agrees; a disagreement must sit on an integer boundary."""
    diff = g_kt != o_kt
    near = np.abs(x - np.round(x)) < KT_GAP
    assert not (diff & ~near).any(), np.flatnonzero(diff & ~near)[:10]
    assert (np.abs(g_kt - o_kt) <= 1).all()
    return ~diff


@pytest.mark.parametrize("T,E,k,k_min", [(64, 8, 4, 2), (300, 64, 8, 4), (257, 128, 8, 4),
                                         (130, 256, 16, 4), (77, 40, 3, 1), (33, 16, 8, 8)])
@pytest.mark.parametrize("norm", [True, False])
def test_dynamic_k_router_on_oracle_logits(orc, T, E, k, k_min, norm):
    rng = np.random.default_rng(T + 3 * E + k)
    scale = rng.choice([0.2, 0.7, 1.5, 3.0, 10.0], size=(T, 1))  # flat to peaked rows
    lg = (rng.standard_normal((T, E)) * scale).astype(np.float32)
    idx_ref, w_ref, kt_ref, x = orc.route_dynamic(lg, k, k_min, norm)
    cfg = MoEConfig("t", T=T, H=64, E=E, k=k, I=64, norm=norm, dtype="bf16")
    c = binding.make_config(cfg)
    g_kt = torch.full((T,), -5, dtype=torch.int32, device="cuda")
    opts = binding.options(dynamic_k_min=k_min, k_per_token=g_kt)
    g_idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    g_w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    binding.router_topk_ex(c, opts, None, None, None, _f32(lg), g_idx, g_w)
    torch.cuda.synchronize()
    same = _kt_ok(host(g_kt), kt_ref, x)
    if k_min == k:
        assert same.all()
    assert len(np.unique(kt_ref)) > 1 or k_min == k  # the case spans several k
    assert (host(g_idx)[same] == idx_ref[same]).all()
    np.testing.assert_allclose(host(g_w)[same], w_ref[same], rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("T,E,k", [(64, 8, 4), (1000, 64, 8), (16384, 128, 8), (3, 200, 7)])
def test_dispatch_with_empty_slots_bitexact(orc, T, E, k):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    kt = rng.integers(1, k + 1, T)
    for t in range(T):
        idx[t, kt[t]:] = -1
    counts, offsets, sp, pp = orc.dispatch(idx, E)
    cfg = MoEConfig("t", T=T, H=64, E=E, k=k, I=64, norm=True, dtype="bf16")
    c = binding.make_config(cfg)
    ws = binding.alloc_workspace(c)
    g = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1)]
    g_sp = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    g_pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    binding.dispatch(c, _i32(idx), g[0], g[1], g_sp, g_pp, ws)
    torch.cuda.synchronize()
    assert (host(g[0]) == counts).all() and (host(g[1]) == offsets).all()
    n = offsets[E]
    assert (host(g_sp)[:n] == sp[:n]).all() and (host(g_sp)[n:] == -7).all()
    assert (host(g_pp) == pp).all()


def check_dynamic_block(orc, cfg, inp, k_min, tokens, cap=0):
    blk = binding.MoEBlock(cfg, inp, capacity=cap, dynamic_k_min=k_min)
    blk.forward(dev(inp["x"]))
    torch.cuda.synchronize()
    lg = orc.logits(inp["x"], inp["w_router"], inp.get("logit_bias"))
    o_idx, o_w, o_kt, x = orc.route_dynamic(lg, cfg.k, k_min, cfg.norm)
    g_idx, g_kt = host(blk.topk_idx), host(blk.k_per_token)
    same_kt = _kt_ok(g_kt, o_kt, x)
    # selections of tokens with the same k_t: equal sets except on near ties
    for t in np.flatnonzero(same_kt & (g_idx != o_idx).any(1)):
        check_selection_row(lg[t], g_idx[t][: o_kt[t]], o_idx[t][: o_kt[t]], int(o_kt[t]), t)
    # a token whose k_t differs (on an integer boundary) keeps the first g_kt
    # experts of the oracle's full order, with the same near-tie rule
    full_idx, _, _ = orc.route(lg, cfg.k, cfg.norm)
    for t in np.flatnonzero(~same_kt):
        kt = int(g_kt[t])
        assert (g_idx[t][kt:] == -1).all()
        check_selection_row(lg[t], g_idx[t][:kt], full_idx[t][:kt], kt, t)
    ok = same_kt & (g_idx == o_idx).all(1)
    live = g_idx >= 0
    counts = host(blk.counts)
    assert (counts == np.bincount(g_idx[live], minlength=cfg.E)).all()
    assert counts.sum() == g_kt.sum()
    np.testing.assert_allclose(host(blk.f), counts / counts.sum(), rtol=1e-6)
    keep = live.copy()
    if cap:
        _, _, _, pp, dropped = orc.dispatch_capacity(o_idx, cfg.E, cap)
        if ok.all():
            assert int(host(blk.dropped)[0]) == dropped
        # the keep mask the GPU's own selection implies (the oracle's own
        # wherever the selections agree)
        _, _, _, gpp, g_dropped = orc.dispatch_capacity(g_idx, cfg.E, cap)
        assert int(host(blk.dropped)[0]) == g_dropped
        keep = (gpp >= 0).reshape(g_idx.shape)
    # the k_t and near-tie differences checked above are the only allowed
    # ones: every listed token is compared with the oracle run on the GPU's
    # selection (its empty slots included)
    r = orc.forward_variant(inp, cfg, tokens=tokens, forced_idx=g_idx[tokens], keep=keep[tokens])
    np.testing.assert_allclose(host(blk.topk_w)[tokens], r["w"], rtol=0, atol=1e-5)
    mx, rm = check_output(host(blk.out)[tokens], r["out"], cfg.dtype)
    print(f"{cfg.name} k_min={k_min} cap={cap}: k_t histogram "
          f"{np.bincount(g_kt, minlength=cfg.k + 1)[k_min:].tolist()}, k_t differences "
          f"{int((~same_kt).sum())}, near ties {int((same_kt & ~ok).sum())}, compared "
          f"{len(tokens)} tokens, max|d|/RMS {mx:.4f}", flush=True)
    return blk


DYN_E2E = [
    (WORKLOADS["tiny_f32"], 1),
    (MoEConfig("e128_like", T=1500, H=512, E=128, k=8, I=192, norm=True, dtype="bf16"), 4),
    (MoEConfig("decode_like", T=64, H=512, E=128, k=8, I=256, norm=True, dtype="bf16",
               zipf_s=1.2), 4),
    (MoEConfig("mixtral_like", T=700, H=512, E=8, k=2, I=1024, norm=False, dtype="bf16"), 1),
    (MoEConfig("odd_sizes", T=41, H=192, E=40, k=3, I=320, norm=True, dtype="bf16"), 1),
    (MoEConfig("peaked", T=400, H=256, E=64, k=8, I=128, norm=True, dtype="bf16", zipf_s=2.0), 4),
]


@pytest.mark.parametrize("cfg,k_min", DYN_E2E, ids=lambda v: getattr(v, "name", str(v)))
def test_layer_forward_dynamic_k(orc, cfg, k_min):
    inp = make_inputs(cfg, seed=0)
    check_dynamic_block(orc, cfg, inp, k_min, np.arange(cfg.T, dtype=np.int32))


def test_dynamic_k_with_capacity(orc):
    cfg = MoEConfig("dyn_cap", T=600, H=256, E=32, k=8, I=128, norm=True, dtype="bf16",
                    zipf_s=1.0)
    inp = make_inputs(cfg, seed=9)
    cap = orc.capacity(cfg.T, cfg.E, cfg.k, 0.5)
    check_dynamic_block(orc, cfg, inp, 4, np.arange(cfg.T, dtype=np.int32), cap=cap)


def test_dynamic_k_rejects_select_bias():
    cfg = MoEConfig("rej", T=16, H=64, E=8, k=4, I=64, norm=True, dtype="bf16")
    inp = make_inputs(cfg, seed=1)
    var = make_router_variant_inputs(cfg, seed=1)
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        binding.MoEBlock(cfg, inp, select_bias=var["select_bias"],
                         dynamic_k_min=2).forward(dev(inp["x"]))


def test_full_size_dynamic_k(orc):
    cfg = WORKLOADS["prefill128_bf16"]
    print("[prefill128_bf16 dynamic k] generating inputs", flush=True)
    inp = make_inputs(cfg)
    check_dynamic_block(orc, cfg, inp, 4, sample_tokens(cfg.T, 24, seed=9))

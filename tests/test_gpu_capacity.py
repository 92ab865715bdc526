"""GPU parity of the capacity-limited dispatch (each expert keeps its first C
pairs in pair order; dropped slots add nothing) and of the block run with a
capacity, against the CPU oracle. All calls go through the C ABI."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_40_amd import binding
from sparse_mixture_experts_40_amd.configs import MoEConfig, WORKLOADS
from sparse_mixture_experts_40_amd.inputs import make_inputs

from gpu_common import check_output, check_selection_row, dev, host, sample_tokens

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _skewed_idx(rng, T, E, k, s=1.1):
    """Distinct experts per token, skewed toward low ids (loads above the mean)."""
    p = 1.0 / np.arange(1, E + 1) ** s
    p /= p.sum()
    return np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _gpu_dispatch_capacity(cfg, idx, cap):
    c = binding.make_config(cfg)
    ws = binding.alloc_workspace(c)
    T, E, k = cfg.T, cfg.E, cfg.k
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    dropped = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    binding.dispatch_capacity(c, _i32(idx), cap, counts, offsets, sp, pp, ws, dropped)
    torch.cuda.synchronize()
    return host(counts), host(offsets), host(sp), host(pp), int(host(dropped)[0])


@pytest.mark.parametrize("T,E,k,cf", [(1, 1, 1, 1.0), (64, 8, 2, 1.0), (1000, 64, 8, 1.0),
                                      (1031, 256, 16, 1.25), (4096, 8, 2, 1.0),
                                      (16384, 128, 8, 1.0), (3, 200, 7, 1.0), (500, 16, 4, 0.25),
                                      (2049, 32, 4, 0.5)])
def test_dispatch_capacity_bitexact(orc, T, E, k, cf):
    rng = np.random.default_rng(T * 7 + E + k)
    idx = _skewed_idx(rng, T, E, k)
    cfg = MoEConfig("t", T=T, H=64, E=E, k=k, I=64, norm=True, dtype="bf16")
    cap = orc.capacity(T, E, k, cf)
    assert binding.capacity(binding.make_config(cfg), cf) == cap
    for cp in sorted({cap, 1, T * k}):
        counts, offsets, sp, pp, dropped = orc.dispatch_capacity(idx, E, cp)
        g_counts, g_off, g_sp, g_pp, g_drop = _gpu_dispatch_capacity(cfg, idx, cp)
        assert (g_counts == counts).all(), ("counts", cp)
        assert (g_off == offsets).all(), ("offsets", cp)
        n = offsets[E]
        assert (g_sp[:n] == sp[:n]).all(), ("sorted_pair", cp)
        assert (g_sp[n:] == -7).all(), ("entries past the kept pairs are not written", cp)
        assert (g_pp == pp).all(), ("pair_pos", cp)
        assert g_drop == dropped, ("dropped", cp)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_combine_skips_dropped_slots(orc, dtype):
    rng = np.random.default_rng(31)
    T, k, H = 300, 4, 192
    P = T * k
    y = rng.standard_normal((P, H)).astype(np.float32)  # y_sorted rows
    perm = rng.permutation(P).astype(np.int32)
    keep = rng.random(P) < 0.7
    keep[:k] = False  # token 0: every slot dropped -> zeros
    pair_pos = np.where(keep, perm, -1).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    y_pair = np.zeros((P, H), np.float64)
    y_pair[keep] = y[perm[keep]]
    ref = orc.combine(w.astype(np.float64), y_pair, keep.reshape(T, k))
    cfg = MoEConfig("t", T=T, H=H, E=8, k=k, I=64, norm=True, dtype=dtype)
    c = binding.make_config(cfg)
    out = torch.empty(T, H, dtype=binding.TORCH_DTYPE[dtype], device="cuda")
    binding.combine(c, torch.from_numpy(y).cuda(), _i32(pair_pos), torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    got = host(out)
    assert (got[0] == 0.0).all()
    if dtype == "f32":
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5)
    else:  # one rounding of an fp32 sum: at most half a bf16 ulp (+ fp32 sum error)
        assert (np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5).all()


def _oracle_capacity_keep(orc, cfg, inp, cap):
    """Oracle selection of every token and its capacity keep mask [T,k]."""
    lg = orc.logits(inp["x"], inp["w_router"], inp.get("logit_bias"))
    idx, _, _ = orc.route(lg, cfg.k, cfg.norm)
    _, _, _, pp, dropped = orc.dispatch_capacity(idx, cfg.E, cap)
    return lg, idx, (pp >= 0).reshape(cfg.T, cfg.k), dropped


def _keep_from_selection(idx, E, cap):
    """Keep mask implied by a selection: pair p is kept iff fewer than `cap`
    earlier pairs chose the same expert (a property of any valid result)."""
    flat = idx.ravel()
    rank = np.empty(flat.size, np.int64)
    for e in range(E):
        where = np.flatnonzero(flat == e)
        rank[where] = np.arange(where.size)
    return (rank < cap).reshape(idx.shape)


def check_capacity_block(orc, cfg, inp, cf, tokens):
    cap = orc.capacity(cfg.T, cfg.E, cfg.k, cf)
    blk = binding.MoEBlock(cfg, inp, capacity=cap)
    blk.forward(dev(inp["x"]))
    torch.cuda.synchronize()
    lg, o_idx, o_keep, o_drop = _oracle_capacity_keep(orc, cfg, inp, cap)
    g_idx = host(blk.topk_idx)
    g_keep = _keep_from_selection(g_idx, cfg.E, cap)
    g_drop = int(host(blk.dropped)[0])
    assert g_drop == int((~g_keep).sum())  # the GPU's count matches its own selection
    assert (host(blk.counts) == np.bincount(g_idx.ravel(), minlength=cfg.E)).all()
    mism = np.flatnonzero((g_idx != o_idx).any(1))
    for t in mism:  # only near ties may differ
        check_selection_row(lg[t], g_idx[t], o_idx[t], cfg.k, t)
    keep_diff = int((g_keep != o_keep).sum())
    # a changed selection moves at most one capacity boundary per expert involved
    assert keep_diff <= 2 * cfg.k * len(mism), (keep_diff, len(mism))
    if len(mism) == 0:
        assert keep_diff == 0 and g_drop == o_drop
    # every listed token against the oracle run with the GPU's selection and
    # the keep mask that selection implies (the oracle's own, wherever the
    # selections agree and no earlier near tie moved a capacity boundary)
    r = orc.forward_tokens(inp, cfg, tokens=tokens, forced_idx=g_idx[tokens],
                           keep=g_keep[tokens])
    np.testing.assert_allclose(host(blk.topk_w)[tokens], r["w"], rtol=0, atol=1e-5)
    mx, rm = check_output(host(blk.out)[tokens], r["out"], cfg.dtype)
    print(f"{cfg.name} cf={cf} cap={cap}: dropped {g_drop}/{cfg.T * cfg.k}, selection "
          f"mismatches {len(mism)}, keep differences {keep_diff}, compared {len(tokens)} "
          f"tokens, max|d|/RMS {mx:.4f}", flush=True)
    return g_drop


CAP_E2E = [
    (MoEConfig("e128_like", T=2500, H=512, E=128, k=8, I=192, norm=True, dtype="bf16"), 1.0),
    (MoEConfig("mixtral_like", T=700, H=512, E=8, k=2, I=1024, norm=False, dtype="bf16"), 1.0),
    (MoEConfig("decode_like", T=64, H=512, E=128, k=8, I=256, norm=True, dtype="bf16",
               zipf_s=1.2), 1.25),
    (WORKLOADS["tiny_f32"], 1.0),
    (MoEConfig("odd_sizes", T=41, H=192, E=40, k=3, I=320, norm=False, dtype="bf16"), 0.5),
    (MoEConfig("skewed_tight", T=300, H=256, E=16, k=4, I=128, norm=True, dtype="bf16",
               zipf_s=1.5), 0.5),
]


@pytest.mark.parametrize("cfg,cf", CAP_E2E, ids=lambda v: getattr(v, "name", str(v)))
def test_layer_forward_capacity_matches_oracle(orc, cfg, cf):
    inp = make_inputs(cfg, seed=0)
    dropped = check_capacity_block(orc, cfg, inp, cf, np.arange(cfg.T, dtype=np.int32))
    if cf < 1.25 or cfg.zipf_s > 0:
        assert dropped > 0  # the case exercises dropping


def test_capacity_large_enough_equals_dropless(orc):
    cfg = MoEConfig("loose", T=500, H=256, E=32, k=4, I=128, norm=True, dtype="bf16")
    inp = make_inputs(cfg, seed=2)
    x = dev(inp["x"])
    plain = binding.MoEBlock(cfg, inp)
    capped = binding.MoEBlock(cfg, inp, capacity=cfg.T * cfg.k)
    plain.forward(x)
    capped.forward(x)
    torch.cuda.synchronize()
    assert int(host(capped.dropped)[0]) == 0
    assert torch.equal(plain.out.view(torch.int16), capped.out.view(torch.int16))


@pytest.mark.parametrize("name,cf", [("prefill128_bf16", 1.0), ("decode128_bf16", 1.25)])
def test_full_size_capacity(orc, name, cf):
    cfg = WORKLOADS[name]
    print(f"[{name}] generating inputs", flush=True)
    inp = make_inputs(cfg)
    dropped = check_capacity_block(orc, cfg, inp, cf, sample_tokens(cfg.T, 32, seed=4))
    assert dropped > 0

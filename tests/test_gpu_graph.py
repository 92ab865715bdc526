"""The layer forward captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay bitwise equal to the eager call, with eager work (the
outputs cleared by fill kernels) and a synchronisation between replays, and
again after new input values are copied into the captured input buffer. The
library only launches kernels on the caller's stream (no allocation, no
synchronisation, no memset), so the whole forward can be captured. All calls
go through the C ABI."""
import pytest
import torch

from sparse_mixture_experts_40_amd import binding
from sparse_mixture_experts_40_amd.configs import MoEConfig, WORKLOADS
from sparse_mixture_experts_40_amd.inputs import (make_inputs, make_router_variant_inputs,
                                                  make_w4_inputs)

from gpu_common import dev

pytestmark = pytest.mark.gpu

DECODE = MoEConfig("decode_like", T=64, H=512, E=128, k=8, I=256, norm=True, dtype="bf16",
                   zipf_s=1.2)
CASES = {
    "decode_like": (DECODE, {}),
    "tiled": (MoEConfig("tiled", T=1500, H=512, E=32, k=4, I=512, norm=True, dtype="bf16"), {}),
    "f32": (WORKLOADS["tiny_f32"], {}),
    "capacity_fallback": (DECODE, {"capacity": 4, "fallback_min": 4}),
    "dynamic_k": (MoEConfig("dyn", T=300, H=256, E=32, k=8, I=128, norm=True, dtype="bf16"),
                  {"dynamic_k_min": 4}),
    "w4": (MoEConfig("w4", T=64, H=512, E=16, k=4, I=512, norm=True, dtype="bf16"), {"w4": 1}),
    "capacity": (MoEConfig("cap", T=1500, H=512, E=32, k=4, I=512, norm=True, dtype="bf16",
                           zipf_s=1.0), {"capacity": 120}),
    "noise+bias": (MoEConfig("var", T=700, H=512, E=8, k=2, I=1024, norm=False, dtype="bf16"),
                   {"variant": 1}),
}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _outputs(blk):
    """Every output the forward writes: the block output, the routing, the
    statistics, the z-loss, the drop count (written with a capacity) and the
    per-token k (written with dynamic k)."""
    outs = [blk.out, blk.topk_idx, blk.topk_w, blk.counts, blk.f, blk.P, blk.aux, blk.logits,
            blk.z_loss, blk.dropped]
    if blk.opts is not None and blk.opts.dynamic_k_min:
        outs.append(blk.k_per_token)
    return outs


def _snapshot(blk):
    return [t.clone() for t in _outputs(blk)]


def _same(a, b):
    return all(torch.equal(_bits(x), _bits(y)) for x, y in zip(a, b))


def _capture(fn):
    """fn once eagerly on a side stream (first calls set up cached device
    attributes), then captured into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("case", list(CASES))
def test_layer_forward_graph_replays_match_eager(case):
    cfg, kw = CASES[case]
    kw = dict(kw)
    inp = make_inputs(cfg, seed=1, weights="w4" not in kw)
    if "w4" in kw:
        kw = {**kw, "w4": make_w4_inputs(cfg, seed=1)}
    if kw.pop("variant", 0):
        var = make_router_variant_inputs(cfg, seed=1)
        kw = {**kw, "noise": var["noise"], "w_noise": var["w_noise"],
              "select_bias": var["select_bias"]}
    blk = binding.MoEBlock(cfg, inp, **kw)
    x = dev(inp["x"])
    blk.forward(x)
    torch.cuda.synchronize()
    ref = _snapshot(blk)
    g = _capture(lambda: blk.forward(x))
    for r in range(4):
        for t in _outputs(blk):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(_snapshot(blk), ref), (case, "replay", r)
    # new values in the captured input buffer: replay against an eager call
    x.copy_(dev(make_inputs(cfg, seed=2, weights=False)["x"]))
    g.replay()
    torch.cuda.synchronize()
    got = _snapshot(blk)
    assert not torch.equal(_bits(got[0]), _bits(ref[0]))
    blk.forward(x)
    torch.cuda.synchronize()
    assert _same(_snapshot(blk), got), (case, "new input")


def test_noalloc_forward_graph_replays_match_eager():
    """moe_layer_forward_noalloc, the entry point for callers that cannot
    allocate, under capture: its scratch is the library's array, looked up on
    the first call (before capture)."""
    cfg = DECODE
    inp = make_inputs(cfg, seed=3)
    c = binding.make_config(cfg)
    ws_free = binding.MoEBlock(cfg, inp)
    x = dev(inp["x"])
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")

    def fwd():
        binding.layer_forward_noalloc(c, x, ws_free.w_router, ws_free.logit_bias, ws_free.w_gate,
                                      ws_free.w_up, ws_free.w_down, out, topk_idx=idx)

    fwd()
    torch.cuda.synchronize()
    ref = (out.clone(), idx.clone())
    g = _capture(fwd)
    for r in range(3):
        out.zero_()
        idx.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), r
        assert torch.equal(idx, ref[1]), r
    # the workspace entry point gives the same block output
    ws_free.forward(x)
    torch.cuda.synchronize()
    assert torch.equal(ws_free.out.view(torch.int16), ref[0].view(torch.int16))

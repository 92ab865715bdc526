"""The bf16 layer forward at decode sizes, where the weight-streaming gate/up
kernel sorts the routing pairs in its own LDS instead of a dispatch launch,
against the same block run as separate C-ABI calls on the layer's own
routing: dispatch (with the capacity when one is set), the expert MLP, the
combine and the statistics. The sort is integer work and the expert kernels
are the same, so the block output, the counts, f and the dropped count must be
bitwise equal; P and aux come from the router's probability sums in the
layer and from the logits in moe_aux_stats (two fp32 softmaxes), so they are
compared to 2e-6 relative. Batches past one dispatch chunk (P > 2048 pairs)
take the dispatch launch and are checked the same way."""
import numpy as np
import pytest
import torch

from sparse_mixture_experts_40_amd import binding
from sparse_mixture_experts_40_amd.configs import MoEConfig
from sparse_mixture_experts_40_amd.inputs import make_inputs

from gpu_common import dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _run(T, E, k, cf=0.0, k_min=0, stats=True, zipf=0.0, H=512, I=256):
    cfg = MoEConfig(f"sort_{T}_{E}_{k}", T=T, H=H, E=E, k=k, I=I, norm=True, dtype="bf16",
                    zipf_s=zipf, seed=T + E + k)
    assert cfg.P <= 16 * E, "decode-sized batch (weight-streaming kernels)"
    inp = make_inputs(cfg)
    c = binding.make_config(cfg)
    x, wr, wg, wu, wd = (dev(inp[n]) for n in ("x", "w_router", "w_gate", "w_up", "w_down"))
    lb = dev(inp["logit_bias"]) if inp["logit_bias"] is not None else None
    cap = binding.capacity(c, cf) if cf > 0 else 0
    dropped = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    kt = torch.empty(T, dtype=torch.int32, device="cuda")
    opts = binding.options(capacity=cap, dropped=dropped if cap else None, dynamic_k_min=k_min,
                           k_per_token=kt if k_min else None)
    ws = binding.alloc_workspace(c)
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    f = torch.empty(E, dtype=torch.float32, device="cuda")
    P = torch.empty(E, dtype=torch.float32, device="cuda")
    aux = torch.empty(1, dtype=torch.float32, device="cuda")
    st = dict(counts=counts, f=f, P=P, aux=aux) if stats else {}
    binding.layer_forward_ex(c, opts, x, wr, lb, wg, wu, wd, out, ws, router_logits=logits,
                             topk_idx=idx, topk_w=w, **st)

    # the same block as separate calls on the layer's routing
    ws2 = binding.alloc_workspace(c)
    counts2 = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    dropped2 = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    if cap:
        binding.dispatch_capacity(c, idx, cap, counts2, offsets, sp, pp, ws2, dropped2)
    else:
        binding.dispatch(c, idx, counts2, offsets, sp, pp, ws2)
    y = torch.empty(T * k, H, dtype=torch.float32, device="cuda")
    binding.expert_swiglu(c, x, sp, offsets, wg, wu, wd, y, ws2)
    out2 = torch.empty_like(out)
    binding.combine(c, y, pp, w, out2)
    f2 = torch.empty_like(f)
    P2 = torch.empty_like(P)
    aux2 = torch.empty_like(aux)
    binding.aux_stats(c, logits, idx, ws2, counts=None, f=f2, P=P2, aux=aux2)
    torch.cuda.synchronize()

    assert torch.equal(_bits(out), _bits(out2)), "block output"
    if cap:
        assert int(dropped.item()) == int(dropped2.item()) >= 0
    if stats:
        assert torch.equal(counts, counts2)
        assert torch.equal(f, f2)
        np.testing.assert_allclose(P.cpu().numpy(), P2.cpu().numpy(), rtol=2e-6, atol=1e-9)
        np.testing.assert_allclose(aux.cpu().numpy(), aux2.cpu().numpy(), rtol=2e-6)
    return int(dropped.item()) if cap else 0, int((idx < 0).sum().item())


@pytest.mark.parametrize("T,E,k", [(64, 128, 8), (33, 16, 4), (256, 128, 8), (256, 256, 8),
                                   (5, 8, 2), (1, 64, 8)])
def test_layer_sorting_gate_up_equals_dispatch_chain(T, E, k):
    _run(T, E, k)


def test_layer_sorting_gate_up_skewed_loads():
    # a Zipf logit bias: hot experts with several token blocks, many untouched
    _run(64, 128, 8, zipf=1.2)


def test_layer_sorting_gate_up_without_statistics():
    _run(64, 128, 8, stats=False)


def test_layer_sorting_gate_up_capacity():
    dropped, _ = _run(64, 128, 8, cf=1.0, zipf=1.2)
    assert dropped > 0, "the capacity drops pairs here"


def test_layer_sorting_gate_up_dynamic_k_empty_slots():
    _, empty = _run(100, 64, 6, k_min=2)
    assert empty > 0, "dynamic k leaves empty slots here"


def test_layer_multi_chunk_decode_batch_takes_dispatch_launch():
    # P = 2056 > 2048 pairs per chunk (and <= 16 E): the dispatch launch
    _run(257, 256, 8)

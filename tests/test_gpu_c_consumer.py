"""The C ABI from a plain C program: tests/c_consumer/moe_c_example.c (gcc, C11,
no Python or torch in its process; hipMalloc'd buffers and workspace, the null
stream) runs moe_layer_forward on seeded inputs written to a file. Its outputs
must equal, bit for bit, those of the same forward called through the Python
binding in this process, and its block output meets the oracle's tolerance on
sampled tokens. The example is compiled here with gcc (a second or less)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from sparse_mixture_experts_40_amd import binding
from sparse_mixture_experts_40_amd.configs import MoEConfig, WORKLOADS
from sparse_mixture_experts_40_amd.inputs import make_inputs

from gpu_common import check_output, check_selection_row, dev, host, sample_tokens

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_consumer", "moe_c_example.c")
PKG = os.path.join(ROOT, "sparse_mixture_experts_40_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

CASES = [
    MoEConfig("tiled", T=700, H=512, E=16, k=4, I=512, norm=True, dtype="bf16"),
    MoEConfig("decode_like", T=64, H=512, E=128, k=8, I=256, norm=True, dtype="bf16",
              zipf_s=1.2),
    WORKLOADS["tiny_f32"],
]


@pytest.fixture(scope="module")
def example(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    binding.load()  # libmoe.so must exist
    exe = str(tmp_path_factory.mktemp("c_consumer") / "moe_c_example")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{ROOT}/include", SRC, f"-L{PKG}", "-lmoe",
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM}/lib",
           "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return exe


def _write_inputs(path, cfg, inp):
    bias = inp.get("logit_bias")
    hdr = np.array([cfg.T, cfg.H, cfg.E, cfg.k, cfg.I, int(cfg.norm),
                    binding.MOE_DTYPE[cfg.dtype], int(bias is not None)], np.int32)
    with open(path, "wb") as f:
        f.write(hdr.tobytes())
        for n in ("x", "w_router", "w_gate", "w_up", "w_down"):
            f.write(np.ascontiguousarray(inp[n]).tobytes())
        if bias is not None:
            f.write(np.ascontiguousarray(bias, np.float32).tobytes())


def _read_outputs(path, cfg):
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    raw = open(path, "rb").read()
    es = 2 if cfg.dtype == "bf16" else 4
    parts, off = {}, 0
    for name, n, dt in (("out", T * H * es, np.uint16 if es == 2 else np.float32),
                        ("idx", T * k * 4, np.int32), ("w", T * k * 4, np.float32),
                        ("counts", E * 4, np.int32), ("f", E * 4, np.float32),
                        ("P", E * 4, np.float32), ("aux", 4, np.float32)):
        parts[name] = np.frombuffer(raw[off:off + n], dtype=dt)
        off += n
    assert off == len(raw)
    return parts


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_c_program_matches_binding_and_oracle(orc, example, tmp_path, cfg):
    print(f"[{cfg.name}] C consumer", flush=True)
    inp = make_inputs(cfg, seed=4)
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    _write_inputs(fin, cfg, inp)
    r = subprocess.run([example, fin, fout], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got = _read_outputs(fout, cfg)

    blk = binding.MoEBlock(cfg, inp)
    blk.forward(dev(inp["x"]))
    torch.cuda.synchronize()
    if cfg.dtype == "bf16":
        bits_b = blk.out.view(torch.int16).cpu().numpy().view(np.uint16)
        bits_c = got["out"].reshape(cfg.T, cfg.H)
    else:
        bits_b = host(blk.out).view(np.uint32)
        bits_c = got["out"].reshape(cfg.T, cfg.H).view(np.uint32)
    assert np.array_equal(bits_c, bits_b)
    assert np.array_equal(got["idx"].reshape(cfg.T, cfg.k), host(blk.topk_idx))
    assert np.array_equal(got["w"].reshape(cfg.T, cfg.k).view(np.uint32),
                          host(blk.topk_w).view(np.uint32))
    for name, t in (("counts", blk.counts), ("f", blk.f), ("P", blk.P), ("aux", blk.aux)):
        assert np.array_equal(got[name].view(np.uint32), host(t).view(np.uint32)), name

    # the oracle on sampled tokens (near ties recomputed with the GPU's choice)
    tokens = sample_tokens(cfg.T, min(cfg.T, 24), seed=9)
    idx = got["idx"].reshape(cfg.T, cfg.k)[tokens]
    ref = orc.forward_tokens(inp, cfg, tokens=tokens)
    for i in np.flatnonzero((idx != ref["idx"]).any(1)):
        check_selection_row(ref["logits"][i], idx[i], ref["idx"][i], cfg.k, tokens[i])
    ref = orc.forward_tokens(inp, cfg, tokens=tokens, forced_idx=idx)
    out = got["out"].reshape(cfg.T, cfg.H)[tokens]
    if cfg.dtype == "bf16":
        out = (out.astype(np.uint32) << 16).view(np.float32)
    mx, _ = check_output(out, ref["out"], cfg.dtype)
    print(f"{cfg.name}: C program = binding bit for bit; {len(tokens)} tokens vs the oracle, "
          f"max|d|/RMS {mx:.4f}", flush=True)

"""GPU parity of the triangle-attention module entry points against the
fp64 oracle: tri_attn_project, tri_attn_out_project, tri_attn_module_fwd."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64, npu8

pytestmark = pytest.mark.gpu


def gpu_module(d, H, C, ending):
    out = ops.tri_attn_module_fwd(
        dev(d["z"]), dev(d["mask"]), dev(d["ln_w"]), dev(d["ln_b"]), d["eps"],
        dev(d["w_q"]), dev(d["w_k"]), dev(d["w_v"]), dev(d["w_g"]),
        dev(d["b_g"]), dev(d["w_bias"]), dev(d["w_o"]), dev(d["b_o"]), H, C,
        ending)
    torch.cuda.synchronize()
    return out.cpu()


def oracle_args(d, H, C):
    return dict(z=np64(d["z"]), residue_mask=npu8(d["mask"]),
                ln_w=np64(d["ln_w"]), ln_b=np64(d["ln_b"]), eps=d["eps"],
                w_q=np64(d["w_q"]), w_k=np64(d["w_k"]), w_v=np64(d["w_v"]),
                w_g=np64(d["w_g"]), b_g=np64(d["b_g"]),
                w_bias=np64(d["w_bias"]), w_o=np64(d["w_o"]),
                b_o=np64(d["b_o"]), H=H, C=C)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ending", [False, True])
@pytest.mark.parametrize("N,CZ,H", [(37, 64, 2), (70, 128, 4), (5, 32, 1)])
def test_project_parity(dtype, ending, N, CZ, H):
    log(f"case project {dtype} N={N} CZ={CZ} H={H} ending={ending}")
    d = synth.rand_module(N, CZ, H, 32, dtype, seed=N, ln_affine=True,
                          gate_bias=True, out_bias=True)
    q, k, v, g, bias = ops.tri_attn_project(
        dev(d["z"]), dev(d["ln_w"]), dev(d["ln_b"]), d["eps"], dev(d["w_q"]),
        dev(d["w_k"]), dev(d["w_v"]), dev(d["w_g"]), dev(d["b_g"]),
        dev(d["w_bias"]), H, 32, ending)
    torch.cuda.synchronize()
    a = oracle_args(d, H, 32)
    ref = O.tri_project(a["z"], a["ln_w"], a["ln_b"], a["eps"], a["w_q"],
                        a["w_k"], a["w_v"], a["w_g"], a["b_g"], a["w_bias"],
                        H, 32, ending)
    for name, got, r in zip(("q", "k", "v", "g", "bias"), (q, k, v, g, bias), ref):
        compare(name, np64(got.cpu()), r, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ending", [False, True])
def test_out_project_parity(dtype, ending):
    N, CZ, H = 45, 96, 3
    log(f"case out_project {dtype} ending={ending}")
    gen = torch.Generator().manual_seed(4)
    o = synth.round_to(torch.randn((1, N, N, H, 32), generator=gen), dtype)
    w_o = synth.round_to(torch.randn((CZ, H * 32), generator=gen) / 10, dtype)
    b_o = synth.round_to(torch.randn((CZ,), generator=gen), dtype)
    out = ops.tri_attn_out_project(dev(o), dev(w_o), dev(b_o), CZ, ending)
    torch.cuda.synchronize()
    ref = O.tri_out_project(np64(o), np64(w_o), np64(b_o), ending)
    compare("out", np64(out.cpu()), ref, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ending", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_module_small_parity(dtype, ending, masked):
    N, CZ, H = 67, 64, 2
    log(f"case module {dtype} N={N} ending={ending} masked={masked}")
    d = synth.rand_module(N, CZ, H, 32, dtype, seed=3 + ending,
                          mask="random5" if masked else None, ln_affine=True,
                          gate_bias=True, out_bias=True)
    out = gpu_module(d, H, 32, ending)
    ref = O.tri_module_forward(ending=ending, **oracle_args(d, H, 32))
    compare("out", np64(out), ref, dtype)


def _sampled_module(name, lines):
    w = synth.WORKLOADS[name]
    d = synth.module_inputs(name)
    H, C, ending = w["H"], w["C"], w["ending"]
    out = gpu_module(d, H, C, ending)
    ref = O.tri_module_lines(lines=lines, ending=ending, **oracle_args(d, H, C))
    for t, line in enumerate(lines):
        got = out[:, line] if ending else out[line]
        compare(f"{name} line {line}", np64(got), ref[t], "bf16")


def test_tri_start_384_sampled_lines():
    """Starting node, z [384,384,128], H=4, no mask: sampled rows."""
    log("case tri_start_384")
    _sampled_module("tri_start_384", [0, 1, 127, 128, 255, 383])


def test_tri_end_768_sampled_lines():
    """Ending node, z [768,768,128], H=4, 38 residues masked: sampled
    columns (the configuration the benchmark times)."""
    log("case tri_end_768")
    _sampled_module("tri_end_768", [0, 5, 300, 511, 512, 767])


def test_module_peak_memory_is_quadratic():
    """Peak device memory of the module grows ~4x per doubling of N (the
    O(N^2) pair tensors), not 8x (the O(N^3) logits, 3.62 GB at N=768)."""
    peaks = {}
    for N in (192, 384, 768):
        d = synth.rand_module(N, 128, 4, 32, "bf16", seed=1)
        args = {k: dev(v) if isinstance(v, torch.Tensor) else v for k, v in d.items()}
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        ops.tri_attn_module_fwd(args["z"], None, args["ln_w"], args["ln_b"],
                                args["eps"], args["w_q"], args["w_k"],
                                args["w_v"], args["w_g"], args["b_g"],
                                args["w_bias"], args["w_o"], args["b_o"], 4,
                                32, True)
        torch.cuda.synchronize()
        peaks[N] = torch.cuda.max_memory_allocated() - base
        log(f"  N={N}: peak extra {peaks[N] / 1e6:.1f} MB")
        del args
    assert 3.0 < peaks[384] / peaks[192] < 5.0
    assert 3.0 < peaks[768] / peaks[384] < 5.0
    assert peaks[768] < 0.5 * 768 ** 3 * 4 * 2  # far below the bf16 logits

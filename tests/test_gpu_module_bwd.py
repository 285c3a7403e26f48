"""GPU parity of the module backward entry points against the fp64 oracle:
tri_attn_out_project_bwd, tri_attn_project_bwd and tri_attn_module_bwd,
called through the C ABI.  d_o and the dz of the projection backward alone
(per position, stored in the working dtype, from exact inputs) are held to
the plain bar plus their storage rounding.  The dz of the whole-module
backward passes through four bf16 roundings along each term (the attention
output o, the gradient d_o, the attention gradient dq/dk/dv/dg, and the
stored dz): plain bar plus 4 * 2^-8 |oracle| (helpers.compare, rounds=4).
The weight and LayerNorm-parameter
gradients (fp32 sums over every pair position) to the bar relative to their
largest entry (helpers.compare, scale="peak")."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64, npu8

pytestmark = pytest.mark.gpu

PARAM_NAMES = ("dln_w", "dln_b", "dw_q", "dw_k", "dw_v", "dw_g", "db_g",
               "dw_bias")


def _draw(gen, shape, dtype, std=1.0):
    return synth.round_to(torch.randn(shape, generator=gen) * std, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ending", [False, True])
@pytest.mark.parametrize("N,CZ,H", [(45, 96, 3), (8, 32, 1)])
def test_out_project_bwd_parity(dtype, ending, N, CZ, H):
    log(f"case out_project_bwd {dtype} N={N} CZ={CZ} H={H} ending={ending}")
    gen = torch.Generator().manual_seed(N + CZ)
    o = _draw(gen, (1, N, N, H, 32), dtype)
    w_o = _draw(gen, (CZ, H * 32), dtype, (H * 32) ** -0.5)
    dout = _draw(gen, (N, N, CZ), dtype)
    d_o, dw_o, db_o = ops.tri_attn_out_project_bwd(dev(o), dev(w_o), dev(dout), ending)
    torch.cuda.synchronize()
    r_do, r_dw, r_db = O.tri_out_project_backward(np64(o), np64(w_o), np64(dout), ending)
    compare("d_o", np64(d_o), r_do, dtype)
    compare("dw_o", np64(dw_o), r_dw, dtype, scale="peak", stored="fp32")
    compare("db_o", np64(db_o), r_db, dtype, scale="peak", stored="fp32")


def _proj_case(N, CZ, H, dtype, seed):
    d = synth.rand_module(N, CZ, H, 32, dtype, seed=seed, ln_affine=True,
                          gate_bias=True)
    gen = torch.Generator().manual_seed(1000 + seed)
    for name in ("dq", "dk", "dv", "dg"):
        d[name] = _draw(gen, (1, N, N, H, 32), dtype)
    d["dbias"] = torch.randn((1, H, N, N), generator=gen) * 4.0  # fp32, row sums
    return d


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ending", [False, True])
@pytest.mark.parametrize("N,CZ,H", [(37, 64, 2), (70, 128, 4), (5, 32, 1), (33, 96, 3)])
def test_project_bwd_parity(dtype, ending, N, CZ, H):
    log(f"case project_bwd {dtype} N={N} CZ={CZ} H={H} ending={ending}")
    d = _proj_case(N, CZ, H, dtype, seed=N + H)
    got = ops.tri_attn_project_bwd(
        dev(d["z"]), dev(d["ln_w"]), dev(d["ln_b"]), d["eps"], dev(d["w_q"]),
        dev(d["w_k"]), dev(d["w_v"]), dev(d["w_g"]), dev(d["w_bias"]),
        dev(d["dq"]), dev(d["dk"]), dev(d["dv"]), dev(d["dg"]), dev(d["dbias"]),
        H, 32, ending)
    torch.cuda.synchronize()
    ref = O.tri_project_backward(
        np64(d["z"]), np64(d["ln_w"]), np64(d["ln_b"]), d["eps"],
        np64(d["w_q"]), np64(d["w_k"]), np64(d["w_v"]), np64(d["w_g"]),
        np64(d["w_bias"]), np64(d["dq"]), np64(d["dk"]), np64(d["dv"]),
        np64(d["dg"]), np64(d["dbias"]), ending)
    compare("dz", np64(got["dz"]), ref["dz"], dtype)
    for name in PARAM_NAMES:
        compare(name, np64(got[name]), ref[name], dtype, scale="peak", stored="fp32")


def _module_case(N, CZ, H, dtype, seed, mask):
    d = synth.rand_module(N, CZ, H, 32, dtype, seed=seed, mask=mask,
                          ln_affine=True, gate_bias=True, out_bias=True)
    gen = torch.Generator().manual_seed(2000 + seed)
    d["dout"] = _draw(gen, (N, N, CZ), dtype)
    return d


def _gpu_module_bwd(d, H, ending):
    g = ops.tri_attn_module_bwd(
        dev(d["z"]), dev(d["mask"]), dev(d["ln_w"]), dev(d["ln_b"]), d["eps"],
        dev(d["w_q"]), dev(d["w_k"]), dev(d["w_v"]), dev(d["w_g"]),
        dev(d["b_g"]), dev(d["w_bias"]), dev(d["w_o"]), dev(d["dout"]), H, 32,
        ending)
    torch.cuda.synchronize()
    return g


def _oracle_module_bwd(d, H, ending):
    return O.tri_module_backward(
        np64(d["z"]), npu8(d["mask"]), np64(d["ln_w"]), np64(d["ln_b"]),
        d["eps"], np64(d["w_q"]), np64(d["w_k"]), np64(d["w_v"]),
        np64(d["w_g"]), np64(d["b_g"]), np64(d["w_bias"]), np64(d["w_o"]),
        np64(d["b_o"]), H, 32, ending, np64(d["dout"]))


def _compare_module(got, ref, dtype, d):
    compare("dz", np64(got["dz"]), ref["dz"], dtype, rounds=4 if dtype == "bf16" else 0)
    for name in PARAM_NAMES + ("dw_o", "db_o"):
        compare(name, np64(got[name]), ref[name], dtype, scale="peak", stored="fp32")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("ending", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_module_bwd_small_parity(dtype, ending, masked):
    N, CZ, H = 67, 64, 2
    log(f"case module_bwd {dtype} N={N} ending={ending} masked={masked}")
    d = _module_case(N, CZ, H, dtype, seed=5 + ending, mask="random5" if masked else None)
    _compare_module(_gpu_module_bwd(d, H, ending), _oracle_module_bwd(d, H, ending), dtype, d)


def test_module_bwd_c128_h4_parity():
    """c_z = 128, 4 heads (the pages' pair width), ending node, masked
    residues, bf16: several position tiles, the full contraction of the
    projection backward (4 x 128 + the pair-bias block) and a ragged tail."""
    N, CZ, H = 100, 128, 4
    log(f"case module_bwd bf16 N={N} CZ={CZ} H={H} ending masked")
    d = _module_case(N, CZ, H, "bf16", seed=11, mask="random5")
    _compare_module(_gpu_module_bwd(d, H, True), _oracle_module_bwd(d, H, True), "bf16", d)


def test_module_bwd_tri_end_768_properties():
    """Full size (z [768,768,128], ending node, 38 residues masked, bf16):
    properties that hold at any size.  Every position's dz sums to ~0 over
    channels (LayerNorm is invariant to a shift of a position's channels);
    db_o is the sum of dout over positions (computed in fp64 here); two runs
    agree bit for bit; everything is finite."""
    log("case module_bwd tri_end_768")
    w = synth.WORKLOADS["tri_end_768"]
    N, CZ, H = w["N"], w["CZ"], w["H"]
    d = synth.module_inputs("tri_end_768")
    gen = torch.Generator().manual_seed(7)
    d["dout"] = _draw(gen, (N, N, CZ), "bf16")
    g1 = _gpu_module_bwd(d, H, True)
    g2 = _gpu_module_bwd(d, H, True)
    for name in g1:
        assert torch.equal(g1[name], g2[name]), f"{name} differs between runs"
        assert torch.isfinite(g1[name]).all(), name
    dz = g1["dz"].float()
    s = dz.sum(-1).abs()
    bound = 2.0 ** -8 * dz.abs().sum(-1) + 1e-6
    assert bool((s <= bound).all()), float((s / bound).max())
    compare("db_o", np64(g1["db_o"]), np64(d["dout"]).sum((0, 1)), "bf16", scale="peak", stored="fp32")


def test_project_bwd_tri_end_768_parity():
    """tri_attn_project_bwd at full size: z [768,768,128], ending node, 4
    heads of 32, affine LayerNorm, bf16, incoming gradients dq, dk, dv, dg
    ~ N(0,1) and dBias ~ N(0,16) (a sum over rows).  Every output against
    the oracle's full backward (~20 s of fp64 on the host): dz at all
    589824 positions and every parameter gradient summed over all of them."""
    N, CZ, H = 768, 128, 4
    log(f"case project_bwd bf16 N={N} CZ={CZ} H={H} ending (full size)")
    d = synth.rand_module(N, CZ, H, 32, "bf16", seed=31, ln_affine=True,
                          gate_bias=True)
    gen = torch.Generator().manual_seed(1031)
    for name in ("dq", "dk", "dv", "dg"):
        d[name] = _draw(gen, (1, N, N, H, 32), "bf16")
    d["dbias"] = torch.randn((1, H, N, N), generator=gen) * 4.0
    got = ops.tri_attn_project_bwd(
        dev(d["z"]), dev(d["ln_w"]), dev(d["ln_b"]), d["eps"], dev(d["w_q"]),
        dev(d["w_k"]), dev(d["w_v"]), dev(d["w_g"]), dev(d["w_bias"]),
        dev(d["dq"]), dev(d["dk"]), dev(d["dv"]), dev(d["dg"]), dev(d["dbias"]),
        H, 32, True)
    torch.cuda.synchronize()
    got = {k: v.cpu() for k, v in got.items()}
    log("  oracle ...")
    ref = O.tri_project_backward(
        np64(d["z"]), np64(d["ln_w"]), np64(d["ln_b"]), d["eps"],
        np64(d["w_q"]), np64(d["w_k"]), np64(d["w_v"]), np64(d["w_g"]),
        np64(d["w_bias"]), np64(d["dq"]), np64(d["dk"]), np64(d["dv"]),
        np64(d["dg"]), np64(d["dbias"]), True)
    compare("dz", np64(got["dz"]), ref["dz"], "bf16")
    for name in PARAM_NAMES:
        compare(name, np64(got[name]), ref[name], "bf16", scale="peak", stored="fp32")


def test_out_project_bwd_tri_end_768_parity():
    """tri_attn_out_project_bwd at full size: o [1,768,768,4,32], the
    ending node's transposed write, c_z = 128, bf16: d_o at every position
    (per position, plain bar) and dw_o, db_o summed over all
    589824 positions, against the oracle in full."""
    N, CZ, H = 768, 128, 4
    log(f"case out_project_bwd bf16 N={N} CZ={CZ} H={H} ending (full size)")
    gen = torch.Generator().manual_seed(768)
    o = _draw(gen, (1, N, N, H, 32), "bf16")
    w_o = _draw(gen, (CZ, H * 32), "bf16", (H * 32) ** -0.5)
    dout = _draw(gen, (N, N, CZ), "bf16")
    d_o, dw_o, db_o = ops.tri_attn_out_project_bwd(dev(o), dev(w_o), dev(dout), True)
    torch.cuda.synchronize()
    r_do, r_dw, r_db = O.tri_out_project_backward(np64(o), np64(w_o), np64(dout), True)
    compare("d_o", np64(d_o), r_do, "bf16")
    compare("dw_o", np64(dw_o), r_dw, "bf16", scale="peak", stored="fp32")
    compare("db_o", np64(db_o), r_db, "bf16", scale="peak", stored="fp32")

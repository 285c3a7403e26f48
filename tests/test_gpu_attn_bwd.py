"""GPU parity of evo_attn_bwd (dQ, dK, dV, dGate, dBias summed over rows)
against the fp64 oracle, plus closed-form invariants on the GPU outputs."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64, npu8

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(d, want_dbias=True):
    q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    g, m, b, do = dev(d["gate"]), dev(d["mask"]), dev(d["bias"]), dev(d["dout"])
    out, lse = ops.evo_attn_fwd(q, k, v, g, m, b, want_lse=True)
    grads = ops.evo_attn_bwd(q, k, v, g, m, b, out, lse, do, want_dbias=want_dbias)
    torch.cuda.synchronize()
    return [None if t is None else t.cpu() for t in grads]


def oracle_bwd(d):
    return O.attention_backward(np64(d["q"]), np64(d["k"]), np64(d["v"]),
                                np64(d["gate"]), npu8(d["mask"]),
                                np64(d["bias"]), np64(d["dout"]))


SHAPES = [  # B, R, N, H
    (1, 1, 1, 1), (1, 3, 17, 2), (2, 2, 64, 1), (1, 4, 100, 2), (1, 2, 130, 3),
    (1, 5, 256, 1), (1, 2, 300, 1),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("opts", ["all", "nogate", "rowmask", "plain"])
def test_bwd_parity_small(dtype, shape, opts):
    B, R, N, H = shape
    log(f"case bwd {dtype} B={B} R={R} N={N} H={H} {opts}")
    d = synth.rand_core(B, R, N, H, 32, dtype, seed=N + R, dout=True,
                        gate=opts not in ("nogate", "plain"),
                        bias=opts != "plain",
                        mask=None if opts == "plain" else "random",
                        mask_rows=R if opts == "rowmask" else 1)
    got = gpu_fwd_bwd(d)
    ref = oracle_bwd(d)
    for name, gt, r in zip(("dq", "dk", "dv", "dgate", "dbias"), got, ref):
        if r is None:
            assert gt is None
            continue
        # dBias sums the R rows of dS: bound relative to its own peak.
        scale = "peak" if name == "dbias" else 1.0
        compare(name, np64(gt), r, dtype, scale=scale)


def test_bwd_invariants_on_gpu_outputs():
    """sum_k dBias = 0, sum_k dK = 0, sum_k dV = sum_q dO*sigmoid(G)."""
    d = synth.rand_core(1, 6, 150, 2, 32, "fp32", seed=21, dout=True,
                        mask="random")
    dq, dk, dv, dg, db = gpu_fwd_bwd(d)
    assert db.sum(-1).abs().max() < 1e-4
    assert dk.sum(2).abs().max() < 1e-4
    do_pre = d["dout"] * torch.sigmoid(d["gate"])
    assert (dv.sum(2) - do_pre.sum(2)).abs().max() < 1e-3


def test_bwd_without_dbias_and_deterministic():
    d = synth.rand_core(1, 3, 96, 2, 32, "bf16", seed=8, dout=True, mask="random")
    a = gpu_fwd_bwd(d, want_dbias=False)
    assert a[4] is None
    b = gpu_fwd_bwd(d, want_dbias=True)
    c = gpu_fwd_bwd(d, want_dbias=True)
    for x, y in zip(b, c):
        assert torch.equal(x, y)
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)


def test_tri_start_512_fwd_bwd_sampled():
    """Projection + core forward + core backward at full size: starting
    node, z [512,512,128], H=4, upstream gradient ~ N(0,1).  The oracle
    projects z itself (fp64) and its gradients are compared on sampled lines;
    dBias (a sum over all 512 lines) on sampled query rows."""
    log("case tri_start_512_bwd")
    w = synth.WORKLOADS["tri_start_512_bwd"]
    d = synth.module_inputs("tri_start_512_bwd")
    H, C = w["H"], w["C"]
    q, k, v, g, bias = ops.tri_attn_project(
        dev(d["z"]), dev(d["ln_w"]), dev(d["ln_b"]), d["eps"], dev(d["w_q"]),
        dev(d["w_k"]), dev(d["w_v"]), dev(d["w_g"]), dev(d["b_g"]),
        dev(d["w_bias"]), H, C, False)
    do = dev(d["dout"])
    out, lse = ops.evo_attn_fwd(q, k, v, g, None, bias, want_lse=True)
    dq, dk, dv, dg, db = ops.evo_attn_bwd(q, k, v, g, None, bias, out, lse, do)
    torch.cuda.synchronize()
    dq, dk, dv, dg, db = (t.cpu() for t in (dq, dk, dv, dg, db))
    oq, ok, ov, og, ob = O.tri_project(np64(d["z"]), np64(d["ln_w"]),
                                       np64(d["ln_b"]), d["eps"], np64(d["w_q"]),
                                       np64(d["w_k"]), np64(d["w_v"]),
                                       np64(d["w_g"]), np64(d["b_g"]),
                                       np64(d["w_bias"]), H, C, False)
    dout = np64(d["dout"])
    for r in (0, 1, 255, 511):
        rq, rk, rv, rg_, _ = O.attention_line_backward(
            oq[0, r], ok[0, r], ov[0, r], og[0, r], ob[0], None, dout[0, r])
        compare(f"dq[{r}]", np64(dq[0, r]), rq, "bf16")
        compare(f"dk[{r}]", np64(dk[0, r]), rk, "bf16")
        compare(f"dv[{r}]", np64(dv[0, r]), rv, "bf16")
        compare(f"dgate[{r}]", np64(dg[0, r]), rg_, "bf16")
    picks = [(0, 0), (1, 100), (2, 311), (3, 511)]
    ref = O.dbias_query_rows(oq, ok, ov, og, None, ob, dout, 0, picks)
    got = np.stack([np64(db[0, h, qi]) for h, qi in picks])
    compare("dbias rows", got, ref, "bf16", scale="peak")

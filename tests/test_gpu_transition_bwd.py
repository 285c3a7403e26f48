"""GPU parity of the transition backward (pair_transition_bwd, through the C
ABI) against the fp64 oracle.

dz is a LayerNorm backward of du . w_a + dv . w_b, sums over 2 * HID hidden
units whose du, dv are rounded to the working dtype before the product (as
the forward's hidden layer).  Along the path of a dz term the kernels round
to bf16 four times (the hidden gradient dh, du or dv, the layer-normalised
row of the recomputed forward, and the stored dz), so dz is held to the
plain bar plus 4 * 2^-8 |oracle| (rounds=4); the weight and LayerNorm-parameter gradients
are sums over every position.  dz (per position, stored in the working
dtype) is held to the plain bar; the fp32 parameter gradients to the bar
relative to their largest entry (helpers.compare, scale="peak")."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64

pytestmark = pytest.mark.gpu

NAMES = ("dz", "dln_w", "dln_b", "dw_a", "dw_b", "dw_o")


def gpu_bwd(d):
    g = ops.pair_transition_bwd(dev(d["z"]), dev(d["ln_w"]), dev(d["ln_b"]), d["eps"],
                                dev(d["w_a"]), dev(d["w_b"]), dev(d["w_o"]), dev(d["dout"]))
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in g.items()}


def oracle_args(d):
    return dict(z=np64(d["z"]), ln_w=np64(d["ln_w"]), ln_b=np64(d["ln_b"]), eps=d["eps"],
                w_a=np64(d["w_a"]), w_b=np64(d["w_b"]), w_o=np64(d["w_o"]),
                dout=np64(d["dout"]))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("N,CZ,HID", [(13, 64, 128), (37, 128, 256), (20, 32, 512),
                                      (9, 96, 384), (6, 128, 1024)])
def test_transition_bwd_parity(dtype, N, CZ, HID):
    """Ragged position counts (tails of the 256-position tiles), every
    supported c_z, 1 to 8 weight-gradient segments of 128 hidden units (one
    at a time and four at a time)."""
    log(f"case transition_bwd {dtype} N={N} CZ={CZ} HID={HID}")
    d = synth.rand_transition(N, CZ, HID, dtype, seed=N + HID, dout=True)
    got = gpu_bwd(d)
    ref = O.transition_backward(**oracle_args(d))
    for k in NAMES:
        if k == "dz":
            compare(k, np64(got[k]), ref[k], dtype, rounds=4 if dtype == "bf16" else 0)
        else:
            compare(k, np64(got[k]), ref[k], dtype, scale="peak", stored="fp32")


def test_transition_bwd_768_sampled():
    """Full size (z [768,768,128], hidden 512, bf16): dz on sampled rows of
    z (per position), and the weight gradients of sampled hidden units over
    all 589824 positions, the oracle forming those units alone."""
    log("case transition_bwd_768")
    d = synth.transition_inputs("transition_768", dout=True)
    got = gpu_bwd(d)
    a = oracle_args(d)
    for r in (0, 383, 767):
        e = dict(a, z=a["z"][r:r + 1], dout=a["dout"][r:r + 1])
        ref = O.transition_backward(**e)
        compare(f"dz[{r}]", np64(got["dz"][r:r + 1]), ref["dz"], "bf16", rounds=4)
    units = [0, 77, 255, 256, 511]
    ga, gb, go = O.transition_weight_grad_units(units=units, **a)
    compare("dw_a[units]", np64(got["dw_a"])[units], ga, "bf16", scale="peak", stored="fp32")
    compare("dw_b[units]", np64(got["dw_b"])[units], gb, "bf16", scale="peak", stored="fp32")
    compare("dw_o[:, units]", np64(got["dw_o"])[:, units], go, "bf16", scale="peak", stored="fp32")


def test_transition_bwd_deterministic():
    """Two runs agree bit for bit (fixed-order reductions, no atomics)."""
    d = synth.rand_transition(40, 64, 256, "bf16", seed=3, dout=True)
    a = gpu_bwd(d)
    b = gpu_bwd(d)
    for k in NAMES:
        assert torch.equal(a[k], b[k]), k


def test_transition_bwd_768_parameter_gradients_in_chunks():
    """Full size: every parameter gradient (dln_w, dln_b, dw_a, dw_b, dw_o)
    is a sum over positions, so the oracle's gradients of position chunks add
    up to the whole (fp64); compared in full against the GPU result."""
    log("case transition_bwd_768 chunked")
    d = synth.transition_inputs("transition_768", dout=True)
    got = gpu_bwd(d)
    a = oracle_args(d)
    z = a["z"].reshape(-1, 1, a["z"].shape[-1])
    dout = a["dout"].reshape(-1, 1, a["dout"].shape[-1])
    tot = None
    step = 32768
    for p0 in range(0, z.shape[0], step):
        e = dict(a, z=z[p0:p0 + step], dout=dout[p0:p0 + step])
        g = O.transition_backward(**e)
        g.pop("dz")
        tot = g if tot is None else {k: tot[k] + g[k] for k in tot}
    for k, v in tot.items():
        compare(k, np64(got[k]), v, "bf16", scale="peak", stored="fp32")

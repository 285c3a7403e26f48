"""GPU parity of the outer product mean (outer_product_mean_fwd, through the
C ABI) against the fp64 oracle.

fp32 meets the plain bar.  In bf16 each output is a sum over C*C products
o[i,j,c,d] * w_o, each o a mean over S sequences of a * b, with the
operands, a, b and the product o stored in bf16 in between (six roundings
along each term), in sums that cancel, so an output's error follows the
size of its terms rather than its own and the plain 2e-2 max-abs bar is not
reachable (up to ~4e-2 measured).  As for the multiplicative update, the
first-order worst case of those roundings exceeds the outputs, and the bar
used, the plain one in units of the output's largest entry
(helpers.compare, scale="peak"), is tighter than the probabilistic bound of
independent roundings; the relative L2 bar is unchanged."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64

pytestmark = pytest.mark.gpu


def gpu_opm(d):
    out = ops.outer_product_mean_fwd(dev(d["m"]), dev(d["ln_w"]), dev(d["ln_b"]),
                                     d["eps"], dev(d["w_a"]), dev(d["w_b"]),
                                     dev(d["w_o"]), dev(d["b_o"]))
    torch.cuda.synchronize()
    return out.cpu()


def oracle_args(d):
    return dict(m=np64(d["m"]), ln_w=np64(d["ln_w"]), ln_b=np64(d["ln_b"]),
                eps=d["eps"], w_a=np64(d["w_a"]), w_b=np64(d["w_b"]),
                w_o=np64(d["w_o"]), b_o=np64(d["b_o"]))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("S,N,CM,C,CZ", [(37, 45, 64, 32, 64), (130, 9, 256, 32, 128),
                                         (1, 70, 32, 64, 32), (200, 130, 96, 32, 96),
                                         (64, 260, 128, 32, 128), (33, 20, 256, 128, 128)])
def test_opm_parity(dtype, S, N, CM, C, CZ):
    """Ragged S (not a multiple of the 64-wide stage, and S = 1), ragged N
    (N*C spanning several 256-row product tiles and a tail; N above the 256
    pairs of an output tile), every supported output width class, and the
    widest supported channels (c_m = 256, c = 128, c_z = 128)."""
    log(f"case opm {dtype} S={S} N={N} CM={CM} C={C} CZ={CZ}")
    d = synth.rand_opm(S, N, CM, C, CZ, dtype, seed=S + N)
    got = gpu_opm(d)
    ref = O.outer_product_mean(**oracle_args(d))
    compare("out", np64(got), ref, dtype, scale="peak")


def test_opm_1024x768_sampled():
    """Full size (m [1024,768,256], 32 channels, out [768,768,128], bf16):
    sampled entries, the oracle forming only the residues they need."""
    log("case opm_1024x768")
    d = synth.opm_inputs("opm_1024x768")
    got = gpu_opm(d)
    picks = [(0, 0), (0, 767), (767, 0), (383, 384), (255, 256), (500, 17), (766, 765)]
    ref = O.outer_product_mean_pairs(picks=picks, **oracle_args(d))
    for t, (i, j) in enumerate(picks):
        compare(f"out[{i},{j}]", np64(got[i, j]), ref[t], "bf16", scale="peak")


def test_opm_deterministic_and_sequence_order():
    """Two runs agree bit for bit; reversing the sequence order leaves the
    mean unchanged up to the order of the fp32 sums (bf16 rounding of the
    product allows one unit in the last place)."""
    d = synth.rand_opm(96, 80, 64, 32, 64, "bf16", seed=11)
    a = gpu_opm(d)
    b = gpu_opm(d)
    assert torch.equal(a, b)
    e = dict(d)
    e["m"] = d["m"].flip(0).contiguous()
    c = gpu_opm(e)
    compare("reversed", np64(c), np64(a), "bf16", rounds=2)

"""GPU parity of the outer product mean's backward (outer_product_mean_bwd,
through the C ABI) against the fp64 oracle (outer_product_mean_backward).

Every gradient is compared elementwise, with the bar in units of each
output's largest entry (helpers.compare, scale="peak"); the relative L2 bar
is unchanged.  The parameter gradients are sums over all positions (N^2
pairs or S*N sequence-residue positions), far above the literal absolute
bar in fp32 summation alone; in bf16 the path holds the operands a, b, the
recomputed product, dP and its transpose and the products dA, dB in bf16
between steps, and dA, dB are sums over N*C terms that cancel, so as for the
forward an output's error follows the size of its terms, not its own.
Measured worst: 0.34 of the bar in bf16 (dm at the sampled full-size
positions: 2.2e-2 against a largest entry of 3.0), 0.02 in fp32; relative
L2 <= 5.9e-3."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64

pytestmark = pytest.mark.gpu

GRADS = ("dm", "dln_w", "dln_b", "dw_a", "dw_b", "dw_o", "db_o")


def gpu_bwd(d, m=None):
    r = ops.outer_product_mean_bwd(dev(d["m"] if m is None else m), dev(d["ln_w"]),
                                   dev(d["ln_b"]), d["eps"], dev(d["w_a"]), dev(d["w_b"]),
                                   dev(d["w_o"]), dev(d["dout"]))
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in r.items()}


def oracle_args(d):
    return dict(m=np64(d["m"]), ln_w=np64(d["ln_w"]), ln_b=np64(d["ln_b"]),
                eps=d["eps"], w_a=np64(d["w_a"]), w_b=np64(d["w_b"]),
                w_o=np64(d["w_o"]), dout=np64(d["dout"]))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("S,N,CM,C,CZ", [(37, 45, 64, 32, 64), (130, 9, 256, 32, 128),
                                         (1, 70, 32, 64, 32), (200, 130, 96, 32, 96),
                                         (64, 100, 128, 32, 128), (33, 20, 256, 128, 128)])
def test_opm_bwd_parity(dtype, S, N, CM, C, CZ):
    """The forward test's shapes: ragged S (and S = 1), N*C spanning several
    product tiles and a tail, both LayerNorm widths (up to 128 and 256),
    c = 128."""
    log(f"case opm_bwd {dtype} S={S} N={N} CM={CM} C={C} CZ={CZ}")
    d = synth.rand_opm(S, N, CM, C, CZ, dtype, seed=S + N + 1, dout=True)
    got = gpu_bwd(d)
    ref = O.outer_product_mean_backward(b_o=np64(d["b_o"]), **oracle_args(d))
    for k in GRADS:
        compare(f"S={S} N={N} {k}", np64(got[k]), ref[k], dtype, scale="peak",
                stored=dtype if k == "dm" else "fp32")


def test_opm_bwd_1024x768_sampled():
    """Full size (m [1024,768,256], 32 channels, dout [768,768,128], bf16):
    dm at sampled (sequence, residue) positions, rows of dW_a and dW_b and
    columns of dW_o, the oracle forming only what they need; db_o in full."""
    log("case opm_bwd opm_1024x768")
    d = synth.opm_inputs("opm_1024x768", dout=True)
    got = gpu_bwd(d)
    dm_picks = [(0, 0), (1023, 767), (500, 17), (3, 384)]
    wa_rows, wb_rows, wo_cols = [0, 31], [5], [(0, 0), (31, 31), (3, 17)]
    dm, ra, rb, ro = O.outer_product_mean_backward_sampled(
        dm_picks=dm_picks, wa_rows=wa_rows, wb_rows=wb_rows, wo_cols=wo_cols,
        **oracle_args(d))
    compare("dm[picks]", np64(got["dm"][[s for s, _ in dm_picks], [i for _, i in dm_picks]]),
            dm, "bf16", scale="peak")
    compare("dw_a rows", np64(got["dw_a"][wa_rows]), ra, "bf16", scale="peak", stored="fp32")
    compare("dw_b rows", np64(got["dw_b"][wb_rows]), rb, "bf16", scale="peak", stored="fp32")
    cols = [c * 32 + e for c, e in wo_cols]
    compare("dw_o cols", np64(got["dw_o"][:, cols]), ro, "bf16", scale="peak", stored="fp32")
    compare("db_o", np64(got["db_o"]), np64(d["dout"]).sum((0, 1)), "bf16", stored="fp32")


def test_opm_bwd_deterministic_and_sequence_order():
    """Two runs agree bit for bit; reversing the sequence order reverses dm
    and leaves the parameter gradients unchanged up to the order of the
    sums."""
    d = synth.rand_opm(96, 80, 64, 32, 64, "bf16", seed=12, dout=True)
    a = gpu_bwd(d)
    b = gpu_bwd(d)
    for k in GRADS:
        assert torch.equal(a[k], b[k]), k
    c = gpu_bwd(d, m=d["m"].flip(0).contiguous())
    compare("dm reversed", np64(c["dm"].flip(0)), np64(a["dm"]), "bf16", scale="peak",
            rounds=2)
    for k in GRADS[1:]:
        torch.testing.assert_close(a[k], c[k], rtol=1e-2, atol=1e-2 * float(a[k].abs().max()))

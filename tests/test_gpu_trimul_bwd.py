"""GPU parity of the multiplicative update's backward (tri_mul_bwd, through
the C ABI) against the fp64 oracle (tri_mul_backward).

Every gradient is compared elementwise, with the bar in units of each
output's largest entry (helpers.compare, scale="peak"); the relative L2 bar
is unchanged.  The parameter gradients are sums over all N^2 positions, of
magnitude 10 to 1e4 here: fp32 summation alone puts them ~4e-7 relative
from the fp64 oracle (up to 9e-3 absolute for dw_o at N = 130), far above
the literal 1e-4.  In bf16 the path holds the operands a, b, their
transposes, dT = dout . W_o, the recomputed t and the products dA, dB in
bf16 between steps; dA and dB are sums over N third residues that cancel
like the forward's t, and dz, dW_a, dW_b, dln are sums of them, so as for
the forward an output's error follows the size of its terms, not its own
(dz at N = 5: 2.7e-2 against a largest entry of 4.7).  Measured worst: 0.36
of the bar in bf16 (dw_b, N = 5), 0.01 in fp32; relative L2 <= 4.4e-3."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64, npu8

pytestmark = pytest.mark.gpu

GRADS = ("dz", "dln_w", "dln_b", "dw_a", "dw_b", "dw_o", "db_o")


def gpu_bwd(d, outgoing, z=None, dout=None):
    r = ops.tri_mul_bwd(dev(d["z"] if z is None else z), dev(d["mask"]), dev(d["ln_w"]),
                        dev(d["ln_b"]), d["eps"], dev(d["w_a"]), dev(d["w_b"]),
                        dev(d["w_o"]), dev(d["dout"] if dout is None else dout), outgoing)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in r.items()}


def oracle_args(d):
    return dict(z=np64(d["z"]), residue_mask=npu8(d["mask"]), ln_w=np64(d["ln_w"]),
                ln_b=np64(d["ln_b"]), eps=d["eps"], w_a=np64(d["w_a"]),
                w_b=np64(d["w_b"]), w_o=np64(d["w_o"]), b_o=np64(d["b_o"]),
                dout=np64(d["dout"]))


def check_all(got, ref, dtype, tag):
    for k in GRADS:
        compare(f"{tag} {k}", np64(got[k]), ref[k], dtype, scale="peak",
                stored=dtype if k == "dz" else "fp32")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("outgoing", [True, False])
@pytest.mark.parametrize("N,CZ,C,mask", [(37, 64, 32, "random5"), (130, 128, 128, None),
                                         (5, 32, 64, None), (200, 96, 96, "random5")])
def test_trimul_bwd_parity(dtype, outgoing, N, CZ, C, mask):
    """Ragged N (several product tiles and a tail, permute blocks of 64 with
    a partial last one), both orientations, with and without a residue
    mask."""
    log(f"case trimul_bwd {dtype} N={N} CZ={CZ} C={C} outgoing={outgoing} mask={mask}")
    d = synth.rand_trimul(N, CZ, C, dtype, seed=N + C + 1, mask=mask, dout=True)
    got = gpu_bwd(d, outgoing)
    ref = O.tri_mul_backward(outgoing=outgoing, **oracle_args(d))
    check_all(got, ref, dtype, f"N={N}")


def test_trimul_bwd_out_768():
    """Full size (z [768,768,128], 128 channels, outgoing, 38 residues
    masked, bf16): every gradient against the full oracle."""
    log("case trimul_bwd trimul_out_768")
    d = synth.trimul_inputs("trimul_out_768", dout=True)
    got = gpu_bwd(d, True)
    ref = O.tri_mul_backward(outgoing=True, **oracle_args(d))
    check_all(got, ref, "bf16", "768")


def test_trimul_bwd_deterministic_and_incoming_transpose_identity():
    """Two runs agree bit for bit; the incoming backward on z equals the
    outgoing backward on z with its residue axes swapped: dz transposed back
    bit for bit, the parameter gradients (sums over positions taken in
    another order) to fp32 rounding."""
    d = synth.rand_trimul(96, 64, 64, "bf16", seed=7, mask="random5", dout=True)
    a = gpu_bwd(d, False)
    b = gpu_bwd(d, False)
    for k in GRADS:
        assert torch.equal(a[k], b[k]), k
    c = gpu_bwd(d, True, z=d["z"].transpose(0, 1).contiguous(),
                dout=d["dout"].contiguous())
    assert torch.equal(a["dz"], c["dz"].transpose(0, 1)), "dz"
    for k in GRADS[1:]:
        torch.testing.assert_close(a[k], c[k], rtol=1e-5, atol=1e-5 * float(a[k].abs().max()))

"""GPU parity of the fused LayerNorm + SwiGLU transition (pair_transition_fwd,
through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64

pytestmark = pytest.mark.gpu


def gpu_transition(d):
    out = ops.pair_transition_fwd(dev(d["z"]), dev(d["ln_w"]), dev(d["ln_b"]), d["eps"],
                                  dev(d["w_a"]), dev(d["w_b"]), dev(d["w_o"]))
    torch.cuda.synchronize()
    return out.cpu()


def oracle_out(d, z=None):
    return O.transition_forward(np64(d["z"] if z is None else z), np64(d["ln_w"]),
                                np64(d["ln_b"]), d["eps"], np64(d["w_a"]), np64(d["w_b"]),
                                np64(d["w_o"]))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("N,CZ,HID", [(37, 64, 256), (5, 32, 64), (70, 128, 512), (16, 96, 192),
                                      (9, 128, 4096)])
def test_transition_parity(dtype, N, CZ, HID):
    """Ragged position counts (tails of the 256-position tiles), every
    supported c_z, hidden widths of 1 to 8 chunks of 64, and the widest
    supported hidden layer (4096)."""
    log(f"case transition {dtype} N={N} CZ={CZ} HID={HID}")
    d = synth.rand_transition(N, CZ, HID, dtype, seed=N + HID)
    compare("out", np64(gpu_transition(d)), oracle_out(d), dtype)


def test_transition_768_sampled_rows():
    """Full size (z [768,768,128], hidden 512, bf16): sampled rows of z, the
    oracle applied to those positions only (the transition is per
    position)."""
    log("case transition_768")
    d = synth.transition_inputs("transition_768")
    got = gpu_transition(d)
    for i in (0, 1, 383, 767):
        ref = oracle_out(d, z=d["z"][i:i + 1])
        compare(f"row {i}", np64(got[i:i + 1]), ref, "bf16")


def test_transition_deterministic():
    d = synth.rand_transition(64, 128, 512, "bf16", seed=9)
    assert torch.equal(gpu_transition(d), gpu_transition(d))

"""GPU parity of evo_attn_fwd against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64, npu8

pytestmark = pytest.mark.gpu

DT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def run_gpu(d):
    out, lse = ops.evo_attn_fwd(dev(d["q"]), dev(d["k"]), dev(d["v"]),
                                dev(d["gate"]), dev(d["mask"]), dev(d["bias"]),
                                want_lse=True)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def run_oracle(d):
    return O.attention_forward(np64(d["q"]), np64(d["k"]), np64(d["v"]),
                               np64(d["gate"]), npu8(d["mask"]), np64(d["bias"]))


def check(d, dtype, rows=None):
    out, lse = run_gpu(d)
    if rows is None:
        ref, ref_lse = run_oracle(d)
        compare("out", np64(out), ref, dtype)
        compare("lse", lse.numpy().astype(np.float64), ref_lse, dtype, stored="fp32")
        return
    mask = npu8(d["mask"])
    for (b, r) in rows:
        keep = None
        if mask is not None:
            keep = mask[b, 0 if mask.shape[1] == 1 else r] != 0
        g = None if d["gate"] is None else np64(d["gate"][b, r])
        bias = None if d["bias"] is None else np64(d["bias"][b])
        ref, ref_lse = O.attention_line_forward(
            np64(d["q"][b, r]), np64(d["k"][b, r]), np64(d["v"][b, r]), g, bias,
            keep)
        compare(f"out[{b},{r}]", np64(out[b, r]), ref, dtype)
        compare(f"lse[{b},{r}]", lse[b, r].numpy().astype(np.float64), ref_lse,
                dtype, stored="fp32")


def test_core_fp32_small_workload():
    """32 lines, N=32, H=4, C=32, fp32, bias and gate, no mask, seed 0."""
    log("case core_fp32_small")
    d = synth.core_inputs("core_fp32_small")
    check(d, "fp32")


def test_msa_row_bf16_workload_sampled_rows():
    """MSA row attention with pair bias at full size (128 rows, 256 residues,
    8 heads, last 26 residues masked): sampled rows against the oracle."""
    log("case msa_row_bf16")
    d = synth.core_inputs("msa_row_bf16")
    check(d, "bf16", rows=[(0, 0), (0, 1), (0, 63), (0, 64), (0, 126), (0, 127)])


SHAPES = [  # B, R, N, H
    (1, 1, 1, 1), (2, 3, 17, 2), (1, 5, 100, 3), (2, 2, 130, 1),
    (1, 3, 64, 4), (1, 2, 200, 2), (1, 4, 129, 2),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("opts", ["all", "nogate", "nobias", "rowmask", "plain"])
def test_parity_small_shapes(dtype, shape, opts):
    B, R, N, H = shape
    log(f"case fwd {dtype} B={B} R={R} N={N} H={H} {opts}")
    mask = {"all": "random", "nogate": "random", "nobias": "random",
            "rowmask": "random", "plain": None}[opts]
    d = synth.rand_core(B, R, N, H, 32, dtype, seed=N + 7 * R + H,
                        gate=opts not in ("nogate", "plain"),
                        bias=opts not in ("nobias", "plain"), mask=mask,
                        mask_rows=R if opts == "rowmask" else 1)
    check(d, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fully_masked_line_and_single_key(dtype):
    log(f"case fwd masked edge {dtype}")
    d = synth.rand_core(1, 3, 40, 2, 32, dtype, seed=5, mask="random", mask_rows=3)
    m = d["mask"].clone()
    m[0, 0, :] = 0          # line 0: every key masked -> out 0, lse -inf
    m[0, 1, :] = 0
    m[0, 1, 17] = 1         # line 1: one key left -> sigmoid(g) * V[17]
    d["mask"] = m
    out, lse = run_gpu(d)
    assert torch.all(out[0, 0] == 0)
    assert torch.all(torch.isneginf(lse[0, 0]))
    expect = torch.sigmoid(d["gate"][0, 1].float()) * d["v"][0, 1, 17].float()[None]
    tol = 1e-5 if dtype == "fp32" else 2e-2
    assert (out[0, 1].float() - expect).abs().max() <= tol
    check(d, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_neg_inf_bias_entries_act_as_masks(dtype):
    """-inf pair-bias entries remove single (query, key) pairs, and a query
    whose bias row is all -inf gets out 0 and lse -inf, as with a mask (the
    bf16 path stores them as the lowest finite bf16 and must still give
    p = 0 exactly)."""
    log(f"case fwd -inf bias {dtype}")
    d = synth.rand_core(1, 3, 70, 2, 32, dtype, seed=21, mask="random")
    gen = torch.Generator().manual_seed(3)
    holes = torch.rand(d["bias"].shape, generator=gen) < 0.2
    b = d["bias"].clone()
    b[holes] = float("-inf")
    b[0, 1, 9, :] = float("-inf")   # head 1, query 9: nothing left
    d["bias"] = b
    out, lse = run_gpu(d)
    assert torch.isfinite(out).all()
    assert torch.all(out[:, :, 9, 1] == 0)
    assert torch.all(torch.isneginf(lse[:, :, 1, 9]))
    check(d, dtype)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fully_masked_batch_shared_mask(dtype):
    """A shared key mask (one per batch entry, folded into the prepared
    bias) that removes every key of batch entry 1: its lines give out 0 and
    lse -inf; batch entry 0 is unaffected."""
    log(f"case fwd shared mask empty {dtype}")
    d = synth.rand_core(2, 3, 45, 2, 32, dtype, seed=8, mask="random")
    m = d["mask"].clone()
    m[1] = 0
    d["mask"] = m
    out, lse = run_gpu(d)
    assert torch.all(out[1] == 0)
    assert torch.all(torch.isneginf(lse[1]))
    check(d, dtype)


@pytest.mark.parametrize("shift", [1e4, -1e4])
def test_large_bias_shift(shift):
    """Bias entries near +-1e4: no overflow or NaN (the online softmax
    subtracts the running maximum), and the result matches the oracle on the
    same fp32 inputs.  Bound: near |s| = 1e4 the base-2 logit 1.44e4 is held
    in fp32 with spacing 2^-10, so P carries a relative error up to about
    2 * 2^-10 * ln 2 ~ 1.4e-3; with |V| < 4 the output bound is 6e-3."""
    log(f"case fwd bias shift {shift}")
    d = synth.rand_core(1, 2, 96, 2, 32, "fp32", seed=11, mask="random")
    e = dict(d)
    e["bias"] = d["bias"] + shift
    out, lse = run_gpu(e)
    assert torch.isfinite(out).all()
    ref, ref_lse = run_oracle(e)
    err = np.abs(np64(out) - ref).max()
    log(f"  out max_abs={err:.3e}")
    assert err <= 6e-3
    lerr = np.abs(lse.numpy() - ref_lse).max()
    assert lerr <= 4 * 2.0 ** -10 * abs(shift) / 1e4 * 2


def test_deterministic_bitwise():
    d = synth.rand_core(1, 8, 300, 4, 32, "bf16", seed=3, mask="random")
    a, la = run_gpu(d)
    for _ in range(3):
        b, lb = run_gpu(d)
        assert torch.equal(a, b) and torch.equal(la, lb)


def test_no_lse_and_stream_ordering():
    """lse=NULL path, and a call on a side stream ordered after a producer."""
    d = synth.rand_core(1, 4, 70, 2, 32, "bf16", seed=9, mask="random")
    q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = ops.evo_attn_fwd(q, k, v, dev(d["gate"]), dev(d["mask"]),
                               dev(d["bias"]))
    torch.cuda.synchronize()
    ref, _ = run_oracle(d)
    compare("out", np64(out.cpu()), ref, "bf16")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("profile", ["ramp", "step"])
def test_logits_rising_along_keys(dtype, profile):
    """Pair bias that rises along the keys, so that later key tiles hold
    logits far above everything seen in the first one: the softmax
    reference of the kernel has to be raised tile after tile (ramp: +0.1
    per key, 32 nats over the line) or once by a large jump (step: +100
    nats from key 200 on; e^100 exceeds the fp32 range, so a reference left
    at the first tile's maximum would turn the sums into inf).  N = 320:
    five 64-key tiles, the last one ragged only through the mask."""
    log(f"case fwd rising logits {dtype} {profile}")
    N = 320
    d = synth.rand_core(1, 3, N, 2, 32, dtype, seed=77, mask="random")
    kk = torch.arange(N, dtype=torch.float32)
    add = 0.1 * kk if profile == "ramp" else 100.0 * (kk >= 200).float()
    d["bias"] = synth.round_to(d["bias"].float() + add, dtype)
    out, lse = run_gpu(d)
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    check(d, dtype)


def nan_tail(t, pad=1 << 18):
    """`t` on the GPU at the start of a larger allocation whose remaining
    elements are NaN, so that a read past the tensor's end shows up."""
    if t is None:
        return None
    buf = torch.full((t.numel() + pad,), float("nan"), dtype=t.dtype, device="cuda")
    view = buf[: t.numel()].view(t.shape)
    view.copy_(t.to("cuda"))
    return view


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_padding_keys_read_nothing_past_the_tensors(dtype):
    """Keys past N in the last key tile of the last line read zeros, not the
    memory after K and V (here NaN): N = 100 leaves 28 padding keys."""
    log(f"case fwd nan tail {dtype}")
    d = synth.rand_core(1, 3, 100, 2, 32, dtype, seed=21, mask="random")
    q, k, v, g = (nan_tail(d[n]) for n in ("q", "k", "v", "gate"))
    out, lse = ops.evo_attn_fwd(q, k, v, g, dev(d["mask"]), nan_tail(d["bias"]),
                                want_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    ref, ref_lse = run_oracle(d)
    compare("out", np64(out), ref, dtype)
    compare("lse", lse.cpu().numpy().astype(np.float64), ref_lse, dtype, stored="fp32")

"""GPU checks of evo_attn_fwd_noalloc (the forward that allocates nothing and
keeps its prepared bias in the library's static scratch) against
evo_attn_fwd with a caller workspace, through the C ABI: two calls in a row
on one GPU, the second smaller than the first (the scratch keeps the first
call's contents), each compared bit for bit with the workspace entry point
and, under the parity bar, with the fp64 oracle; and the rejection of a
problem larger than the scratch."""
import numpy as np
import pytest
import torch

import oracle.evo_oracle as O
from evoformer_attention_amd import ops, synth
from helpers import compare, dev, log, np64, npu8

pytestmark = pytest.mark.gpu


def _both(d):
    q, k, v, g, m, b = (dev(d[x]) for x in ("q", "k", "v", "gate", "mask", "bias"))
    B, R, N, H, C = q.shape
    out_ws, lse_ws = ops.evo_attn_fwd(q, k, v, g, m, b, want_lse=True)
    out_na = torch.empty_like(q)
    lse_na = torch.empty((B, R, H, N), dtype=torch.float32, device=q.device)
    ops.evo_attn_fwd_noalloc(q, k, v, g, m, b, out=out_na, lse=lse_na)
    torch.cuda.synchronize()
    return out_ws.cpu(), lse_ws.cpu(), out_na.cpu(), lse_na.cpu()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_workspace_forward_two_calls(dtype):
    for i, (B, R, N, H, mask) in enumerate([(2, 24, 300, 4, "random"),
                                            (1, 5, 130, 2, "random")]):
        log(f"case noalloc {dtype} call {i}: B={B} R={R} N={N} H={H}")
        d = synth.rand_core(B, R, N, H, 32, dtype, seed=90 + i, mask=mask,
                            mask_rows=1)
        out_ws, lse_ws, out_na, lse_na = _both(d)
        assert torch.equal(out_ws, out_na), "out differs from evo_attn_fwd"
        assert torch.equal(lse_ws, lse_na), "lse differs from evo_attn_fwd"
        ref, ref_lse = O.attention_forward(np64(d["q"]), np64(d["k"]), np64(d["v"]),
                                           np64(d["gate"]), npu8(d["mask"]),
                                           np64(d["bias"]))
        compare("out", np64(out_na), ref, dtype)
        compare("lse", lse_na.numpy().astype(np.float64), ref_lse, dtype, stored="fp32")


def test_noalloc_without_bias_or_mask_and_rejects_oversize():
    d = synth.rand_core(1, 3, 70, 2, 32, "bf16", seed=5, bias=False, mask=None)
    out_ws, lse_ws, out_na, lse_na = _both(d)
    assert torch.equal(out_ws, out_na) and torch.equal(lse_ws, lse_na)
    # bf16, H = 8, N = 1100: the prepared bias needs 8 * 1152 * 1152 * 2
    # bytes = 21 MB, above the 16 MiB scratch: rejected before any launch
    N, H = 1100, 8
    q = torch.zeros((1, 1, N, H, 32), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros((1, H, N, N), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 7.0)
    with pytest.raises(ops.EvoAttnError) as ei:
        ops.evo_attn_fwd_noalloc(q, q, q, None, None, bias, out=out)
    assert ei.value.status == ops.EVO_ENOTSUP
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call must leave out untouched"

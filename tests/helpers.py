"""Shared test utilities: tolerances, comparisons and host<->device moves.

Tolerances of the parity bar (written here, used by every GPU parity test):
  fp32 inputs:  max |gpu - oracle| <= 1e-4
  bf16 inputs (fp32 accumulation): |gpu - oracle| <= 2e-2 + 2^-8 |oracle|
                elementwise, and ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2.
The 2^-8 |oracle| term is the rounding of the stored bf16 output itself
(unit roundoff of an 8-bit significand): a value of magnitude 5 cannot be
stored closer than ~0.02, so the 2e-2 absolute bound is applied beyond the
output's own representation error.
"""
import sys

import numpy as np
import torch

FP32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
BF16_UNIT_ROUNDOFF = 2.0 ** -8


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t):
    """CPU/GPU tensor (any float dtype) or None -> float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()


def npu8(t):
    return None if t is None else t.detach().cpu().numpy()


def dev(t, device="cuda"):
    return None if t is None else t.to(device).contiguous()


def compare(name, got, ref, dtype, scale=1.0):
    """Assert the parity bar for `dtype` ("fp32"/"bf16").  `scale` widens the
    absolute bound for quantities whose natural magnitude is `scale` times
    that of the inputs (e.g. sums over many rows); it is stated where used.
    scale="peak" uses max(1, max|ref|): the bar then applies to the output
    measured in units of its own largest entry (used for dBias, a sum over
    every row of a batch, whose entries grow with the number of rows while
    its relative error stays that of one row)."""
    if isinstance(scale, str):
        r = np.asarray(ref, np.float64)
        fin_r = r[np.isfinite(r)]
        scale = max(1.0, float(np.abs(fin_r).max()) if fin_r.size else 1.0)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{name}: non-finite pattern differs"
    if np.any(~fin):
        assert np.array_equal(got[~fin], ref[~fin]), f"{name}: infinities differ"
    d = np.abs(got[fin] - ref[fin])
    max_abs = float(d.max()) if d.size else 0.0
    # excess over the output-rounding allowance (bf16 only)
    rep = BF16_UNIT_ROUNDOFF * np.abs(ref[fin]) if dtype == "bf16" else 0.0
    excess = float((d - rep).max()) if d.size else 0.0
    nrm = float(np.linalg.norm(ref[fin]))
    rel = float(np.linalg.norm(got[fin] - ref[fin]) / nrm) if nrm > 0 else max_abs
    peak = float(np.abs(ref[fin]).max()) if d.size else 0.0
    log(f"  {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} (max|ref|={peak:.3e})")
    if dtype == "fp32":
        assert max_abs <= FP32_MAX_ABS * scale, f"{name}: max_abs {max_abs:.3e}"
    else:
        assert excess <= BF16_MAX_ABS * scale, f"{name}: max_abs {max_abs:.3e} (excess {excess:.3e})"
        assert rel <= BF16_REL_L2, f"{name}: rel_l2 {rel:.3e}"
    return max_abs, rel

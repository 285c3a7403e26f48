"""Shared test utilities: tolerances, comparisons and host<->device moves.

The parity bar (written here, used by every GPU parity test), elementwise
against the fp64 oracle:
  fp32 inputs:  |gpu - oracle| <= 1e-4
  bf16 inputs (fp32 accumulation): |gpu - oracle| <= 2e-2 (+ the output's
                own storage rounding, see below) and
                ||gpu - oracle||_2 / ||oracle||_2 <= 1e-2.

Storage rounding.  An output that the library stores in bf16 cannot be
closer to the exact value than half a unit in its last place, up to
2^-8 |oracle| (8 significant bits, round to nearest even): 0.016 at 4,
0.031 at 8.  For outputs stored in bf16 that term (rounds=1) is added to
the absolute bar of each element; outputs stored in fp32 (LSE, dBias,
every parameter gradient) get nothing added.  Every output of the attention
path itself (out, LSE, dQ, dK, dV, dGate, dBias, the module's projections
and output) is held to exactly this.

The other pair operations pass their values through several bf16 tensors
in between (operands, products, hidden layers): each such rounding has
relative size at most 2^-8, and to first order they add, so an output whose
path holds `rounds` of them is allowed rounds * 2^-8 |oracle| on top of the
absolute bar (the count is stated where used, from the kernel's data flow).
Their fp32 parameter gradients, sums over all N^2 positions of such terms,
and the outputs of the multiplicative update and the outer product mean
(sums that cancel, whose error follows the size of their terms) use
scale="peak": the absolute bar times max(1, max|oracle|).

A derived worst-case bound (`bound`, elementwise, from the kernel's own
roundings) may stand in for the bar where the plain bar is below what the
algorithm can reach; it is used only where stated.

The relative L2 bar applies when the oracle's rms is at least the absolute
bar; below that the whole tensor is inside the max-abs bar's own floor
(e.g. a gradient that is zero up to rounding) and max-abs alone decides.

When EVO_PARITY_LOG names a file, every comparison appends one JSON record
(test, case, achieved max-abs and rel-L2, the bar) to it;
tests/parity_summary.py turns those records into a table.
"""
import json
import os
import sys

import numpy as np
import torch

FP32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 1e-2
STORE_ROUNDOFF = 2.0 ** -8   # half an ulp of bf16, relative


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


def _record(rec):
    path = os.environ.get("EVO_PARITY_LOG")
    if not path:
        return
    rec["test"] = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def compare(name, got, ref, dtype, scale=1.0, stored=None, rounds=None, bound=None):
    """Assert the parity bar for inputs of `dtype` ("fp32"/"bf16") on an
    output stored as `stored` ("fp32"/"bf16"; default: the input dtype).
    `scale`: 1.0 or "peak"; `rounds`: bf16 roundings on the path (default 1
    for a bf16-stored output, else 0); `bound`: optional elementwise derived
    bound (see the module docstring)."""
    stored = stored or dtype
    assert stored in ("fp32", "bf16"), stored
    if rounds is None:
        rounds = 1 if stored == "bf16" else 0
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{name}: non-finite pattern differs"
    if np.any(~fin):
        assert np.array_equal(got[~fin], ref[~fin]), f"{name}: infinities differ"
    r = ref[fin]
    d = np.abs(got[fin] - r)
    max_abs = float(d.max()) if d.size else 0.0
    nrm = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(got[fin] - r) / nrm) if nrm > 0 else 0.0
    peak = float(np.abs(r).max()) if d.size else 0.0
    rms = float(np.sqrt(np.mean(r * r))) if d.size else 0.0
    if scale == "peak":
        mult = max(1.0, peak)
    else:
        assert isinstance(scale, (int, float)), scale
        mult = float(scale)
    literal = FP32_MAX_ABS if dtype == "fp32" else BF16_MAX_ABS
    bar_abs = literal * mult
    allow = rounds * STORE_ROUNDOFF * np.abs(r)
    eff = bar_abs + allow
    if bound is not None:
        eff = np.maximum(eff, np.asarray(bound, np.float64)[fin])
    excess = float((d - allow).max()) if d.size else 0.0
    ratio = float((d / eff).max()) if d.size else 0.0
    bar_rel = None if dtype == "fp32" else BF16_REL_L2
    rel_applies = bar_rel is not None and rms >= bar_abs
    log(f"  {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e} (max|ref|={peak:.3e}; "
        f"stored {stored}, rounds {rounds}; bar {bar_abs:.1e}; worst/bar {ratio:.2f})")
    _record(dict(case=name, dtype=dtype, stored=stored, rounds=rounds, n=int(d.size),
                 max_abs=max_abs, excess=excess, ratio=ratio, rel_l2=rel, max_ref=peak,
                 rms_ref=rms, scale=str(scale), bound=bound is not None,
                 bar_abs=bar_abs, bar_rel=bar_rel if rel_applies else None,
                 literal_ok=bool(max_abs <= literal and
                                 (not rel_applies or rel <= bar_rel))))
    assert ratio <= 1.0, (f"{name}: max_abs {max_abs:.3e} (beyond rounding allowance "
                          f"{excess:.3e}) exceeds its bar (worst element at {ratio:.2f}x)")
    if rel_applies:
        assert rel <= bar_rel, f"{name}: rel_l2 {rel:.3e}"
    return max_abs, rel


def round_bf16(x):
    """Round float64 values to the nearest bf16 value (8 significant bits,
    ties to even), directly from float64, with no float32 step in between;
    returned as float64.  For the oracle's view of a tensor that crosses the
    C ABI in bf16 (the plain reading of a bf16 boundary)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0) / 256.0, e)   # np.round: ties to even

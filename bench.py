"""Benchmark of the Evoformer biased-attention hot path on one MI355X.

One step = the whole hot path over one synthetic batch, through the C ABI:
  tri_attn_project   LayerNorm + Q/K/V/gate/pair-bias projections
  evo_attn_fwd       biased gated attention forward (with LSE)
  tri_attn_out_project
  evo_attn_bwd       dQ, dK, dV, dGate and dBias (summed over rows)
on the triangle-attention ending-node workload N_res = 768, c_z = 128,
4 heads of 32, 38 residues masked, bf16 (default --workload tri_end_768).

value = attention flops per step / step time, counting 4*L*C for the
forward and 2.5x that for the backward (L = rows * heads * N^2 logits); the
projections' time is inside the step but their flops are not counted.

Prints one JSON line.  Options: --steps K --warmup W --gpus 1
--workload NAME --no-cpu-baseline --cpu-lines L --calibrate-copy
--write-traffic FETCH_CSV WRITE_CSV, and --module-train (a training step of
the whole module instead: forward, then the backward with the LayerNorm,
projection and output-projection gradients), --trimul (the triangular
multiplicative update instead), --transition (the fused LayerNorm + SwiGLU
transition instead), --transition-bwd (its backward instead) and --opm (the
outer product mean instead).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOADS_BENCH = ("tri_end_768", "tri_start_384", "tri_start_512_bwd")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="tri_end_768", choices=WORKLOADS_BENCH)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-lines", type=int, default=192,
                    help="attention lines in the oracle's timed sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain elementwise copy "
                         "of COPY_BYTES (read) + COPY_BYTES (write), for scaling "
                         "the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--module-train", action="store_true",
                    help="time a training step of the whole module instead: "
                         "tri_attn_module_fwd + tri_attn_module_bwd (LayerNorm, "
                         "projection and output-projection gradients included)")
    ap.add_argument("--trimul", action="store_true",
                    help="time the triangular multiplicative update instead "
                         "(tri_mul_fwd, outgoing edges, z [768,768,128], 128 "
                         "channels, 38 residues masked)")
    ap.add_argument("--transition", action="store_true",
                    help="time the fused LayerNorm + SwiGLU transition instead "
                         "(pair_transition_fwd, z [768,768,128], hidden 512)")
    ap.add_argument("--transition-bwd", action="store_true",
                    help="time the transition backward instead "
                         "(pair_transition_bwd, z [768,768,128], hidden 512)")
    ap.add_argument("--opm", action="store_true",
                    help="time the outer product mean instead "
                         "(outer_product_mean_fwd, m [1024,768,256], 32 "
                         "channels, out [768,768,128])")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU work: turn two rocprofv3 --pmc counter files "
                         "(FETCH_SIZE run, WRITE_SIZE run) of a --calibrate-copy "
                         "bench into profiles/traffic.json")
    return ap.parse_args()


COPY_BYTES = 1 << 29          # 512 MiB read and 512 MiB written by the copy
TRAFFIC_KERNELS = {"attn_fwd": "attn_fwd_kernel", "bwd_dkdv": "bwd_dkdv_kernel",
                   "bwd_dq": "bwd_dq_kernel", "bwd_dbias": "bwd_dbias_kernel",
                   "rowgemm": "rowgemm_kernel", "bwd_prep": "bwd_prep_kernel"}
COPY_KERNEL = "neg_kernel"    # torch.neg(out=): a plain streaming copy


def kernel_sources_digest():
    """Digest of the HIP sources; stored traffic counters are reported only
    while it matches the digest they were taken with."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "evoformer_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(workload, {}).get(kernel)
    if not ent or ent.get("sources_digest") != kernel_sources_digest():
        return None
    return ent.get("bytes_per_launch")


def _counter_means(path, counter):
    """Mean counter value per dispatch, by kernel short name."""
    import csv
    sums = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            for short, pat in list(TRAFFIC_KERNELS.items()) + [("copy", COPY_KERNEL)]:
                if pat in name:
                    break
            else:
                continue
            key = (short, row["Dispatch_Id"])
            sums[key] = sums.get(key, 0.0) + float(row["Counter_Value"])
    per = {}
    for (short, _), v in sums.items():
        per.setdefault(short, []).append(v)
    return {k: sum(v) / len(v) for k, v in per.items()}


def write_traffic(fetch_csv, write_csv, workload):
    """profiles/traffic.json from the two counter runs.  Each counter (KiB
    per dispatch) is scaled by known bytes / counter bytes of the copy kernel
    measured in the same run."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("no copy-calibration dispatch in the counter files "
                         "(run the bench with --calibrate-copy)")
    f_scale = COPY_BYTES / (fetch["copy"] * 1024.0)
    w_scale = COPY_BYTES / (write["copy"] * 1024.0)
    out = {"_method": ("FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over "
                       "dispatches) from two rocprofv3 --pmc runs of "
                       "'bench.py --steps 2 --warmup 1 --no-cpu-baseline "
                       "--calibrate-copy'; each scaled by the factor that maps "
                       "the same counter of a plain %d-byte elementwise copy to "
                       "its known size" % COPY_BYTES),
           "copy_calibration": {"fetch_kib": fetch["copy"], "write_kib": write["copy"],
                                "known_bytes": COPY_BYTES,
                                "fetch_scale": f_scale, "write_scale": w_scale}}
    ent = {}
    digest = kernel_sources_digest()
    for short in TRAFFIC_KERNELS:
        if short in fetch and short in write:
            fb = fetch[short] * 1024.0 * f_scale
            wb = write[short] * 1024.0 * w_scale
            ent[short] = {"fetch_kib": fetch[short], "write_kib": write[short],
                          "fetch_bytes": fb, "write_bytes": wb,
                          "bytes_per_launch": fb + wb, "sources_digest": digest}
    out[workload] = ent
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def cpu_baseline(d, w, n_lines):
    """The fp64 oracle on a bounded sample of the same workload: module
    forward and core backward of `n_lines` attention lines (the oracle's own
    line-wise definitions), timed on this host's cores."""
    import numpy as np
    import torch
    import oracle.evo_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = 1

    def np64(t):
        return None if t is None else t.to(torch.float64).numpy()

    N, H, C, ending = w["N"], w["H"], w["C"], w["ending"]
    args = dict(z=np64(d["z"]), residue_mask=None if d["mask"] is None else d["mask"].numpy(),
                ln_w=np64(d["ln_w"]), ln_b=np64(d["ln_b"]), eps=d["eps"],
                w_q=np64(d["w_q"]), w_k=np64(d["w_k"]), w_v=np64(d["w_v"]),
                w_g=np64(d["w_g"]), b_g=np64(d["b_g"]), w_bias=np64(d["w_bias"]),
                w_o=np64(d["w_o"]), b_o=np64(d["b_o"]), H=H, C=C)
    lines = list(range(0, N, max(1, N // n_lines)))[:n_lines]
    rng = np.random.default_rng(0)
    t0 = time.perf_counter()
    O.tri_module_lines(lines=lines, ending=ending, **args)
    q, k, v, g, bias = O.tri_project(args["z"], args["ln_w"], args["ln_b"],
                                     args["eps"], args["w_q"], args["w_k"],
                                     args["w_v"], args["w_g"], args["b_g"],
                                     args["w_bias"], H, C, ending, lines=lines)
    t1 = time.perf_counter()
    keep = None if args["residue_mask"] is None else args["residue_mask"] != 0
    for t in range(len(lines)):
        dout = rng.standard_normal((N, H, C))
        O.attention_line_backward(q[0, t], k[0, t], v[0, t], g[0, t],
                                  bias[0], keep, dout)
    t2 = time.perf_counter()
    flops = len(lines) * 14.0 * H * N * N * C
    return {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOP/s",
            "cores": int(cores), "kind": "oracle",
            "sample": (f"{len(lines)} of {N} attention lines of {w['name']}: "
                       f"line-wise module forward + core backward "
                       f"({t2 - t0:.1f} s wall, of which {t1 - t0:.1f} s forward "
                       f"including the pair bias of the whole z)")}


def module_train(a):
    """One training step of the triangle-attention module on the workload:
    the module forward, then the module backward (which recomputes the
    forward's activations from z, as an activation-checkpointed Evoformer
    block does).  Prints one JSON line; the roofline entry is the projection
    backward (tri_attn_project_bwd, HBM-bound), timed on its own."""
    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS[a.workload])
    N, CZ, H, C, ending = w["N"], w["CZ"], w["H"], w["C"], w["ending"]
    d = synth.module_inputs(a.workload)
    gen = torch.Generator().manual_seed(7)
    dout = synth.round_to(torch.randn((N, N, CZ), generator=gen), w["dtype"])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    dout = dout.to(dev)
    dt = g["z"].dtype
    ws_f = torch.empty(ops.tri_attn_workspace_bytes(dt, N, CZ, H, C), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(ops.tri_attn_bwd_workspace_bytes(dt, N, CZ, H, C), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        out = ops.tri_attn_module_fwd(
            g["z"], g["mask"], g["ln_w"], g["ln_b"], g["eps"], g["w_q"], g["w_k"],
            g["w_v"], g["w_g"], g["b_g"], g["w_bias"], g["w_o"], g["b_o"], H, C,
            ending, workspace=ws_f)
        grads = ops.tri_attn_module_bwd(
            g["z"], g["mask"], g["ln_w"], g["ln_b"], g["eps"], g["w_q"], g["w_k"],
            g["w_v"], g["w_g"], g["b_g"], g["w_bias"], g["w_o"], dout, H, C,
            ending, workspace=ws_b)
        return out, grads

    def timed(fn, iters):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    ms = timed(step, a.steps)
    # the projection backward alone, on gradients of the same shapes
    gq = [torch.randn((1, N, N, H, C), device=dev).to(dt) for _ in range(4)]
    gb = torch.randn((1, H, N, N), device=dev)
    ws_p = torch.empty(ops.tri_attn_proj_bwd_workspace_bytes(dt, N, CZ, H, C),
                       dtype=torch.uint8, device=dev)

    def pbwd():
        return ops.tri_attn_project_bwd(
            g["z"], g["ln_w"], g["ln_b"], g["eps"], g["w_q"], g["w_k"], g["w_v"],
            g["w_g"], g["w_bias"], *gq, gb, H, C, ending, workspace=ws_p)

    ms_p = timed(pbwd, a.steps)
    pbytes = M.project_bwd_min_bytes(N, CZ, H, C, 2)
    gbs = pbytes / (ms_p * 1e-3) / 1e9
    flops = M.module_step_flops(N, CZ, H, C)
    res = {
        "metric": "Triangle-attention module training step (fwd + bwd) TFLOP/s (bf16), tri-attn N_res=768",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "N_res": N, "c_z": CZ, "heads": H,
                   "head_dim": C, "node": "ending" if ending else "starting",
                   "step": "module fwd + module bwd (recomputes the forward; "
                           "dz and every parameter gradient)"},
        "roofline": {"bound": "hbm", "kernel": "tri_attn_project_bwd (call)",
                     "achieved": round(gbs, 1), "peak": M.MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / M.MI355X_HBM_GBS, 4), "traffic": None},
        "project_bwd_ms": round(ms_p, 4),
    }
    print(json.dumps(res), flush=True)


def trimul_bench(a):
    """The triangular multiplicative update on trimul_out_768.  Prints one
    JSON line; the roofline entry is the whole tri_mul_fwd call against the
    dense bf16 matrix-core peak, its flops dominated by the per-channel
    products (2 C N^3)."""
    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS["trimul_out_768"])
    N, CZ, C = w["N"], w["CZ"], w["C"]
    d = synth.trimul_inputs("trimul_out_768")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ws = torch.empty(ops.tri_mul_workspace_bytes(g["z"].dtype, N, CZ, C), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((N, N, CZ), dtype=g["z"].dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return ops.tri_mul_fwd(g["z"], g["mask"], g["ln_w"], g["ln_b"], g["eps"], g["w_a"],
                               g["w_b"], g["w_o"], g["b_o"], w["outgoing"], workspace=ws,
                               out=out)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    tf = M.trimul_flops(N, CZ, C) / (ms * 1e-3) / 1e12
    res = {
        "metric": "Triangular multiplicative update (outgoing) TFLOP/s (bf16), N_res=768, c=128",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "trimul_out_768", "N_res": N, "c_z": CZ, "channels": C,
                   "edges": "outgoing", "masked_residues": int((d["mask"] == 0).sum())},
        "roofline": {"bound": "mfma", "kernel": "tri_mul_fwd (call)", "achieved": round(tf, 2),
                     "peak": M.MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / M.MI355X_BF16_DENSE_TFLOPS, 4), "traffic": None},
    }
    print(json.dumps(res), flush=True)


def transition_bench(a):
    """The fused transition on transition_768.  Prints one JSON line; the
    roofline entry is the call (a weight-preparation kernel of ~1% plus the
    fused kernel) against the dense bf16 matrix-core peak."""
    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS["transition_768"])
    N, CZ, HID = w["N"], w["CZ"], w["HID"]
    d = synth.transition_inputs("transition_768")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ws = torch.empty(ops.pair_transition_workspace_bytes(g["z"].dtype, N, CZ, HID),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(g["z"])
    stream = torch.cuda.current_stream(dev)

    def step():
        return ops.pair_transition_fwd(g["z"], g["ln_w"], g["ln_b"], g["eps"], g["w_a"],
                                       g["w_b"], g["w_o"], out=out, workspace=ws)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    tf = M.transition_flops(N, CZ, HID) / (ms * 1e-3) / 1e12
    res = {
        "metric": "Fused LayerNorm + SwiGLU pair transition TFLOP/s (bf16), N_res=768",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "transition_768", "N_res": N, "c_z": CZ, "hidden": HID},
        "roofline": {"bound": "mfma", "kernel": "pair_transition_fwd (call)",
                     "achieved": round(tf, 2), "peak": M.MI355X_BF16_DENSE_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / M.MI355X_BF16_DENSE_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)


def transition_bwd_bench(a):
    """The transition backward on transition_768 (dz and every parameter
    gradient).  Prints one JSON line; the roofline entry is the whole call
    against the dense bf16 matrix-core peak."""
    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS["transition_768"])
    N, CZ, HID = w["N"], w["CZ"], w["HID"]
    d = synth.transition_inputs("transition_768", dout=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ws = torch.empty(ops.pair_transition_bwd_workspace_bytes(g["z"].dtype, N, CZ, HID),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return ops.pair_transition_bwd(g["z"], g["ln_w"], g["ln_b"], g["eps"], g["w_a"],
                                       g["w_b"], g["w_o"], g["dout"], workspace=ws)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    tf = M.transition_bwd_flops(N, CZ, HID) / (ms * 1e-3) / 1e12
    res = {
        "metric": "LayerNorm + SwiGLU pair transition backward TFLOP/s (bf16), N_res=768",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "transition_768", "N_res": N, "c_z": CZ, "hidden": HID,
                   "pass": "backward (dz, dln_w, dln_b, dw_a, dw_b, dw_o)"},
        "roofline": {"bound": "mfma", "kernel": "pair_transition_bwd (call)",
                     "achieved": round(tf, 2), "peak": M.MI355X_BF16_DENSE_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / M.MI355X_BF16_DENSE_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)


def opm_bench(a):
    """The outer product mean on opm_1024x768.  Prints one JSON line; the
    roofline entry is the whole call (projections, the product on the matrix
    cores, the output projection) against the dense bf16 matrix-core peak."""
    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS["opm_1024x768"])
    S, N, CM, C, CZ = w["S"], w["N"], w["CM"], w["C"], w["CZ"]
    d = synth.opm_inputs("opm_1024x768")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ws = torch.empty(ops.outer_product_mean_workspace_bytes(g["m"].dtype, S, N, CM, C, CZ),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((N, N, CZ), dtype=g["m"].dtype, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return ops.outer_product_mean_fwd(g["m"], g["ln_w"], g["ln_b"], g["eps"], g["w_a"],
                                          g["w_b"], g["w_o"], g["b_o"], out=out, workspace=ws)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    tf = M.opm_flops(S, N, CM, C, CZ) / (ms * 1e-3) / 1e12
    res = {
        "metric": "Outer product mean TFLOP/s (bf16), N_seq=1024, N_res=768",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "opm_1024x768", "N_seq": S, "N_res": N, "c_m": CM,
                   "c": C, "c_z": CZ},
        "roofline": {"bound": "mfma", "kernel": "outer_product_mean_fwd (call)",
                     "achieved": round(tf, 2), "peak": M.MI355X_BF16_DENSE_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / M.MI355X_BF16_DENSE_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(res), flush=True)


def main():
    a = parse()
    if a.transition_bwd:
        if a.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        transition_bwd_bench(a)
        return
    if a.opm:
        if a.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        opm_bench(a)
        return
    if a.transition:
        if a.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        transition_bench(a)
        return
    if a.trimul:
        if a.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        trimul_bench(a)
        return
    if a.module_train:
        if a.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        module_train(a)
        return
    if a.write_traffic:
        write_traffic(a.write_traffic[0], a.write_traffic[1], a.workload)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): this "
              "library has no multi-GPU path (no sharding, no collectives).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS[a.workload])
    w["name"] = a.workload
    N, CZ, H, C, ending = w["N"], w["CZ"], w["H"], w["C"], w["ending"]
    d = synth.module_inputs(a.workload)
    if d["dout"] is None:
        gen = torch.Generator().manual_seed(1)
        d["dout"] = synth.round_to(torch.randn((1, N, N, H, C), generator=gen), w["dtype"])
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    key_mask = g["mask"].view(1, 1, N) if g["mask"] is not None else None
    ws_bwd = torch.empty(ops.evo_attn_bwd_workspace_bytes(torch.bfloat16, 1, N, N, H, C),
                         dtype=torch.uint8, device=dev)
    ws_fwd = torch.empty(ops.evo_attn_fwd_workspace_bytes(torch.bfloat16, 1, N, N, H, C),
                         dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        q, k, v, gt, bias = ops.tri_attn_project(
            g["z"], g["ln_w"], g["ln_b"], g["eps"], g["w_q"], g["w_k"], g["w_v"],
            g["w_g"], g["b_g"], g["w_bias"], H, C, ending)
        if ev:
            ev[1].record(stream)
        o, lse = ops.evo_attn_fwd(q, k, v, gt, key_mask, bias, want_lse=True,
                                  workspace=ws_fwd)
        if ev:
            ev[2].record(stream)
        out = ops.tri_attn_out_project(o, g["w_o"], g["b_o"], CZ, ending)
        if ev:
            ev[3].record(stream)
        grads = ops.evo_attn_bwd(q, k, v, gt, key_mask, bias, o, lse, g["dout"],
                                 workspace=ws_bwd)
        if ev:
            ev[4].record(stream)
        return out, grads

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
           for _ in range(a.steps)]
    torch.cuda.reset_peak_memory_stats()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(a.steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms = total_ms / a.steps
    parts = {"project": 0.0, "attn_fwd": 0.0, "out_project": 0.0, "attn_bwd": 0.0}
    for e in evs:
        for j, name in enumerate(parts):
            parts[name] += e[j].elapsed_time(e[j + 1]) / a.steps
    peak_mem = torch.cuda.max_memory_allocated()
    if a.calibrate_copy:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    R = N
    fwd_fl = M.fwd_flops(1, R, N, H, C)
    bwd_fl = M.bwd_flops(1, R, N, H, C)
    value = (fwd_fl + bwd_fl) / (ms * 1e-3) / 1e12
    fwd_tf = fwd_fl / (parts["attn_fwd"] * 1e-3) / 1e12
    bwd_tf = bwd_fl / (parts["attn_bwd"] * 1e-3) / 1e12
    # Dominant kernel of the step: the attention forward (one kernel per
    # call, so its event pair brackets exactly one launch).
    traffic = stored_traffic("attn_fwd", a.workload)
    roof = {"bound": "mfma", "kernel": "attn_fwd_kernel", "achieved": round(fwd_tf, 2),
            "peak": M.MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
            "frac": round(fwd_tf / M.MI355X_BF16_DENSE_TFLOPS, 4),
            "traffic": traffic}
    res = {
        "metric": "EvoAttention fwd/bwd TFLOP/s (bf16) and % MFMA peak, tri-attn N_res=768",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a.workload, "N_res": N, "c_z": CZ, "heads": H,
                   "head_dim": C, "node": "ending" if ending else "starting",
                   "masked_residues": int((d["mask"] == 0).sum()) if d["mask"] is not None else 0,
                   "step": "project + attn fwd + out project + attn bwd (dQ,dK,dV,dGate,dBias)"},
        "roofline": roof,
        "breakdown_ms": {k: round(v, 4) for k, v in parts.items()},
        "attn_fwd_tflops": round(fwd_tf, 2), "attn_bwd_tflops": round(bwd_tf, 2),
        "attn_fwd_mfma_frac": round(fwd_tf / M.MI355X_BF16_DENSE_TFLOPS, 4),
        "peak_mem_gb": round(peak_mem / 1e9, 3),
        "logits_avoided_gb": round(M.triangle_logit_bytes(N, H, 2) / 1e9, 3),
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(d, w, a.cpu_lines)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the Evoformer biased-attention hot path on one MI355X.

Default (--workload tri_end_768): one step = the whole hot path over one
synthetic batch, through the C ABI:
  tri_attn_project   LayerNorm + Q/K/V/gate/pair-bias projections
  evo_attn_fwd       biased gated attention forward (with LSE)
  tri_attn_out_project
  evo_attn_bwd       dQ, dK, dV, dGate and dBias (summed over rows)
on the triangle-attention ending-node workload N_res = 768, c_z = 128,
4 heads of 32, 38 residues masked, bf16.

value = attention flops per step / step time, counting 4*L*C for the
forward and 2.5x that for the backward (L = rows * heads * N^2 logits); the
projections' time is inside the step but their flops are not counted.

The other workloads of the configuration set (--workload NAME, or --all for
all five lines):
  core_fp32_small    evo_attn_fwd, fp32, 32 lines of 32 keys, 4 heads
  msa_row_bf16       evo_attn_fwd, MSA row attention: 128 rows x 256
                     residues, 8 heads, 26 keys masked (HBM roofline)
  tri_start_384      tri_attn_module_fwd, starting node, z [384,384,128]
  tri_start_512_bwd  tri_attn_project + evo_attn_fwd + evo_attn_bwd, starting
                     node, z [512,512,128]
Each line carries the roofline of its dominant kernel or call, the step
time's median / p10 / p90 over the timed steps (warm) and over the same
number of steps with a 1 GiB write between steps (cold cache, outside the
timed region), the softmax ceiling measured with the library's issue-rate
probe, and the fp64 oracle's time on a bounded sample of the same workload
on this host's cores.

Prints one JSON line per workload.  Options: --steps K --warmup W --gpus 1
--workload NAME --all --no-cpu-baseline --cpu-lines L --calibrate-copy
--write-traffic FETCH_CSV WRITE_CSV, --write-counters CSV..., and
--module-train (a training step of the whole module instead), --trimul
(the triangular multiplicative update), --trimul-bwd (its backward),
--transition (the fused LayerNorm +
SwiGLU transition), --transition-bwd (its backward), --opm (the outer
product mean) and --opm-bwd (its backward).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOADS_BENCH = ("tri_end_768", "core_fp32_small", "msa_row_bf16", "tri_start_384",
                   "tri_start_512_bwd")
COLD_BYTES = 1 << 30          # written between steps for the cold-cache timing


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="tri_end_768", choices=WORKLOADS_BENCH)
    ap.add_argument("--all", action="store_true",
                    help="one line for every workload of the configuration set")
    ap.add_argument("--write-counters", nargs="+", metavar="CSV",
                    help="no GPU work: per-kernel summaries of rocprofv3 --pmc "
                         "counter files of the default workload, written to "
                         "profiles/<kernel>_tri_end_768_counters.md")
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
    ap.add_argument("--trimul-bwd", action="store_true",
                    help="time the multiplicative update's backward instead "
                         "(tri_mul_bwd, the same workload, every gradient)")
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
    ap.add_argument("--opm-bwd", action="store_true",
                    help="time the outer product mean's backward instead "
                         "(outer_product_mean_bwd, the same workload, every gradient)")
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


# The sources that define and launch the kernels whose counters are stored
# (attention forward and backward, the projection row-GEMM, their shared
# device helpers).
DIGEST_SOURCES = ("attn_fwd.hip", "attn_bwd.hip", "tri_project.hip", "evo_device.h")


def kernel_sources_digest():
    """Digest of the measured kernels' sources; stored traffic counters are
    reported only while it matches the digest they were taken with."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "evoformer_attention_amd", "csrc")
    for name in DIGEST_SOURCES:
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


def host_info():
    """(CPUs this process may run on, CPU model, BLAS thread-pool size)."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count() or 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    return nproc, model, blas


def cpu_baseline(name, w, d, n_lines):
    """The fp64 oracle on a bounded sample of the same workload, timed on
    this host's cores: core workloads run their attention lines (all of them
    for the small fp32 one, n_lines of the MSA one); module workloads the
    oracle's line-wise module forward (with the pair bias of the whole z) and,
    where the step has one, the core backward of each sampled line.  The
    matrix products use the BLAS thread pool; everything else one thread."""
    import numpy as np
    import torch
    import oracle.evo_oracle as O
    nproc, model, blas = host_info()

    def np64(t):
        return None if t is None else t.to(torch.float64).numpy()

    N, H, C = w["N"], w["H"], w["C"]
    rng = np.random.default_rng(0)
    t0 = time.perf_counter()
    if w["kind"] == "core":
        R = w["R"]
        rows = list(range(R)) if R <= n_lines else list(range(0, R, R // n_lines))[:n_lines]
        mask = None if d["mask"] is None else d["mask"].numpy()
        bias = None if d["bias"] is None else np64(d["bias"][0])
        keep = None if mask is None else mask[0, 0] != 0

        def run_lines(seconds):
            """Repeat the sampled lines for at least `seconds` (a workload
            this small is repeated for a stable time); (reps, elapsed s)."""
            reps, ts = 0, time.perf_counter()
            while True:
                for r in rows:
                    O.attention_line_forward(np64(d["q"][0, r]), np64(d["k"][0, r]),
                                             np64(d["v"][0, r]), np64(d["gate"][0, r]),
                                             bias, keep)
                reps += 1
                if time.perf_counter() - ts > seconds:
                    return reps, time.perf_counter() - ts
        reps, _ = run_lines(2.0)
        t1 = t2 = time.perf_counter()
        flops = reps * len(rows) * 4.0 * H * N * N * C
        what = (f"{len(rows)} of {R} attention lines of {name}: forward"
                + (f", {reps} times" if reps > 1 else ""))
        # the same lines with the BLAS pool held to one thread: a per-core figure
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                reps1, dt1 = run_lines(1.0)
            single = reps1 * len(rows) * 4.0 * H * N * N * C / dt1 / 1e12
        except Exception:  # noqa: BLE001
            single = None
    else:
        ending = w.get("ending", False)
        args = dict(z=np64(d["z"]),
                    residue_mask=None if d["mask"] is None else d["mask"].numpy(),
                    ln_w=np64(d["ln_w"]), ln_b=np64(d["ln_b"]), eps=d["eps"],
                    w_q=np64(d["w_q"]), w_k=np64(d["w_k"]), w_v=np64(d["w_v"]),
                    w_g=np64(d["w_g"]), b_g=np64(d["b_g"]), w_bias=np64(d["w_bias"]),
                    w_o=np64(d["w_o"]), b_o=np64(d["b_o"]), H=H, C=C)
        lines = list(range(0, N, max(1, N // n_lines)))[:n_lines]
        O.tri_module_lines(lines=lines, ending=ending, **args)
        t1 = time.perf_counter()
        backward = name != "tri_start_384"
        if backward:
            q, k, v, g, bias = O.tri_project(args["z"], args["ln_w"], args["ln_b"],
                                             args["eps"], args["w_q"], args["w_k"],
                                             args["w_v"], args["w_g"], args["b_g"],
                                             args["w_bias"], H, C, ending, lines=lines)
            keep = None if args["residue_mask"] is None else args["residue_mask"] != 0
            for t in range(len(lines)):
                dout = rng.standard_normal((N, H, C))
                O.attention_line_backward(q[0, t], k[0, t], v[0, t], g[0, t],
                                          bias[0], keep, dout)
        t2 = time.perf_counter()
        flops = len(lines) * (14.0 if backward else 4.0) * H * N * N * C
        what = (f"{len(lines)} of {N} attention lines of {name}: line-wise module forward"
                + (" + core backward" if backward else "")
                + f" ({t1 - t0:.1f} s forward including the pair bias of the whole z)")
    out = {"value": flops / (t2 - t0) / 1e12, "unit": "TFLOP/s",
           "cores": int(blas), "kind": "oracle",
           "sample": f"{what}; {t2 - t0:.1f} s wall",
           "host_cpus": int(nproc), "cpu_model": model}
    if w["kind"] == "core" and single is not None:
        out["single_thread_value"] = single
    return out


def stats(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median_ms": round(float(np.median(a)), 4),
            "p10_ms": round(float(np.percentile(a, 10)), 4),
            "p90_ms": round(float(np.percentile(a, 90)), 4)}


def time_steps(step, steps, warmup, stream, dev):
    """Run `warmup` untimed steps, then exactly `steps` steps bracketed by a
    synchronisation on both sides (ms per step from one event pair around
    them, per-step times from events between them), then the same number of
    steps each preceded by a 1 GiB write that evicts L2 and the last-level
    cache (outside the timed steps).  Returns (ms_per_step, warm stats, cold
    stats)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    warm = [e0.elapsed_time(e1) for e0, e1 in ev]
    junk = torch.empty(COLD_BYTES, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(steps):
        junk.fill_(i & 255)
        torch.cuda.synchronize()
        e0, e1 = ev[i]
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del junk
    return total / steps, stats(warm), stats(cold)


def softmax_ceiling(dev):
    """Issue intervals of v_exp_f32 and v_fma_f32 relative to the bf16 MFMA
    (16 clocks per v_mfma_f32_16x16x32_bf16 and SIMD at the dense peak), from
    the library's probe, and the fraction of the matrix-core peak they leave
    the forward: per 256 logits the forward issues 2 counted MFMAs (32 clocks
    at peak) plus half a row-sum MFMA (8 clocks), 4 exp wave-instructions and
    6 other VALU ones (the bias fma and the bf16 packing).  exp_only assumes
    the exps overlap the MFMAs fully, fwd_valu the whole VALU mix, fwd_serial
    none of it; each is the counted MFMA time over the busier unit's."""
    import torch
    from evoformer_attention_amd import ops
    waves, iters = 8, 4096
    out = torch.empty(65536 * waves, dtype=torch.float32, device=dev)
    t = {}
    for kind in (0, 1, 2):
        ops.evo_probe_issue_rate(kind, waves, 64, out)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        ops.evo_probe_issue_rate(kind, waves, iters, out)
        e1.record()
        torch.cuda.synchronize()
        t[kind] = e0.elapsed_time(e1) / (waves * iters * 8)
    c_exp = 16.0 * t[0] / t[2]
    c_fma = 16.0 * t[1] / t[2]
    valu = 4 * c_exp + 6 * c_fma
    mfma = 32.0 + 8.0
    return {"exp_clocks": round(c_exp, 2), "fma_clocks": round(c_fma, 2),
            "mfma_clocks": 16.0,
            "exp_only": round(32.0 / max(mfma, 4 * c_exp), 3),
            "fwd_valu": round(32.0 / max(mfma, valu), 3),
            "fwd_serial": round(32.0 / (mfma + valu), 3),
            "method": "evo_probe_issue_rate, 8 waves per SIMD; clocks relative to "
                      "the MFMA interval (16 at the dense peak)"}


COUNTER_KERNELS = ("attn_fwd_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel", "bwd_dbias_kernel")


def write_counters(csvs):
    """profiles/<kernel>_tri_end_768_counters.md from rocprofv3 --pmc CSVs of
    the default workload: per-dispatch means of every counter and the
    derived figures (per-SIMD normalisation over 256 CUs x 4 SIMDs, the
    clock from GRBM_GUI_ACTIVE summed over 8 XCDs)."""
    import csv
    per = {k: {} for k in COUNTER_KERNELS}
    dur = {k: [] for k in COUNTER_KERNELS}
    for path in csvs:
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                for k in COUNTER_KERNELS:
                    if k in row["Kernel_Name"]:
                        per[k].setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                        dur[k].append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
                        break
    for k, cnt in per.items():
        if not cnt:
            continue
        m = {c: sum(v) / len(v) for c, v in cnt.items()}
        lines = [f"# {k}: rocprofv3 counters, tri_end_768 (bf16, N_res = 768, 4 heads of 32)", "",
                 "Commands (each a separate run of the default bench step):", ""]
        lines += [f"    cd /tmp && TMPDIR=/tmp timeout -s KILL 90 rocprofv3 --pmc {g} -d <dir> "
                  f"-o pmc --output-format csv -- python3 {ROOT}/bench.py --steps 2 --warmup 1 "
                  f"--no-cpu-baseline" for g in COUNTER_GROUPS]
        lines += ["", "| counter | mean per dispatch |", "|---|---|"]
        lines += [f"| {c} | {v:.4g} |" for c, v in sorted(m.items())]
        simd = 256 * 4
        d = {}
        if "GRBM_GUI_ACTIVE" in m:
            cyc = m["GRBM_GUI_ACTIVE"] / 8
            d["kernel clocks (GRBM_GUI_ACTIVE / 8 XCDs)"] = f"{cyc:.4g}"
            ns = sum(dur[k]) / len(dur[k])
            d["dispatch duration (ns, from the trace timestamps)"] = f"{ns:.4g}"
            d["clock (GHz)"] = f"{cyc / ns:.3f}"
            simd_cyc = cyc * simd
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                d["MFMA busy (% of SIMD-clocks)"] = f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cyc:.1f}"
            if "SQ_ACTIVE_INST_VALU" in m:
                d["VALU busy (% of SIMD-clocks; counter in quad-clocks)"] = \
                    f"{100 * 4 * m['SQ_ACTIVE_INST_VALU'] / simd_cyc:.1f}"
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in m and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                d["MFMA clocks with a VALU op in flight (% of MFMA busy)"] = \
                    f"{100 * m['SQ_VALU_MFMA_COEXEC_CYCLES'] / m['SQ_VALU_MFMA_BUSY_CYCLES']:.1f}"
        if "SQ_INSTS_VALU" in m and "SQ_INSTS_MFMA" in m and m["SQ_INSTS_MFMA"]:
            d["VALU instructions per MFMA (excluding the MFMAs)"] = \
                f"{(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / m['SQ_INSTS_MFMA']:.2f}"
        if "SQ_INSTS_VALU_TRANS_F32" in m and "SQ_INSTS_MFMA" in m and m["SQ_INSTS_MFMA"]:
            d["transcendental instructions per MFMA"] = \
                f"{m['SQ_INSTS_VALU_TRANS_F32'] / m['SQ_INSTS_MFMA']:.2f}"
        if "SQ_WAIT_ANY" in m and "SQ_WAVE_CYCLES" in m:
            d["wave time waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES, %)"] = \
                f"{100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.1f}"
        if "SQ_LDS_BANK_CONFLICT" in m and "SQ_INSTS_LDS" in m and m["SQ_INSTS_LDS"]:
            d["LDS bank-conflict clocks per LDS instruction"] = \
                f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_INSTS_LDS']:.2f}"
        if "SQ_WAVE_CYCLES" in m and "GRBM_GUI_ACTIVE" in m:
            d["mean resident waves per SIMD (4 x SQ_WAVE_CYCLES, in quad-clocks, / kernel clocks / 1024 SIMDs)"] = \
                f"{4 * m['SQ_WAVE_CYCLES'] / (m['GRBM_GUI_ACTIVE'] / 8 * simd):.2f}"
        traffic = stored_traffic({"attn_fwd_kernel": "attn_fwd", "bwd_dkdv_kernel": "bwd_dkdv",
                                  "bwd_dq_kernel": "bwd_dq", "bwd_dbias_kernel": "bwd_dbias"}[k],
                                 "tri_end_768")
        if traffic is not None:
            d["HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated; profiles/traffic.json)"] = \
                f"{traffic:.4g}"
        lines += ["", "| derived | value |", "|---|---|"]
        lines += [f"| {a} | {b} |" for a, b in d.items()]
        lines += ["", f"Sources digest: {kernel_sources_digest()}"]
        path = os.path.join(ROOT, "profiles", f"{k}_tri_end_768_counters.md")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(path)


COUNTER_GROUPS = (
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAVE_CYCLES "
    "SQ_WAIT_ANY SQ_WAVES SQ_BUSY_CYCLES",
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU "
    "SQ_INSTS_VALU_TRANS_F32 SQ_BUSY_CU_CYCLES SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS "
    "SQ_ACTIVE_INST_VMEM GRBM_GUI_ACTIVE",
)


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


def trimul_bwd_bench(a):
    """The multiplicative update's backward on trimul_out_768 (dz and every
    parameter gradient).  Prints one JSON line; the roofline entry is the
    whole call against the dense bf16 matrix-core peak, with the gradient
    flops counted (the recomputed forward is not)."""
    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS["trimul_out_768"])
    N, CZ, C = w["N"], w["CZ"], w["C"]
    d = synth.trimul_inputs("trimul_out_768", dout=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ws = torch.empty(ops.tri_mul_bwd_workspace_bytes(g["z"].dtype, N, CZ, C),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return ops.tri_mul_bwd(g["z"], g["mask"], g["ln_w"], g["ln_b"], g["eps"], g["w_a"],
                               g["w_b"], g["w_o"], g["dout"], w["outgoing"], workspace=ws)

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
    tf = M.trimul_bwd_flops(N, CZ, C) / (ms * 1e-3) / 1e12
    res = {
        "metric": "Triangular multiplicative update (outgoing) backward TFLOP/s (bf16), "
                  "N_res=768, c=128",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "trimul_out_768", "N_res": N, "c_z": CZ, "channels": C,
                   "edges": "outgoing", "masked_residues": int((d["mask"] == 0).sum()),
                   "pass": "backward (dz, dln_w, dln_b, dw_a, dw_b, dw_o, db_o)"},
        "roofline": {"bound": "mfma", "kernel": "tri_mul_bwd (call)", "achieved": round(tf, 2),
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


def opm_bwd_bench(a):
    """The outer product mean's backward on opm_1024x768 (dm and every
    parameter gradient).  Prints one JSON line; the roofline entry is the
    whole call against the dense bf16 matrix-core peak, with the gradient
    flops counted (the recomputed forward is not)."""
    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS["opm_1024x768"])
    S, N, CM, C, CZ = w["S"], w["N"], w["CM"], w["C"], w["CZ"]
    d = synth.opm_inputs("opm_1024x768", dout=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    ws = torch.empty(ops.outer_product_mean_bwd_workspace_bytes(g["m"].dtype, S, N, CM, C, CZ),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        return ops.outer_product_mean_bwd(g["m"], g["ln_w"], g["ln_b"], g["eps"], g["w_a"],
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
    tf = M.opm_bwd_flops(S, N, CM, C, CZ) / (ms * 1e-3) / 1e12
    res = {
        "metric": "Outer product mean backward TFLOP/s (bf16), N_seq=1024, N_res=768",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "opm_1024x768", "N_seq": S, "N_res": N, "c_m": CM,
                   "channels": C, "c_z": CZ,
                   "pass": "backward (dm, dln_w, dln_b, dw_a, dw_b, dw_o, db_o)"},
        "roofline": {"bound": "mfma", "kernel": "outer_product_mean_bwd (call)",
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


def mean_ms(fn, iters, warmup, stream):
    """Mean time of `fn` over `iters` back-to-back calls (one event pair)."""
    import torch
    for _ in range(warmup):
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


def roofline(kernel, flops, nbytes, ms, peak_tflops, bound=None, traffic=None):
    """Roofline entry of one timed kernel or call: its algorithmic flops and
    HBM bytes against the dense matrix-core peak of its dtype and 8 TB/s.
    The bound is the larger of the two lower limits on its time unless the
    metric fixes it; both fractions are reported."""
    from evoformer_attention_amd import metrics as M
    s = ms * 1e-3
    t_f = flops / (peak_tflops * 1e12)
    t_b = nbytes / (M.MI355X_HBM_GBS * 1e9)
    bound = bound or ("mfma" if t_f >= t_b else "hbm")
    tf = flops / s / 1e12
    gbs = nbytes / s / 1e9
    if bound == "mfma":
        ach, peak, unit = tf, peak_tflops, "TFLOP/s"
    else:
        ach, peak, unit = gbs, M.MI355X_HBM_GBS, "GB/s"
    return {"bound": bound, "kernel": kernel, "achieved": round(ach, 2), "peak": peak,
            "unit": unit, "frac": round(ach / peak, 4), "traffic": traffic,
            "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
            "launch_ms": round(ms, 4),
            "mfma_frac": round(tf / peak_tflops, 4),
            "hbm_frac": round(gbs / M.MI355X_HBM_GBS, 4)}


METRIC = "EvoAttention fwd/bwd TFLOP/s (bf16) and % MFMA peak, tri-attn N_res=768"


def attention_bench(a, name, ceiling):
    """One JSON line for one workload of the configuration set."""
    import torch
    from evoformer_attention_amd import metrics as M
    from evoformer_attention_amd import ops, synth

    w = dict(synth.WORKLOADS[name])
    w["name"] = name
    N, H, C = w["N"], w["H"], w["C"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    dt = torch.float32 if w["dtype"] == "fp32" else torch.bfloat16
    esz = 4 if w["dtype"] == "fp32" else 2
    peak = M.MI355X_FP32_MFMA_TFLOPS if w["dtype"] == "fp32" else M.MI355X_BF16_DENSE_TFLOPS
    extra = {}

    def dev_dict(d):
        return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}

    if w["kind"] == "core":
        d = synth.core_inputs(name)
        g = dev_dict(d)
        B, R = w["B"], w["R"]
        ws = torch.empty(ops.evo_attn_fwd_workspace_bytes(dt, B, R, N, H, C),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(g["q"])

        def step():
            return ops.evo_attn_fwd(g["q"], g["k"], g["v"], g["gate"], g["mask"], g["bias"],
                                    out=out, workspace=ws)

        ms, warm, cold = time_steps(step, a.steps, a.warmup, stream, dev)
        flops = M.fwd_flops(B, R, N, H, C)
        nbytes = M.fwd_min_bytes(B, R, N, H, C, esz,
                                 mask_rows=0 if d["mask"] is None else 1)
        roof = roofline("evo_attn_fwd (call: bias preparation + attn_fwd_kernel)",
                        flops, nbytes, warm["median_ms"], peak)
        masked = 0 if d["mask"] is None else int((d["mask"][0, 0] == 0).sum())
        config = {"workload": name, "batch": B, "rows": R, "N": N, "heads": H, "head_dim": C,
                  "masked_keys": masked, "gate": True, "bias": True,
                  "step": "evo_attn_fwd (no LSE)"}
        cpu_lines = R
        value = flops / (ms * 1e-3) / 1e12
    else:
        d = synth.module_inputs(name)
        CZ, ending = w["CZ"], w["ending"]
        g = dev_dict(d)
        key_mask = g["mask"].view(1, 1, N) if g["mask"] is not None else None
        masked = int((d["mask"] == 0).sum()) if d["mask"] is not None else 0
        config = {"workload": name, "N_res": N, "c_z": CZ, "heads": H, "head_dim": C,
                  "node": "ending" if ending else "starting", "masked_residues": masked}
        ws_fwd = torch.empty(ops.evo_attn_fwd_workspace_bytes(dt, 1, N, N, H, C),
                             dtype=torch.uint8, device=dev)
        fwd_fl = M.fwd_flops(1, N, N, H, C)
        bwd_fl = M.bwd_flops(1, N, N, H, C)
        mrows = 0 if key_mask is None else 1

        def project():
            return ops.tri_attn_project(g["z"], g["ln_w"], g["ln_b"], g["eps"], g["w_q"],
                                        g["w_k"], g["w_v"], g["w_g"], g["b_g"], g["w_bias"],
                                        H, C, ending)

        if name == "tri_start_384":
            ws_m = torch.empty(ops.tri_attn_workspace_bytes(dt, N, CZ, H, C),
                               dtype=torch.uint8, device=dev)
            out = torch.empty((N, N, CZ), dtype=dt, device=dev)

            def step():
                return ops.tri_attn_module_fwd(
                    g["z"], g["mask"], g["ln_w"], g["ln_b"], g["eps"], g["w_q"], g["w_k"],
                    g["w_v"], g["w_g"], g["b_g"], g["w_bias"], g["w_o"], g["b_o"], H, C,
                    ending, workspace=ws_m, out=out)

            ms, warm, cold = time_steps(step, a.steps, a.warmup, stream, dev)
            q, k, v, gt, bias = project()
            o = torch.empty_like(q)
            ms_f = mean_ms(lambda: ops.evo_attn_fwd(q, k, v, gt, key_mask, bias, out=o,
                                                    workspace=ws_fwd),
                           a.steps, a.warmup, stream)
            roof = roofline("evo_attn_fwd (call: bias preparation + attn_fwd_kernel), "
                            "on the module's projected tensors",
                            fwd_fl, M.fwd_min_bytes(1, N, N, H, C, esz, mask_rows=mrows),
                            ms_f, peak)
            value = fwd_fl / (ms * 1e-3) / 1e12
            mod_fl = fwd_fl + M.project_flops(N, CZ, H, C) + M.out_project_flops(N, CZ, H, C)
            extra["module_tflops"] = round(mod_fl / (ms * 1e-3) / 1e12, 2)
            extra["attn_fwd_ms"] = round(ms_f, 4)
            cpu_lines = N
            config["step"] = ("tri_attn_module_fwd (LayerNorm, projections, attention, "
                              "output projection)")
        else:
            if d["dout"] is None:
                gen = torch.Generator().manual_seed(1)
                d["dout"] = synth.round_to(torch.randn((1, N, N, H, C), generator=gen),
                                           w["dtype"])
                g["dout"] = d["dout"].to(dev)
            ws_bwd = torch.empty(ops.evo_attn_bwd_workspace_bytes(dt, 1, N, N, H, C),
                                 dtype=torch.uint8, device=dev)
            with_out = name == "tri_end_768"
            names = (["project", "attn_fwd"] + (["out_project"] if with_out else [])
                     + ["attn_bwd"])

            def step(ev=None):
                marks = iter(ev or ())

                def mark():
                    if ev:
                        next(marks).record(stream)
                mark()
                q, k, v, gt, bias = project()
                mark()
                o, lse = ops.evo_attn_fwd(q, k, v, gt, key_mask, bias, want_lse=True,
                                          workspace=ws_fwd)
                mark()
                out = None
                if with_out:
                    out = ops.tri_attn_out_project(o, g["w_o"], g["b_o"], CZ, ending)
                    mark()
                grads = ops.evo_attn_bwd(q, k, v, gt, key_mask, bias, o, lse, g["dout"],
                                         workspace=ws_bwd)
                mark()
                return out, grads

            ms, warm, cold = time_steps(step, a.steps, a.warmup, stream, dev)
            # per-call breakdown in a second pass, events between the calls
            # (the peak memory of these steps: the cold-cache write is freed)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                   for _ in range(a.steps)]
            torch.cuda.synchronize()
            torch.cuda.reset_peak_memory_stats()
            for e in evs:
                step(e)
            torch.cuda.synchronize()
            parts = {}
            for j, pn in enumerate(names):
                vals = sorted(e[j].elapsed_time(e[j + 1]) for e in evs)
                parts[pn] = vals[len(vals) // 2]
            value = (fwd_fl + bwd_fl) / (ms * 1e-3) / 1e12
            fwd_tf = fwd_fl / (parts["attn_fwd"] * 1e-3) / 1e12
            bwd_tf = bwd_fl / (parts["attn_bwd"] * 1e-3) / 1e12
            extra["breakdown_ms"] = {k: round(v, 4) for k, v in parts.items()}
            extra["attn_fwd_tflops"] = round(fwd_tf, 2)
            extra["attn_bwd_tflops"] = round(bwd_tf, 2)
            extra["attn_fwd_mfma_frac"] = round(fwd_tf / peak, 4)
            extra["peak_mem_gb"] = round(torch.cuda.max_memory_allocated() / 1e9, 3)
            extra["logits_avoided_gb"] = round(M.triangle_logit_bytes(N, H, 2) / 1e9, 3)
            if with_out:
                # The metric is a matrix-core fraction: the forward kernel
                # against the bf16 peak (the event pair around evo_attn_fwd
                # also holds the bias preparation, about 1% of it).
                roof = roofline("attn_fwd_kernel", fwd_fl,
                                M.fwd_min_bytes(1, N, N, H, C, esz, lse=True, mask_rows=mrows),
                                parts["attn_fwd"], peak, bound="mfma",
                                traffic=stored_traffic("attn_fwd", name))
                config["step"] = ("project + attn fwd + out project + attn bwd "
                                  "(dQ,dK,dV,dGate,dBias)")
            else:
                roof = roofline("evo_attn_bwd (call: bwd_prep, bwd_dkdv, bwd_dq, bwd_dbias)",
                                bwd_fl, M.bwd_min_bytes(1, N, N, H, C, esz, mask_rows=mrows),
                                parts["attn_bwd"], peak)
                extra["attn_fwd_roofline"] = roofline(
                    "attn_fwd_kernel", fwd_fl,
                    M.fwd_min_bytes(1, N, N, H, C, esz, lse=True, mask_rows=mrows),
                    parts["attn_fwd"], peak)
                config["step"] = ("project + attn fwd + attn bwd (dQ,dK,dV,dGate and dBias "
                                  "summed over rows)")
        if name != "tri_start_384":
            cpu_lines = a.cpu_lines
    if a.calibrate_copy and name == "tri_end_768":
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    res = {"metric": METRIC if name == "tri_end_768" else
           f"EvoAttention TFLOP/s ({w['dtype']}), {name}",
           "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32" if w["dtype"] == "fp32" else "bf16", "data": "synthetic",
           "config": config, "roofline": roof,
           "step_ms_warm": warm, "step_ms_cold": cold,
           "exp_ceiling": ceiling}
    res.update(extra)
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(name, w, d, cpu_lines)
    print(json.dumps(res), flush=True)


def main():
    a = parse()
    if a.write_traffic:
        write_traffic(a.write_traffic[0], a.write_traffic[1], a.workload)
        return
    if a.write_counters:
        write_counters(a.write_counters)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): this "
              "library has no multi-GPU path (no sharding, no collectives).",
              file=sys.stderr)
        sys.exit(2)
    for flag, fn in (("transition_bwd", transition_bwd_bench), ("opm_bwd", opm_bwd_bench),
                     ("opm", opm_bench),
                     ("transition", transition_bench), ("trimul_bwd", trimul_bwd_bench),
                     ("trimul", trimul_bench),
                     ("module_train", module_train)):
        if getattr(a, flag):
            fn(a)
            return
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ceiling = softmax_ceiling(dev)
    for name in (WORKLOADS_BENCH if a.all else (a.workload,)):
        attention_bench(a, name, ceiling)


if __name__ == "__main__":
    main()

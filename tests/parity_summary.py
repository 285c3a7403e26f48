"""Turn the parity records of a GPU test run into a Markdown table.

    EVO_PARITY_LOG=gpurun_out/parity.jsonl python -m pytest tests -m gpu ...
    python tests/parity_summary.py gpurun_out/parity.jsonl profiles/parity_summary.md

Each record is one comparison made by helpers.compare: the achieved max-abs
and relative-L2 error of a GPU output against the fp64 oracle, and the bar
it was held to.  The table lists the five workload configurations first,
then every test with its worst case per output name.
"""
import collections
import json
import sys

CONFIGS = [
    ("C1 core_fp32_small (fp32 fwd)", "test_core_fp32_small_workload"),
    ("C2 msa_row_bf16 (fwd, sampled rows)", "test_msa_row_bf16_workload_sampled_rows"),
    ("C3 tri_start_384 (module fwd, sampled lines)", "test_tri_start_384_sampled_lines"),
    ("C4 tri_end_768 (module fwd, sampled lines)", "test_tri_end_768_sampled_lines"),
    ("C5 tri_start_512_bwd (project + fwd + bwd, sampled)", "test_tri_start_512_fwd_bwd_sampled"),
]


def _short(test):
    return test.split("::")[-1] if "::" in test else test


def _name(case):
    """Output name of a case label ("dq[255]" -> "dq", "out[0,1]" -> "out")."""
    for sep in ("[", " line ", " rows"):
        if sep in case:
            return case.split(sep)[0]
    return case


def main(src, dst):
    recs = [json.loads(l) for l in open(src) if l.strip()]
    by_test = collections.OrderedDict()
    for r in recs:
        by_test.setdefault(r["test"], []).append(r)
    lines = ["# Parity of the GPU path against the fp64 oracle", "",
             f"Source: `{src}` ({len(recs)} comparisons). Bars: fp32 max-abs 1e-4; bf16 "
             "max-abs 2e-2 and rel-L2 1e-2. For outputs stored in bf16 the bar applies "
             "beyond the output's own storage rounding (2^-8 |oracle|; `beyond` column); "
             "fp32-stored outputs (LSE, dBias, parameter gradients) get no such term. "
             "`peak` = bar x max(1, max|oracle|), used only for fp32 parameter gradients "
             "of the other pair operations. `plain bar` says whether max-abs <= 2e-2 "
             "(1e-4 fp32) holds outright.", "",
             "## The five workload configurations", "",
             "| config | output | dtype | stored | max-abs | beyond | rel-L2 | max abs(ref) | bar | plain bar |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for label, test in CONFIGS:
        rs = [r for t, v in by_test.items() if _short(t) == test for r in v]
        if not rs:
            lines.append(f"| {label} | (not run) | | | | | | | | |")
            continue
        worst = collections.OrderedDict()
        for r in rs:
            k = _name(r["case"])
            if k not in worst or r["max_abs"] > worst[k]["max_abs"]:
                worst[k] = r
        for k, r in worst.items():
            rel = max(x["rel_l2"] for x in rs if _name(x["case"]) == k)
            exc = max(x["excess"] for x in rs if _name(x["case"]) == k)
            lines.append(f"| {label} | {k} | {r['dtype']} | {r['stored']} | {r['max_abs']:.2e} | "
                         f"{exc:.2e} | {rel:.2e} | {r['max_ref']:.2e} | {r['bar_abs']:.1e} | "
                         f"{'yes' if r['literal_ok'] else 'no'} |")
    lines += ["", "## Every test function (worst case per output over its parametrised cases)", "",
              "| test | output | dtype | stored | cases | max-abs | beyond | rel-L2 | bar | scale | plain bar |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    by_fn = collections.OrderedDict()
    for test, rs in by_test.items():
        by_fn.setdefault(test.split("[")[0], []).extend(rs)
    for test, rs in by_fn.items():
        groups = collections.OrderedDict()
        for r in rs:
            groups.setdefault((_name(r["case"]), r["dtype"]), []).append(r)
        for (k, dt), g in groups.items():
            w = max(g, key=lambda x: x["max_abs"])
            rel = max(x["rel_l2"] for x in g)
            ok = all(x["literal_ok"] for x in g)
            exc = max(x["excess"] for x in g)
            lines.append(f"| `{test.split('/')[-1]}` | {k} | {dt} | {w['stored']} | {len(g)} | "
                         f"{w['max_abs']:.2e} | {exc:.2e} | {rel:.2e} | {w['bar_abs']:.1e} | "
                         f"{w['scale']} | {'yes' if ok else 'no'} |")
    with open(dst, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])

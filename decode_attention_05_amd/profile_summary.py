"""Summaries of rocprofv3 runs of the decode body-row kernel.

Reads the CSV output directories of the runs listed below (each made with
`--kernel-trace --pmc ... --output-format csv -o run`) and writes, for the
body-row kernel with and without a row subset:

* `profiles/decode_counters_<workload>[_subset].json`: HBM bytes per launch
  (FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads for
  a plain device copy of known size), the achieved clock (GRBM_GUI_ACTIVE
  summed over the 8 XCDs, divided by 8 and by the dispatch's duration), and
  the SQ counters, keyed by the hash of the kernel sources so that bench.py
  uses them only while they describe the current kernel;
* `profiles/decode_mfma_<workload>_counters.md`: the same as a table, with
  the commands that made the runs.

Usage (from the repository root, after the runs):
  python -m decode_attention_05_amd.profile_summary --config 3 \\
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-mib 512 \\
      --sq DIR [DIR ...] --trace DIR --commands FILE
or, for a kernel trace alone (profiles/decode_<workload>_kernel_stats.md):
  python -m decode_attention_05_amd.profile_summary --config 2 --trace DIR --commands FILE
or, for the HBM bytes of every kernel whose name holds MATCH
(profiles/<what>_<workload>_traffic.md):
  python -m decode_attention_05_amd.profile_summary --config 2 --what fit --match fit_ \\
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --commands FILE
or, for the calls of one operation in a trace (profiles/<what>_<workload>_kernel_stats.md),
the launches from each START kernel to the next END kernel:
  python -m decode_attention_05_amd.profile_summary --config 2 --trace DIR --commands FILE \\
      --what fold --window append_setup_kernel append_merge_kernel
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
XCDS = 8
BODY = "decode_mfma_kernel<"
COPY = "__amd_rocclr_copyBuffer"


def _rows(d: str) -> list[dict]:
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = []
    for f in files:
        out.extend(csv.DictReader(open(f)))
    return out


def per_kernel(d: str) -> dict:
    """{kernel name: {counter: mean per dispatch, '_dispatches': n, '_us': mean duration}}"""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(dict)
    for r in _rows(d):
        k = r["Kernel_Name"]
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        dur[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = {}
    for k, cs in vals.items():
        out[k] = {c: sum(v) / len(v) for c, v in cs.items()}
        out[k]["_dispatches"] = len(dur[k])
        out[k]["_us"] = sum(dur[k].values()) / len(dur[k])
    return out


def short(name: str) -> str:
    """decode_mfma_kernel<false, true> from the demangled name."""
    n = name.replace("(anonymous namespace)::", "").replace("lowram::", "")
    if n.startswith("void "):
        n = n[5:]
    depth = 0
    for i, ch in enumerate(n):          # up to the argument list, past template brackets
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return n[:i]
    return n


def body_kernels(table: dict) -> dict:
    return {short(k): v for k, v in table.items() if BODY in k}


def calibration(copy_fetch: str, copy_write: str, mib: int) -> dict:
    f = per_kernel(copy_fetch)[COPY]["FETCH_SIZE"]
    w = per_kernel(copy_write)[COPY]["WRITE_SIZE"]
    kib = mib * 1024
    return {"copy_mib": mib, "fetch_kib_per_copy": f, "write_kib_per_copy": w,
            "fetch_scale": kib / f, "write_scale": kib / w}


def trace_table(d: str) -> list[str]:
    """Per-kernel durations of a --kernel-trace --stats run (all its launches)."""
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    out = ["## Kernel trace (every launch of the run)", "",
           "| kernel | calls | mean µs | min µs | max µs | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in csv.DictReader(open(files[0])):
        name = short(r["Name"])
        name = name if len(name) <= 80 else name[:77] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} % |")
    return out + [""]


def window_table(d: str, start: str, end: str) -> list[str]:
    """Per-kernel durations over the launches from each `start` kernel to the
    next `end` kernel (one call of the operation each), and each call's span
    on the device (first start to last end, gaps between launches included)."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = sorted(csv.DictReader(open(files[0])), key=lambda r: int(r["Start_Timestamp"]))
    calls, cur = [], None
    for r in rows:
        name = r["Kernel_Name"]
        if start in name:
            cur = []
        if cur is not None:
            cur.append(r)
            if end in name:
                calls.append(cur)
                cur = None
    if not calls:
        raise SystemExit(f"no {start} .. {end} window in {d}")
    per = collections.defaultdict(list)
    spans = []
    for call in calls:
        t0 = int(call[0]["Start_Timestamp"])
        t1 = max(int(r["End_Timestamp"]) for r in call)
        spans.append((t1 - t0) / 1e3)
        for r in call:
            per[short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    spans.sort()
    out = [f"## Kernel trace of {len(calls)} calls (launches from `{start}` to `{end}`)", "",
           f"Device span per call (first launch's start to last launch's end): median {spans[len(spans) // 2]:.2f} µs, "
           f"min {spans[0]:.2f} µs, max {spans[-1]:.2f} µs.", "",
           "| kernel | launches | mean µs | min µs | max µs |", "|---|---|---|---|---|"]
    for k, v in per.items():
        out.append(f"| `{k}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    return out + [""]


def main() -> None:
    import sys
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash
    from decode_attention_05_amd import device as dev
    from decode_attention_05_amd import synth

    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--fetch", help="FETCH_SIZE run (with --write and the copy runs; else a trace summary only)")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int, default=512)
    ap.add_argument("--sq", nargs="*", default=[])
    ap.add_argument("--trace", default=None, help="directory of a --kernel-trace --stats run")
    ap.add_argument("--commands", required=True, help="text file with the commands of the runs")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--what", default="decode", help="the operation a trace-only summary covers")
    ap.add_argument("--match", default=None,
                    help="with the counter runs: a per-kernel traffic table of the kernels whose name holds this")
    ap.add_argument("--window", nargs=2, metavar=("START", "END"),
                    help="summarise the launches from each START kernel to the next END kernel")
    a = ap.parse_args()

    s = synth.CONFIGS[a.config]
    if not a.fetch:                                  # kernel trace only
        if not a.trace:
            raise SystemExit("give --trace, or the counter runs")
        commands = open(a.commands).read().strip()
        md = [f"# Kernel trace, {s.name} {a.what}", "",
              f"Workload: B={s.batch}, {s.group_layers} layers, {s.n_q_heads}/{s.n_kv_heads} heads, "
              f"d={s.head_dim}, r={s.rank}, {s.n_rows} body rows, {s.n_resid} residual rows per list, "
              f"{s.tail} tail rows.", "",
              "Commands (from the repository root on the GPU box):", "", "```", commands,
              f"python -m decode_attention_05_amd.profile_summary --config {a.config} --trace {a.trace} "
              + (f"--what {a.what} --window {a.window[0]} {a.window[1]} " if a.window else "")
              + "--commands <the command above>", "```", "",
              f"Kernel source hash: `{kernel_source_hash()}`.", ""]
        md += window_table(a.trace, *a.window) if a.window else trace_table(a.trace)
        with open(os.path.join(a.out, f"{a.what}_{s.name}_kernel_stats.md"), "w") as fh:
            fh.write("\n".join(md) + "\n")
        print("\n".join(md))
        return
    cal = calibration(a.copy_fetch, a.copy_write, a.copy_mib)
    if a.match:                                      # generic per-kernel traffic table
        fk, wk = per_kernel(a.fetch), per_kernel(a.write)
        commands = open(a.commands).read().strip()
        md = [f"# HBM traffic per launch, {s.name} {a.what}", "",
              f"Workload: B={s.batch}, {s.group_layers} layers, {s.n_q_heads}/{s.n_kv_heads} heads, "
              f"d={s.head_dim}, r={s.rank}, {s.n_rows} body rows.", "",
              "Commands (from the repository root on the GPU box; one counter per run):", "", "```", commands,
              f"python -m decode_attention_05_amd.profile_summary --config {a.config} --what {a.what} "
              f"--match {a.match} --fetch {a.fetch} --write {a.write} --copy-fetch {a.copy_fetch} "
              f"--copy-write {a.copy_write} --copy-mib {a.copy_mib} --commands <the commands above>", "```", "",
              f"Calibration: a {a.copy_mib} MiB device copy reads {cal['fetch_kib_per_copy']:.0f} KiB (FETCH_SIZE) "
              f"and writes {cal['write_kib_per_copy']:.0f} KiB (WRITE_SIZE): factors {cal['fetch_scale']:.4f} and "
              f"{cal['write_scale']:.4f}. Means per dispatch, durations of the counter runs.", "",
              "| kernel | dispatches | read MB (scaled) | write MB (scaled) | duration µs |", "|---|---|---|---|---|"]
        for k in sorted(fk):
            if a.match not in k or k not in wk:
                continue
            rd = fk[k]["FETCH_SIZE"] * 1024 * cal["fetch_scale"] / 1e6
            wr = wk[k]["WRITE_SIZE"] * 1024 * cal["write_scale"] / 1e6
            md.append(f"| `{short(k)}` | {fk[k]['_dispatches']} | {rd:.1f} | {wr:.1f} | {fk[k]['_us']:.1f} |")
        with open(os.path.join(a.out, f"{a.what}_{s.name}_traffic.md"), "w") as fh:
            fh.write("\n".join(md) + "\n")
        print("\n".join(md))
        return
    fetch, write = body_kernels(per_kernel(a.fetch)), body_kernels(per_kernel(a.write))
    sq = {}
    for d in a.sq:
        for k, v in body_kernels(per_kernel(d)).items():
            sq.setdefault(k, {}).update({c: x for c, x in v.items()})
    commands = open(a.commands).read().strip()
    src_hash = kernel_source_hash()
    n_sub = -(-s.n_rows * s.subset_frac[0] // s.subset_frac[1]) if s.subset_frac else 0
    md = [f"# Decode body-row kernel counters, {s.name}",
          "",
          f"Workload: B={s.batch}, {s.group_layers} layers, {s.n_q_heads}/{s.n_kv_heads} heads, d={s.head_dim}, "
          f"r={s.rank}, {s.n_rows} body rows, {s.n_resid} residual rows per list, {s.tail} tail rows.",
          "",
          "Commands (from the repository root on the GPU box; rocprofv3 CSV output, then this summary):",
          "", "```", commands,
          f"python -m decode_attention_05_amd.profile_summary --config {a.config} --fetch {a.fetch} "
          f"--write {a.write} --copy-fetch {a.copy_fetch} --copy-write {a.copy_write} --copy-mib {a.copy_mib} "
          f"--sq {' '.join(a.sq)}" + (f" --trace {a.trace}" if a.trace else "") +
          " --commands <the commands above>", "```", "",
          f"Kernel source hash: `{src_hash}`. Calibration: a {a.copy_mib} MiB device copy reads "
          f"{cal['fetch_kib_per_copy']:.0f} KiB (FETCH_SIZE) and writes {cal['write_kib_per_copy']:.0f} KiB "
          f"(WRITE_SIZE), so FETCH_SIZE is scaled by {cal['fetch_scale']:.4f} and WRITE_SIZE by "
          f"{cal['write_scale']:.4f}. Values are means per dispatch; durations are those of the counter runs "
          "(kernels serialised by the profiler).", ""]
    if a.trace:
        md += trace_table(a.trace)
    for name in sorted(fetch):
        subset = name.endswith("true>")
        n_att = n_sub if subset else s.n_rows
        rd = fetch[name]["FETCH_SIZE"] * 1024 * cal["fetch_scale"]
        wr = write[name]["WRITE_SIZE"] * 1024 * cal["write_scale"]
        alg = dev.algorithmic_body_kernel_bytes(s, n_att, subset)
        q = sq.get(name, {})
        clock = None
        if "GRBM_GUI_ACTIVE" in q and q.get("_us"):
            clock = q["GRBM_GUI_ACTIVE"] / XCDS / q["_us"]
        summary = {c: round(v) for c, v in sorted(q.items()) if not c.startswith("_")}
        if "SQ_INSTS_MFMA" in q:
            summary["mfma_flops_issued"] = q["SQ_INSTS_MFMA"] * 16 * 16 * 32 * 2
        if clock and "SQ_VALU_MFMA_BUSY_CYCLES" in q:
            # busy cycles summed over the 1024 SIMDs, against the dispatch's cycles
            summary["mfma_busy_frac"] = round(q["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (clock * q["_us"]), 4)
        rec = {"workload": s.name, "subset": subset, "kernel": name, "kernel_source_hash": src_hash,
               "copy_calibration": cal, "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
               "body_kernel_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": alg,
               "attended_rows": n_att, "clock_mhz": None if clock is None else round(clock, 1),
               "counter_run_duration_us": round(q.get("_us", fetch[name]["_us"]), 2),
               "dispatches": {"fetch": fetch[name]["_dispatches"], "write": write[name]["_dispatches"],
                              "sq": q.get("_dispatches")},
               "summary": summary, "commands": commands.splitlines()}
        path = os.path.join(a.out, f"decode_counters_{s.name}{'_subset' if subset else ''}.json")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
        md += [f"## `{name}` ({'the subset' if subset else 'every body row'}: {n_att} rows per sequence)", "",
               "| quantity | value |", "|---|---|",
               f"| HBM read per launch (FETCH_SIZE, scaled) | {rd / 1e6:.1f} MB |",
               f"| HBM write per launch (WRITE_SIZE, scaled) | {wr / 1e6:.1f} MB |",
               f"| algorithmic bytes per launch | {alg / 1e6:.1f} MB |",
               f"| traffic / algorithmic | {(rd + wr) / alg:.3f} |"]
        if clock:
            md.append(f"| achieved clock (GRBM_GUI_ACTIVE / 8 / duration) | {clock:.0f} MHz |")
        if "mfma_busy_frac" in summary:
            md.append(f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / cycles) | {summary['mfma_busy_frac']:.3f} |")
        md.append(f"| duration in the counter runs | {rec['counter_run_duration_us']} µs |")
        for c, v in summary.items():
            if c.startswith("SQ_") or c.startswith("GRBM_"):
                md.append(f"| {c} | {v} |")
        md.append("")
    with open(os.path.join(a.out, f"decode_mfma_{s.name}_counters.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


if __name__ == "__main__":
    main()

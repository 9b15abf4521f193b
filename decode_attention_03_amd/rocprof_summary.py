"""Profile the decode benchmark under rocprofv3 and write short text summaries.

    python3 -m decode_attention_03_amd.rocprof_summary --config 2 --raw RAW --out profiles

This process never touches the GPU: it starts rocprofv3 as a child process
(program directly after ``--``, working directory /tmp) over ``bench.py``,
then reads the CSV files rocprofv3 wrote under RAW.  Three kinds of run:

* ``--kernel-trace --stats`` over ``bench.py --config C --only``: per-kernel
  call counts and durations, set beside the split-kernel time that bench.py
  measured with HIP events in the same run;
* one ``--pmc FETCH_SIZE`` and one ``--pmc WRITE_SIZE`` pass over a short
  ``bench.py --config C --only`` run: HBM kilobytes per dispatch of the split
  kernel;
* the same two passes over ``bench.py --copy-probe BYTES`` (a streaming
  elementwise kernel that reads BYTES and writes BYTES): the calibration
  that turns counter readings into bytes;
* one pass of rocprofv3's derived utilisation metrics (VALUBusy, MfmaUtil,
  LdsUtil, SALUBusy: percent of the kernel's active GPU time the vector ALUs,
  matrix cores, LDS and scalar ALU were busy) on the split kernel.

With ``--section S`` it profiles one extra section of ``bench.py`` instead
(cascade, paged, shard): the kernel trace plus HBM bytes per dispatch of
every kernel the section launches, in ``<S>_<workload>.md``.

Written under OUT: ``<kernel>_<workload>.md`` (trace summary and traffic),
``traffic_<workload>.json`` (what bench.py reports as ``roofline.traffic``,
keyed by the hash of the kernel's sources so that it lapses when the kernel
changes).
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from decode_attention_03_amd import build, workloads  # noqa: E402

BENCH = os.path.join(ROOT, "bench.py")
COPY_BYTES = 1 << 30
# rocprofv3 kernel names -> kernel family (the source files it is built from)
FAMILIES = (("split_valu", "split_valu"), ("split_mfma", "split_mfma"), ("combine", "combine"))


def family_of(kernel_name: str) -> str | None:
    for needle, fam in FAMILIES:
        if needle in kernel_name:
            return fam
    return None


def run(cmd: list[str], limit_s: int, log_path: str) -> str:
    """Run a profiler command from /tmp; return its stdout, raise on failure."""
    env = dict(os.environ, TMPDIR="/tmp")
    full = ["timeout", "-s", "KILL", str(limit_s), *cmd]
    print("[prof] " + " ".join(cmd), file=sys.stderr, flush=True)
    t0 = time.time()
    res = subprocess.run(full, cwd="/tmp", env=env, capture_output=True, text=True)
    with open(log_path, "a", encoding="utf-8") as f:
        f.write(f"$ {' '.join(cmd)}\n{res.stdout}\n{res.stderr}\n")
    print(f"[prof] rc={res.returncode} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"profiler run failed (rc {res.returncode}); see {log_path}")
    return res.stdout


def read_csv(path: str) -> list[dict]:
    with open(path, newline="", encoding="utf-8") as f:
        return list(csv.DictReader(f))


def trace_stats(trace_csv: str) -> list[dict]:
    """Per-kernel count / mean / min / max duration (µs) from a kernel trace."""
    by: dict[str, list[float]] = {}
    for r in read_csv(trace_csv):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        by.setdefault(r["Kernel_Name"], []).append(dur)
    total = sum(sum(v) for v in by.values())
    out = []
    for name, v in by.items():
        out.append({"kernel": name, "calls": len(v), "avg_us": sum(v) / len(v), "min_us": min(v),
                    "max_us": max(v), "share": sum(v) / total if total else 0.0})
    out.sort(key=lambda r: -r["share"])
    return out


def counter_per_dispatch(csv_path: str, counter: str, match=None) -> tuple[float, int, str]:
    """Mean value of one counter over the dispatches whose kernel name `match`es
    (match None: the kernel dispatched most often in the file)."""
    rows = [r for r in read_csv(csv_path) if r["Counter_Name"] == counter]
    if match is None:
        calls: dict[str, set] = {}
        for r in rows:
            calls.setdefault(r["Kernel_Name"], set()).add(r["Dispatch_Id"])
        if calls:
            top = max(calls, key=lambda k: len(calls[k]))
            match = lambda name: name == top  # noqa: E731
    vals: dict[str, float] = {}
    name = ""
    for r in rows:
        if match is None or not match(r["Kernel_Name"]):
            continue
        vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        name = r["Kernel_Name"]
    if not vals:
        raise RuntimeError(f"no {counter} rows for the requested kernel in {csv_path}")
    return sum(vals.values()) / len(vals), len(vals), name


def last_json_line(text: str) -> dict:
    for line in reversed(text.strip().splitlines()):
        if line.startswith("{"):
            return json.loads(line)
    raise RuntimeError("bench.py printed no JSON line")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=2, help="named workload (1-5)")
    ap.add_argument("--raw", required=True, help="directory for rocprofv3's raw output")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"), help="summary directory")
    ap.add_argument("--pmc-steps", type=int, default=3)
    ap.add_argument("--skip-copy", action="store_true",
                    help="reuse the copy calibration already in RAW")
    ap.add_argument("--section", choices=("cascade", "paged", "shard", "groups", "ragged_mha"),
                    default=None, help="profile one section of bench.py instead of a named workload")
    args = ap.parse_args()
    if args.section:
        return section_main(args)

    w = workloads.WORKLOADS[args.config]
    raw = os.path.abspath(args.raw)
    out = os.path.abspath(args.out)
    os.makedirs(raw, exist_ok=True)
    os.makedirs(out, exist_ok=True)
    log_path = os.path.join(raw, f"{w.name}.log")
    py = sys.executable
    tag = f"c{args.config}"

    def shown(cmd: list[str]) -> str:
        """A command as recorded: RAW for the raw directory, paths relative to the repository."""
        return " ".join(cmd).replace(raw, "RAW").replace(ROOT + "/", "")

    # 1. the bench run that reports roofline.achieved, on its own (the
    # profiler's per-dispatch bookkeeping stretches the gaps between launches,
    # so event timings taken under it are not the kernel's), then the same
    # command under the kernel trace
    bench_cmd = [py, BENCH, "--config", str(args.config), "--only", "--cpu-budget", "0"]
    res = last_json_line(run(bench_cmd, 300, log_path))
    trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "-d", raw, "-o", f"{tag}_trace",
                 "--output-format", "csv", "--", *bench_cmd]
    run(trace_cmd, 300, log_path)
    stats = trace_stats(os.path.join(raw, f"{tag}_trace_kernel_trace.csv"))

    # 2. HBM counters on the split kernel, one counter per pass
    short = [py, BENCH, "--config", str(args.config), "--only", "--cpu-budget", "0",
             "--steps", str(args.pmc_steps), "--warmup", "1"]
    pmc_cmds = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cmd = ["rocprofv3", "--pmc", counter, "-d", raw, "-o", f"{tag}_{counter}",
               "--output-format", "csv", "--", *short]
        run(cmd, 240, log_path)
        pmc_cmds[counter] = cmd

    # 2b. unit utilisation of the split kernel (derived metrics, one pass)
    util_metrics = ("VALUBusy", "MfmaUtil", "LdsUtil", "SALUBusy")
    util_cmd = ["rocprofv3", "--pmc", *util_metrics, "-d", raw, "-o", f"{tag}_util",
                "--output-format", "csv", "--", *short]
    run(util_cmd, 240, log_path)

    # 3. calibration on a streaming kernel of known size
    copy = [py, BENCH, "--copy-probe", str(COPY_BYTES)]
    copy_cmds = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cmd = ["rocprofv3", "--pmc", counter, "-d", raw, "-o", f"copy_{counter}",
               "--output-format", "csv", "--", *copy]
        if not args.skip_copy:
            run(cmd, 120, log_path)
        copy_cmds[counter] = cmd

    def is_split(name: str) -> bool:
        return family_of(name) in ("split_valu", "split_mfma")

    cal = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        v, n, cname = counter_per_dispatch(
            os.path.join(raw, f"copy_{counter}_counter_collection.csv"), counter)
        cal[counter] = {"kernel": cname, "counter_per_dispatch": v, "dispatches": n,
                        "bytes_per_unit": COPY_BYTES / v}
    meas = {}
    kname = ""
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        v, n, kname = counter_per_dispatch(
            os.path.join(raw, f"{tag}_{counter}_counter_collection.csv"), counter, is_split)
        meas[counter] = {"counter_per_dispatch": v, "dispatches": n,
                         "bytes": v * cal[counter]["bytes_per_unit"]}
    util = {}
    for mname in util_metrics:
        v, n, _ = counter_per_dispatch(os.path.join(raw, f"{tag}_util_counter_collection.csv"),
                                       mname, is_split)
        util[mname] = round(v, 2)
    fam = family_of(kname)
    roof = res["roofline"]
    alg = roof["algorithmic_bytes_per_launch"]
    hbm = meas["FETCH_SIZE"]["bytes"] + meas["WRITE_SIZE"]["bytes"]
    rec = {
        "workload": w.name, "kernel": fam, "kernel_name": kname,
        "kernel_source_hash": build.source_hash(fam),
        "hbm_bytes_per_launch": round(hbm),
        "fetch_bytes_per_launch": round(meas["FETCH_SIZE"]["bytes"]),
        "write_bytes_per_launch": round(meas["WRITE_SIZE"]["bytes"]),
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": round(hbm / alg, 4),
        "calibration": {c: {k: (round(x, 4) if isinstance(x, float) else x)
                            for k, x in d.items()} for c, d in cal.items()},
        "copy_probe_bytes": COPY_BYTES,
        "utilisation_percent": util,
        "commands": {"fetch": shown(pmc_cmds["FETCH_SIZE"]),
                     "write": shown(pmc_cmds["WRITE_SIZE"]),
                     "copy_fetch": shown(copy_cmds["FETCH_SIZE"]),
                     "copy_write": shown(copy_cmds["WRITE_SIZE"])},
    }
    with open(os.path.join(out, f"traffic_{w.name}.json"), "w", encoding="utf-8") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")

    split_rows = [r for r in stats if family_of(r["kernel"]) in ("split_valu", "split_mfma")]
    lines = [
        f"# {fam} on {w.name}",
        "",
        f"Workload: batch {w.batch}, {w.heads_q} query / {w.heads_kv} KV heads, d {w.head_dim}, "
        f"N {w.max_kv_len}{' (ragged)' if w.ragged else ''}, {w.dtype}; " +
        (f"{res['config']['num_splits']} splits of {res['config']['split_len']} tokens."
         if res["config"].get("num_splits") else f"plan: {res['config'].get('plan')}."),
        "",
        "Made by (repository root):",
        "",
        "    python3 -m decode_attention_03_amd.rocprof_summary "
        f"--config {args.config} --raw RAW --out profiles",
        "",
        "which runs, from /tmp:",
        "",
        "    " + shown(bench_cmd),
        "    " + shown(trace_cmd),
        "    " + shown(pmc_cmds["FETCH_SIZE"]),
        "    " + shown(pmc_cmds["WRITE_SIZE"]),
        "    " + shown(copy_cmds["FETCH_SIZE"]),
        "    " + shown(copy_cmds["WRITE_SIZE"]),
        "    " + shown(util_cmd),
        "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats)",
        "",
        "| kernel | calls | avg µs | min µs | max µs | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in stats:
        lines.append(f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {100 * r['share']:.1f} % |")
    if split_rows:
        s = split_rows[0]
        # bench.py times fd_decode's split stage alone (fd_decode_stages)
        timed, what = s["avg_us"], "split kernel"
        lines += [
            "",
            f"bench.py (same command, not under the profiler): {what} {roof['kernel_us']} µs "
            f"by HIP events over the timed region; kernel trace average {timed:.2f} µs "
            f"(ratio {timed / roof['kernel_us']:.3f}); "
            f"roofline.achieved {roof['achieved']} GB/s = {alg} algorithmic bytes / that time "
            f"({100 * roof['frac']:.1f} % of 8 TB/s); step {res['us_per_step']} µs, "
            f"value {res['value']} GB/s.",
        ]
    lines += [
        "",
        "## HBM traffic (rocprofv3 --pmc, one counter per pass)",
        "",
        "| | counter / dispatch | dispatches | bytes per counter unit | bytes / launch |",
        "|---|---|---|---|---|",
        f"| copy probe FETCH_SIZE ({COPY_BYTES} B read) | {cal['FETCH_SIZE']['counter_per_dispatch']:.1f} | "
        f"{cal['FETCH_SIZE']['dispatches']} | {cal['FETCH_SIZE']['bytes_per_unit']:.2f} | {COPY_BYTES} |",
        f"| copy probe WRITE_SIZE ({COPY_BYTES} B written) | {cal['WRITE_SIZE']['counter_per_dispatch']:.1f} | "
        f"{cal['WRITE_SIZE']['dispatches']} | {cal['WRITE_SIZE']['bytes_per_unit']:.2f} | {COPY_BYTES} |",
        f"| split kernel FETCH_SIZE | {meas['FETCH_SIZE']['counter_per_dispatch']:.1f} | "
        f"{meas['FETCH_SIZE']['dispatches']} | | {meas['FETCH_SIZE']['bytes']:.0f} |",
        f"| split kernel WRITE_SIZE | {meas['WRITE_SIZE']['counter_per_dispatch']:.1f} | "
        f"{meas['WRITE_SIZE']['dispatches']} | | {meas['WRITE_SIZE']['bytes']:.0f} |",
        "",
        f"HBM bytes per launch {hbm:.0f} against {alg} algorithmic bytes: "
        f"ratio {hbm / alg:.4f}.  Kernel source hash {rec['kernel_source_hash']}.",
        "",
        "## Unit utilisation of the split kernel (rocprofv3 derived metrics, % of active time)",
        "",
        "| VALUBusy | MfmaUtil | LdsUtil | SALUBusy |",
        "|---|---|---|---|",
        f"| {util['VALUBusy']} | {util['MfmaUtil']} | {util['LdsUtil']} | {util['SALUBusy']} |",
        "",
        "The kernel is bound by HBM (traffic above); these show how much of each unit's time the",
        "streaming leaves in use.",
        "",
    ]
    md = os.path.join(out, f"{fam}_{w.name}.md")
    with open(md, "w", encoding="utf-8") as f:
        f.write("\n".join(lines))
    print(f"[prof] wrote {md}", file=sys.stderr, flush=True)
    return 0


def calibrate(raw: str, skip: bool, log_path: str) -> tuple[dict, dict]:
    """Copy-probe passes (FETCH_SIZE, WRITE_SIZE): bytes per counter unit."""
    copy = [sys.executable, BENCH, "--copy-probe", str(COPY_BYTES)]
    cmds, cal = {}, {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cmd = ["rocprofv3", "--pmc", counter, "-d", raw, "-o", f"copy_{counter}",
               "--output-format", "csv", "--", *copy]
        if not skip:
            run(cmd, 120, log_path)
        cmds[counter] = cmd
        v, n, cname = counter_per_dispatch(
            os.path.join(raw, f"copy_{counter}_counter_collection.csv"), counter)
        cal[counter] = {"kernel": cname, "counter_per_dispatch": v, "dispatches": n,
                        "bytes_per_unit": COPY_BYTES / v}
    return cal, cmds


def section_main(args) -> int:
    """Kernel trace and HBM bytes per dispatch of every kernel that one bench.py
    section launches (cascade: the shared-prefix kernel, the suffix kernel and
    the combine; paged: the ragged grouped workload over 16-token pages;
    shard: one GPU's share of the long-context workload and the merge;
    groups: six shapes with 32 to 128 query heads per KV head; ragged_mha:
    two ragged multi-head batches, balanced on the vector kernel and as
    fixed splits)."""
    raw = os.path.abspath(args.raw)
    out = os.path.abspath(args.out)
    os.makedirs(raw, exist_ok=True)
    os.makedirs(out, exist_ok=True)
    sec = args.section
    log_path = os.path.join(raw, f"section_{sec}.log")
    py = sys.executable

    def shown(cmd: list[str]) -> str:
        return " ".join(cmd).replace(raw, "RAW").replace(ROOT + "/", "")

    bench_cmd = [py, BENCH, "--section", sec]
    res = last_json_line(run(bench_cmd, 300, log_path))
    trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "-d", raw, "-o", f"{sec}_trace",
                 "--output-format", "csv", "--", *bench_cmd]
    run(trace_cmd, 300, log_path)
    stats = trace_stats(os.path.join(raw, f"{sec}_trace_kernel_trace.csv"))
    short = [py, BENCH, "--section", sec, "--steps", str(args.pmc_steps), "--warmup", "1"]
    pmc_cmds = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cmd = ["rocprofv3", "--pmc", counter, "-d", raw, "-o", f"{sec}_{counter}",
               "--output-format", "csv", "--", *short]
        run(cmd, 240, log_path)
        pmc_cmds[counter] = cmd
    cal, copy_cmds = calibrate(raw, args.skip_copy, log_path)
    per = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        path = os.path.join(raw, f"{sec}_{counter}_counter_collection.csv")
        names = sorted({r["Kernel_Name"] for r in read_csv(path) if r["Counter_Name"] == counter})
        for name in names:
            v, n, _ = counter_per_dispatch(path, counter, lambda k, name=name: k == name)
            per.setdefault(name, {})[counter] = v * cal[counter]["bytes_per_unit"]
    lines = [
        f"# bench.py section `{sec}`: {res.get('workload', '')}",
        "",
        "Made by (repository root):",
        "",
        f"    python3 -m decode_attention_03_amd.rocprof_summary --section {sec} --raw RAW "
        "--out profiles",
        "",
        "which runs, from /tmp:",
        "",
        "    " + shown(bench_cmd),
        "    " + shown(trace_cmd),
        "    " + shown(pmc_cmds["FETCH_SIZE"]),
        "    " + shown(pmc_cmds["WRITE_SIZE"]),
        "    " + shown(copy_cmds["FETCH_SIZE"]),
        "    " + shown(copy_cmds["WRITE_SIZE"]),
        "",
        "bench.py section result (same command, not under the profiler):",
        "",
        "    " + json.dumps(res),
        "",
        "## Kernel trace (rocprofv3 --kernel-trace --stats) and HBM bytes per dispatch",
        "",
        "HBM bytes: FETCH_SIZE and WRITE_SIZE per dispatch (one counter per pass), scaled by what "
        f"the same counters read for a copy kernel of {COPY_BYTES} bytes each way "
        f"({cal['FETCH_SIZE']['bytes_per_unit']:.2f} and "
        f"{cal['WRITE_SIZE']['bytes_per_unit']:.2f} bytes per unit).",
        "",
        "| kernel | calls | avg µs | min µs | max µs | share | HBM read B | HBM write B |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for r in stats:
        b = per.get(r["kernel"], {})
        rd = f"{b['FETCH_SIZE']:.0f}" if "FETCH_SIZE" in b else ""
        wr = f"{b['WRITE_SIZE']:.0f}" if "WRITE_SIZE" in b else ""
        lines.append(f"| `{r['kernel']}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {100 * r['share']:.1f} % | {rd} | {wr} |")
    lines.append("")
    wname = res.get("workload", sec)
    md = os.path.join(out, (wname if wname.startswith(sec + "_") else f"{sec}_{wname}") + ".md")
    with open(md, "w", encoding="utf-8") as f:
        f.write("\n".join(lines))
    print(f"[prof] wrote {md}", file=sys.stderr, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Per-work-group timing of the token-balanced split kernel.

    python3 -m decode_attention_03_amd.wg_clocks --build          # CPU: the instrumented library
    python3 -m decode_attention_03_amd.wg_clocks --config 4 --out profiles   # GPU: stamps + summary

--build compiles the library with -DFD_WG_CLOCKS=1 into libfd_wgclocks.so
(beside libfd.so; the product library is untouched).  In that build the
token-balanced split kernel writes, for every work-group, the constant
100 MHz clock when it starts and when it ends, the pieces and K/V tokens it
processed and its block index, with ordinary global stores into a buffer
given through fd_debug_wg_clocks.  The run times `--launches` split-stage
launches of the named workload's fd_decode (after a settle period, each into
its own stamp buffer) and summarises, per launch and over all of them: when
work-groups start and finish relative to the first start, how long each
runs, the rate each one streams K/V at, and how these differ between the
eight XCDs (the XCC_ID register).  Whether a slow step comes from a few
work-groups finishing late (a tail) or from every work-group streaming
slower shows up as the spread of finish times against the spread of rates.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

VARIANT = os.path.join(PKG, "libfd_wgclocks.so")
FLAGS = ["-DFD_WG_CLOCKS=1"]
CLOCK_HZ = 100e6  # s_memrealtime


def build_variant() -> str:
    from decode_attention_03_amd import build

    return build.build(extra_flags=FLAGS, out=VARIANT)


def _pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(p / 100 * (len(xs) - 1))))]


def analyse(stamps: list[list[tuple]], row_bytes: int) -> dict:
    """stamps[launch] = [(start, end, pieces, tokens, block)] per work-group
    that did work; times in clock ticks."""
    per_launch = []
    ends, durs, rates, starts = [], [], [], []
    by_xcd: dict[int, list[float]] = {}
    for wgs in stamps:
        t0 = min(s for s, *_ in wgs)
        t_end = max(e for _, e, *_ in wgs)
        span = (t_end - t0) / CLOCK_HZ * 1e6
        busy = sum((e - s) for s, e, *_ in wgs) / CLOCK_HZ * 1e6
        fin = [(e - t0) / CLOCK_HZ * 1e6 for _, e, *_ in wgs]
        per_launch.append({"span_us": span, "mean_busy_frac": busy / (span * len(wgs)),
                           "finish_p50_us": _pct(fin, 50), "finish_p90_us": _pct(fin, 90),
                           "finish_min_us": min(fin)})
        for s, e, pieces, tokens, blk in wgs:
            d = (e - s) / CLOCK_HZ * 1e6
            starts.append((s - t0) / CLOCK_HZ * 1e6)
            ends.append((e - t0) / CLOCK_HZ * 1e6)
            durs.append(d)
            r = tokens * row_bytes / (d * 1e-6) / 1e9 if d > 0 else 0.0
            rates.append(r)
            by_xcd.setdefault((blk >> 24) & 0xff, []).append(r)
    spans = [x["span_us"] for x in per_launch]
    return {
        "launches": len(stamps), "work_groups": len(stamps[0]) if stamps else 0,
        "span_us": {"median": statistics.median(spans), "min": min(spans), "max": max(spans)},
        "mean_busy_frac": statistics.mean(x["mean_busy_frac"] for x in per_launch),
        "start_us": {p: _pct(starts, p) for p in (0, 50, 90, 99, 100)},
        "finish_us": {p: _pct(ends, p) for p in (0, 10, 50, 90, 99, 100)},
        "duration_us": {p: _pct(durs, p) for p in (0, 10, 50, 90, 100)},
        "rate_GBps": {p: _pct(rates, p) for p in (0, 10, 50, 90, 100)},
        "rate_by_xcd_GBps": {x: statistics.mean(v) for x, v in sorted(by_xcd.items())},
    }


def run(config: int, launches: int, out_dir: str | None, raw_path: str | None = None,
        library: str | None = None) -> dict:
    import torch

    from decode_attention_03_amd import workloads

    if not torch.cuda.is_available():
        raise RuntimeError("needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.init()
    torch.empty(1, device=dev)
    torch.cuda.synchronize(dev)
    from decode_attention_03_amd import build, fd

    path = library or VARIANT  # another instrumented build (its flags include FD_WG_CLOCKS=1)
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run with --build first (on the CPU)")
    rec = fd.check_fresh(path, build.record_path(path), allow_flags=True)
    if "-DFD_WG_CLOCKS=1" not in (rec.get("flags") or []):
        raise RuntimeError(f"{path} is not an instrumented build (-DFD_WG_CLOCKS=1)")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fd_decode_stages.argtypes = [P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, P, P, S, I, P]
    lib.fd_decode_stages.restype = I
    lib.fd_debug_wg_clocks.argtypes, lib.fd_debug_wg_clocks.restype = [P, S], I
    lib.fd_last_error.argtypes, lib.fd_last_error.restype = [], ctypes.c_char_p

    class Plan(ctypes.Structure):
        _fields_ = [("route", I), ("kernel", I), ("num_splits", I), ("split_len", I),
                    ("waves_per_group", I), ("query_tiles", I), ("launches", I),
                    ("work_groups", ctypes.c_int64), ("workspace_bytes", S)]

    lib.fd_decode_plan.argtypes = [I] * 11 + [ctypes.POINTER(Plan)]
    lib.fd_decode_plan.restype = I
    w = workloads.WORKLOADS[config]
    inp = workloads.generate(w)
    code = {"f32": 0, "f16": 1, "bf16": 2}[w.dtype]
    n_max = inp["max_kv_len"]
    lens = inp["kv_lens"]
    plan = Plan()
    rc = lib.fd_decode_plan(w.batch, w.heads_q, w.heads_kv, n_max, w.head_dim, code,
                            int(lens is not None), 0, 0, 0, 0, ctypes.byref(plan))
    if rc != 0 or plan.route != 3:
        raise RuntimeError(f"workload {w.name} does not take the token-balanced plan "
                           f"(rc {rc}, route {plan.route})")
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    kl = None if lens is None else lens.to(dev)
    o = torch.empty((w.batch, w.heads_q, w.head_dim), dtype=q.dtype, device=dev)
    lse = torch.empty((w.batch, w.heads_q), dtype=torch.float32, device=dev)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    nwg = int(plan.work_groups)
    bufs = [torch.zeros(nwg * 4, dtype=torch.int64, device=dev) for _ in range(launches)]
    stream = torch.cuda.current_stream(dev)
    args = (P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
            None if kl is None else P(kl.data_ptr()), w.batch, w.heads_q, w.heads_kv, n_max,
            w.head_dim, code, code, F(w.scale), 0, 0, P(o.data_ptr()), P(lse.data_ptr()),
            P(ws.data_ptr()), plan.workspace_bytes, 1, P(stream.cuda_stream))

    def launch():
        rc = lib.fd_decode_stages(*args)
        if rc != 0:
            raise RuntimeError(lib.fd_last_error().decode())

    lib.fd_debug_wg_clocks(None, 0)
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < 0.2:  # clocks out of idle before the stamped launches
        launch()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    for b in bufs:
        lib.fd_debug_wg_clocks(P(b.data_ptr()), b.numel() * 8)
        launch()
    lib.fd_debug_wg_clocks(None, 0)
    torch.cuda.synchronize()
    stamps = []
    for b in bufs:
        a = b.view(-1, 4).cpu().tolist()
        stamps.append([(s, e, wk >> 32, wk & 0xffffffff, blk) for s, e, wk, blk in a
                       if wk >> 32 > 0])
    if raw_path:  # every stamp, per launch: [start, end, pieces, tokens, where] per share
        with open(raw_path, "w", encoding="utf-8") as f:
            json.dump({"workload": w.name, "plan_work_groups": nwg,
                       "launches": [[list(x) for x in L] for L in stamps]}, f)
    row_bytes = w.head_dim * 2 * inp["k"].element_size()  # K + V of one token of one KV head
    res = {"workload": w.name, "plan_work_groups": nwg, **analyse(stamps, row_bytes)}
    if out_dir:
        write_summary(res, config, out_dir)
    return res


def write_summary(res: dict, config: int, out_dir: str) -> str:
    def fmt(d):
        return ", ".join(f"p{k} {v:.1f}" for k, v in d.items())

    lines = [
        f"# Per-work-group clocks of the token-balanced split kernel on {res['workload']}",
        "",
        "Made by (repository root; the first command on the CPU, the second on the GPU):",
        "",
        "    python3 -m decode_attention_03_amd.wg_clocks --build",
        f"    python3 -m decode_attention_03_amd.wg_clocks --config {config} --out profiles",
        "",
        "Instrumented build (-DFD_WG_CLOCKS=1): each work-group stores its start and end "
        "times (the constant 100 MHz clock), its pieces and K/V tokens, and where it ran (block index, XCD, CU and SIMD from the hardware-ID registers). "
        f"{res['launches']} split-stage launches of fd_decode's plan after a 0.2 s settle; "
        f"{res['work_groups']} of {res['plan_work_groups']} work-groups had work.",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| kernel span, first start to last end (µs) | median {res['span_us']['median']:.1f}, "
        f"min {res['span_us']['min']:.1f}, max {res['span_us']['max']:.1f} |",
        f"| mean busy fraction (Σ durations / (work-groups × span)) | "
        f"{res['mean_busy_frac']:.4f} |",
        f"| start after the first start (µs) | {fmt(res['start_us'])} |",
        f"| finish after the first start (µs) | {fmt(res['finish_us'])} |",
        f"| work-group duration (µs) | {fmt(res['duration_us'])} |",
        f"| work-group K/V rate (GB/s) | {fmt(res['rate_GBps'])} |",
        "| mean rate by XCD (XCC_ID register, GB/s) | " +
        ", ".join(f"{x}: {r:.2f}" for x, r in res["rate_by_xcd_GBps"].items()) + " |",
        "",
    ]
    os.makedirs(out_dir, exist_ok=True)
    path = os.path.join(out_dir, f"wg_clocks_{res['workload']}.md")
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines))
    return path


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--build", action="store_true", help="build the instrumented library")
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--launches", type=int, default=20)
    ap.add_argument("--out", default=None, help="write the summary here")
    ap.add_argument("--raw", default=None, help="write every stamp here (JSON)")
    ap.add_argument("--from-raw", default=None,
                    help="summarise stamps saved with --raw instead of running (no GPU)")
    ap.add_argument("--library", default=None,
                    help="an instrumented tuning variant instead of libfd_wgclocks.so")
    args = ap.parse_args()
    if args.build:
        print(build_variant())
        return 0
    if args.from_raw:  # summarise stamps written earlier by --raw (no GPU)
        with open(args.from_raw, encoding="utf-8") as f:
            raw = json.load(f)
        from decode_attention_03_amd import workloads

        w = workloads.WORKLOADS[args.config]
        if raw["workload"] != w.name:
            raise SystemExit(f"{args.from_raw} holds {raw['workload']}, not {w.name}")
        stamps = [[tuple(x) for x in launch] for launch in raw["launches"]]
        elem = 4 if w.dtype == "f32" else 2
        res = {"workload": w.name, "plan_work_groups": raw.get("plan_work_groups", len(stamps[0])),
               **analyse(stamps, w.head_dim * 2 * elem)}
        if args.out:
            write_summary(res, args.config, args.out)
        print(json.dumps(res), flush=True)
        return 0
    res = run(args.config, args.launches, args.out, args.raw, args.library)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

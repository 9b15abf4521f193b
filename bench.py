#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X: µs per decode step and effective
KV bandwidth (bytes of K and V a step must read / step time) against the
8 TB/s HBM peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--section S]

One "step" is one fd_decode call (split kernel + combine kernel) over one
batch of the workload, inputs already resident in HBM.  The headline
workload is the ragged grouped-query bf16 batch (--config 4: 16 sequences of
512-32768 tokens, 64 query heads on 8 KV heads, d = 128), one of the two
long-context bf16 workloads; the other named workloads are timed in the same
run and reported under "workloads".  Each workload keeps
enough copies of its K/V in HBM that consecutive steps read different copies,
so a step cannot be served from the 256 MB Infinity Cache (the 0.5 MiB fp32
workload is cache-resident by nature and reports µs only).

Printed: one JSON line on stdout.  Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

from decode_attention_03_amd import build, fd, workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "effective KV GB/s (% of 8 TB/s HBM peak) and µs per decode step"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class Prepared:
    """A workload resident on the GPU with pre-bound fd_decode arguments."""

    def __init__(self, w: workloads.Workload, dev: torch.device, num_splits: int = 0,
                 host: dict | None = None):
        self.w = w
        t0 = time.time()
        inp = workloads.generate(w) if host is None else host
        self.host = inp
        lens = inp["kv_lens"]
        self.kv_bytes = workloads.kv_bytes(w, lens)
        footprint = inp["k"].numel() * inp["k"].element_size() * 2
        # copies so that consecutive steps stream different memory: with >= 1 GiB
        # read between two reads of one copy, no step hits the Infinity Cache
        if footprint < (64 << 20):
            self.copies = 1
        else:
            self.copies = max(2, min(16, math.ceil((1 << 30) / footprint) + 1))
        self.q = inp["q"].to(dev)
        self.kv = []
        for _ in range(self.copies):
            self.kv.append((inp["k"].to(dev), inp["v"].to(dev)))
        self.lens = None if lens is None else lens.to(dev)
        batch, hq, hkv, d = w.batch, w.heads_q, w.heads_kv, w.head_dim
        self.n_max = inp["max_kv_len"]
        if num_splits == 0 and w.num_splits:
            num_splits = w.num_splits
        # the library's automatic plan unless the workload or the caller fixes B
        self.auto = num_splits == 0
        # the library's own account of what fd_decode launches here
        self.dplan = fd.decode_plan(batch, hq, hkv, self.n_max, d, inp["q"].dtype,
                                    lens is not None, num_splits)
        self.balanced = self.dplan["route"] == "balanced"
        if self.balanced:  # B, L of fixed splits, for the split stage timed on its own
            self.B, self.L = fd.choose_splits(batch, hq, hkv, self.n_max, d, inp["q"].dtype,
                                              ragged=True)
        else:
            self.B, self.L = self.dplan["num_splits"], self.dplan["split_len"]
        self.plan = "token-balanced" if self.balanced else "fixed-splits"
        self.o = torch.empty((batch, hq, d), dtype=workloads.TORCH_DTYPES[w.out_dtype],
                             device=dev)
        self.lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
        dec_b, dec_l = (0, 0) if self.auto else (self.B, self.L)
        self.dec_b, self.dec_l = dec_b, dec_l
        ws = self.dplan["workspace_bytes"]
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.ws_bytes = ws
        # partial buffers of the split kernel when it is timed on its own
        # (fd_decode_split always writes partials, also for one split)
        self.o_part = torch.empty((batch, hq, self.B, d), dtype=torch.float32, device=dev)
        self.lse_part = torch.empty((batch, hq, self.B), dtype=torch.float32, device=dev)
        self.lib = fd.library()
        self.stream = torch.cuda.current_stream(dev)
        sp = ctypes.c_void_p(self.stream.cuda_stream)
        code = {torch.float32: fd.F32, torch.float16: fd.F16, torch.bfloat16: fd.BF16}
        self.in_code = code[self.q.dtype]
        self.out_code = code[self.o.dtype]
        P = ctypes.c_void_p
        lens_p = None if self.lens is None else P(self.lens.data_ptr())
        self.decode_args = []
        self.split_args = []
        self.stage_args = []  # fd_decode_stages with the split stage only
        for k, v in self.kv:
            self.decode_args.append((P(self.q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
                                     lens_p, batch, hq, hkv, self.n_max, d, self.in_code,
                                     self.out_code, ctypes.c_float(w.scale), dec_b, dec_l,
                                     P(self.o.data_ptr()), P(self.lse.data_ptr()),
                                     P(self.ws.data_ptr()), self.ws_bytes, sp))
            self.split_args.append((P(self.q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()),
                                    lens_p, batch, hq, hkv, self.n_max, d, self.in_code,
                                    ctypes.c_float(w.scale), self.B, self.L,
                                    P(self.o_part.data_ptr()), P(self.lse_part.data_ptr()), sp))
            self.stage_args.append(self.decode_args[-1][:-1] + (fd.STAGE_SPLIT, sp))
        # algorithmic bytes of the timed split launch: K/V rows, q, and the
        # partials written (fixed splits: B per row; balanced: at most one per
        # work-group piece, bounded by work-groups + units, counted in full)
        if self.balanced:
            # units: (sequence, KV head) of hq / hkv rows on the matrix cores,
            # (sequence, query head) of one row on the vector kernel
            vec = self.dplan["kernel"] == "vector"
            g = hq // hkv  # fp32 groups: up to eight query heads per vector unit
            hpw = 1
            if vec and w.dtype == "f32":
                hpw = 8 if g % 8 == 0 and d <= 128 else 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
            units, rows = (batch * hq // hpw, hpw) if vec else (batch * hkv, g)
            pieces = self.dplan["work_groups"] + units
            self.part_bytes = pieces * rows * (d + 1) * 4
        else:
            self.part_bytes = batch * hq * self.B * (d + 1) * 4 if self.B > 1 else 0
        self.split_bytes = self.kv_bytes + self.q.numel() * self.q.element_size() + self.part_bytes
        log(f"[bench] {w.name}: plan={self.plan} B={self.B} L={self.L} copies={self.copies} "
            f"kv={self.kv_bytes / 2**20:.1f} MiB prep={time.time() - t0:.1f}s")

    def decode(self, i: int) -> None:
        rc = self.lib.fd_decode(*self.decode_args[i % self.copies])
        if rc != fd.OK:
            raise fd.FDError(rc, fd.last_error())

    def split(self, i: int) -> None:
        rc = self.lib.fd_decode_split(*self.split_args[i % self.copies])
        if rc != fd.OK:
            raise fd.FDError(rc, fd.last_error())

    def split_stage(self, i: int) -> None:
        """The split launch of fd_decode alone (fd_decode_stages)."""
        rc = self.lib.fd_decode_stages(*self.stage_args[i % self.copies])
        if rc != fd.OK:
            raise fd.FDError(rc, fd.last_error())

    def free(self) -> None:
        self.kv.clear()
        self.q = self.o = self.lse = self.ws = self.o_part = self.lse_part = None


SETTLE_MS = 100.0


def settle(run, min_ms: float = SETTLE_MS) -> None:
    """Run `run(i)` back to back until `min_ms` of wall time has passed.  The
    GPU's clocks take ~15 ms of load to leave an idle state (measured: the
    grouped kernel's first ~90 steps after a 0.5 s pause are up to 17 %
    slower, HIP events agreeing with the wall clock), so every timed region is
    preceded by this, then by the requested warm-up steps."""
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        run(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_steps(p: Prepared, steps: int, warmup: int) -> dict:
    """Wall clock over exactly `steps` fd_decode calls (synchronized on both
    sides), plus HIP events around each call for the median."""
    settle(p.decode)
    for i in range(warmup):
        p.decode(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        p.decode(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(p.stream)
        p.decode(i)
        ev[i][1].record(p.stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return {"wall_us_per_step": wall / steps * 1e6, "event_us_median": per[len(per) // 2],
            "event_us_p10": per[len(per) // 10], "event_us_p90": per[(9 * len(per)) // 10]}


def time_graph_steps(p: Prepared, steps: int, per_graph: int = 20) -> float:
    """µs per decode step with `per_graph` steps captured in one HIP graph and
    the graph replayed: the GPU-side cost of a step without the per-call host
    overhead (what a serving loop that replays graphs pays)."""
    s = torch.cuda.Stream(device=p.q.device)
    s.wait_stream(torch.cuda.current_stream(p.q.device))
    saved = p.decode_args
    sp = ctypes.c_void_p(s.cuda_stream)
    p.decode_args = [a[:-1] + (sp,) for a in saved]  # same arguments on the capture stream
    try:
        with torch.cuda.stream(s):
            p.decode(0)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(per_graph):
                p.decode(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // per_graph)
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (reps * per_graph) * 1e6
    finally:
        p.decode_args = saved


def time_split_kernel(p: Prepared, steps: int, warmup: int) -> float:
    """Average duration (µs) of fd_decode's split kernel alone (its split
    stage through fd_decode_stages: the same kernel and plan as inside the
    step): HIP events on its stream around `steps` back-to-back launches,
    divided by `steps`."""
    run = p.split_stage
    settle(run)
    for i in range(warmup):
        run(i)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(p.stream)
    for i in range(steps):
        run(i)
    end.record(p.stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps * 1e3


def time_partial_formats(w: workloads.Workload, dev: torch.device, steps: int, warmup: int) -> dict:
    """The two partial formats the pages derive, on one workload with fixed
    splits: LSE pair (fd_decode_split + fd_combine) against the m/l/o triple
    (fd_decode_split_mlo + fd_combine_mlo).  HIP events over the timed region."""
    p = Prepared(w, dev)
    B, L = p.B, p.L
    batch, hq, d = w.batch, w.heads_q, w.head_dim
    shape = (batch, hq, B)
    m_part = torch.empty(shape, dtype=torch.float32, device=dev)
    l_part = torch.empty(shape, dtype=torch.float32, device=dev)
    lib, P = p.lib, ctypes.c_void_p
    sp = ctypes.c_void_p(p.stream.cuda_stream)
    mlo_args = []
    for a in p.split_args:  # same arguments, m_part and l_part in place of lse_part
        mlo_args.append(tuple(a[:14]) + (P(m_part.data_ptr()), P(l_part.data_ptr()), sp))
    comb_lse = (P(p.o_part.data_ptr()), P(p.lse_part.data_ptr()), batch, hq, B, d,
                P(p.o.data_ptr()), p.out_code, P(p.lse.data_ptr()), sp)
    comb_mlo = (P(p.o_part.data_ptr()), P(m_part.data_ptr()), P(l_part.data_ptr()), batch, hq,
                B, d, P(p.o.data_ptr()), p.out_code, P(p.lse.data_ptr()), sp)

    def region(fn) -> float:
        settle(fn)
        for i in range(warmup):
            fn(i)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(p.stream)
        for i in range(steps):
            fn(i)
        end.record(p.stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps * 1e3

    def check(rc):
        if rc != fd.OK:
            raise fd.FDError(rc, fd.last_error())

    def lse_route(i):
        check(lib.fd_decode_split(*p.split_args[i % p.copies]))
        check(lib.fd_combine(*comb_lse))

    def mlo_route(i):
        check(lib.fd_decode_split_mlo(*mlo_args[i % p.copies]))
        check(lib.fd_combine_mlo(*comb_mlo))

    out = {"workload": w.name, "num_splits": B, "split_len": L,
           "lse_route_us": round(region(lse_route), 2),
           "mlo_route_us": round(region(mlo_route), 2),
           "lse_split_us": round(region(lambda i: check(lib.fd_decode_split(
               *p.split_args[i % p.copies]))), 2),
           "mlo_split_us": round(region(lambda i: check(lib.fd_decode_split_mlo(
               *mlo_args[i % p.copies]))), 2),
           "lse_combine_us": round(region(lambda i: check(lib.fd_combine(*comb_lse))), 2),
           "mlo_combine_us": round(region(lambda i: check(lib.fd_combine_mlo(*comb_mlo))), 2),
           "partial_bytes_lse": batch * hq * B * (d + 1) * 4,
           "partial_bytes_mlo": batch * hq * B * (d + 2) * 4}
    p.free()
    return out


def time_paged(w: workloads.Workload, dev: torch.device, page_size: int, steps: int,
               warmup: int) -> dict:
    """fd_decode_paged on a workload laid out in pages of page_size tokens
    (seeded page permutation), library plan, against the same step over the
    contiguous cache.  Wall clock over `steps` steps; enough page-cache copies
    that consecutive steps read different memory."""
    inp = workloads.generate(w)
    lens = inp["kv_lens"]  # None (every sequence full) as in the contiguous run
    if lens is None and inp["max_kv_len"] % page_size:
        raise ValueError("page_size must divide the cache length of a uniform workload")
    pg = workloads.paginate(inp, page_size, seed=page_size)
    kvb = workloads.kv_bytes(w, lens)
    footprint = pg["k_pages"].numel() * pg["k_pages"].element_size() * 2
    copies = 1 if footprint < (64 << 20) else max(2, min(16, math.ceil((1 << 30) / footprint) + 1))
    q = inp["q"].to(dev)
    kl = None if lens is None else lens.to(dev)
    bt = pg["block_table"].to(dev)
    pages = [(pg["k_pages"].to(dev), pg["v_pages"].to(dev)) for _ in range(copies)]
    batch, hq, hkv, d = w.batch, w.heads_q, w.heads_kv, w.head_dim
    ps, max_pages, num_pages = page_size, pg["max_pages"], pg["num_pages"]
    B, L = (w.num_splits, 0) if w.num_splits else (0, 0)  # L 0: the library's chunking
    out_dt = workloads.TORCH_DTYPES[w.out_dtype]
    o = torch.empty((batch, hq, d), dtype=out_dt, device=dev)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    need = fd.decode_workspace_bytes(batch, hq, hkv, max_pages * ps, d, q.dtype, kl is not None,
                                     B, L)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    lib, P = fd.library(), ctypes.c_void_p
    stream = torch.cuda.current_stream(dev)
    sp = P(stream.cuda_stream)
    code = {torch.float32: fd.F32, torch.float16: fd.F16, torch.bfloat16: fd.BF16}
    kl_p = None if kl is None else P(kl.data_ptr())
    args = [(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(bt.data_ptr()), kl_p, batch,
             hq, hkv, ps, max_pages, num_pages, d, code[q.dtype], code[out_dt],
             ctypes.c_float(w.scale), B, L, P(o.data_ptr()), P(lse.data_ptr()), P(ws.data_ptr()),
             need, sp) for k, v in pages]

    def step(i):
        rc = lib.fd_decode_paged(*args[i % copies])
        if rc != fd.OK:
            raise fd.FDError(rc, fd.last_error())

    settle(step)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    del pages, q, kl, bt, o, lse, ws
    return {"page_size": ps, "pages": num_pages, "us_per_step": round(us, 2),
            "kv_GBps": round(kvb / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(kvb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


CASCADE = workloads.Workload("cascade_gqa_bf16_b16_hq64_hkv8_d128_prefix16384_suffix512_4096",
                             batch=16, heads_q=64, heads_kv=8, head_dim=128, max_kv_len=4096,
                             dtype="bf16", out_dtype="bf16", seed=8, ragged=(512, 4096))
CASCADE_PREFIX = 16384


def time_cascade(steps: int, warmup: int, dev: torch.device, materialised: bool = True) -> dict:
    """Shared-prefix decode (fd_decode_cascade: one prefix copy for the batch)
    against fd_decode over the materialised per-sequence caches (prefix +
    suffix each).  Wall clock over `steps` steps, several input copies so that
    consecutive steps read different memory (within a step the prefix is
    shared by design)."""
    w = CASCADE
    c = workloads.cascade(w, CASCADE_PREFIX)
    cc = workloads.cascade_concat(c)
    lens = c["suffix_lens"]
    row = w.heads_kv * w.head_dim * 2 * 2  # K+V bytes of one token, all KV heads
    logical = int(cc["kv_lens"].sum()) * row      # what the sequences attend over
    unique = (CASCADE_PREFIX + int(lens.sum())) * row  # distinct K/V in the cascade
    lib, P = fd.library(), ctypes.c_void_p
    sp = P(torch.cuda.current_stream(dev).cuda_stream)
    batch, hq, hkv, d = w.batch, w.heads_q, w.heads_kv, w.head_dim
    q = c["q"].to(dev)
    o = torch.empty((batch, hq, d), dtype=q.dtype, device=dev)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)

    def region(run, copies):
        settle(lambda i: run(i % copies))
        for i in range(warmup):
            run(i % copies)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run(i % copies)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e6

    def check(rc):
        if rc != fd.OK:
            raise fd.FDError(rc, fd.last_error())

    # cascade
    footprint = unique
    copies = max(2, min(16, math.ceil((1 << 30) / footprint) + 1))
    sl = lens.to(dev)
    bufs = [tuple(c[n].to(dev) for n in ("k_prefix", "v_prefix", "k_suffix", "v_suffix"))
            for _ in range(copies)]
    need = fd.cascade_workspace_bytes(batch, hq, hkv, CASCADE_PREFIX, c["max_suffix_len"], d,
                                      q.dtype, True)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    cargs = [(P(q.data_ptr()), P(kp.data_ptr()), P(vp.data_ptr()), CASCADE_PREFIX,
              P(ks.data_ptr()), P(vs.data_ptr()), P(sl.data_ptr()), batch, hq, hkv,
              c["max_suffix_len"], d, fd.BF16, fd.BF16, ctypes.c_float(w.scale),
              P(o.data_ptr()), P(lse.data_ptr()), P(ws.data_ptr()), need, sp)
             for kp, vp, ks, vs in bufs]
    us_c = region(lambda i: check(lib.fd_decode_cascade(*cargs[i])), copies)
    del bufs, cargs, ws
    torch.cuda.empty_cache()
    if not materialised:
        return {"workload": w.name, "prefix_len": CASCADE_PREFIX,
                "suffix_tokens": int(lens.sum()), "cascade_us_per_step": round(us_c, 2),
                "logical_kv_bytes": logical, "unique_kv_bytes": unique,
                "prefix_kv_bytes": CASCADE_PREFIX * row,
                "cascade_unique_GBps": round(unique / (us_c * 1e-6) / 1e9, 1)}
    # plain decode over the materialised caches
    copies_p = max(2, min(16, math.ceil((1 << 30) / logical) + 1))
    kl = cc["kv_lens"].to(dev)
    pbufs = [(cc["k"].to(dev), cc["v"].to(dev)) for _ in range(copies_p)]
    need = fd.decode_workspace_bytes(batch, hq, hkv, cc["max_kv_len"], d, q.dtype, True)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    pargs = [(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(kl.data_ptr()), batch, hq,
              hkv, cc["max_kv_len"], d, fd.BF16, fd.BF16, ctypes.c_float(w.scale), 0, 0,
              P(o.data_ptr()), P(lse.data_ptr()), P(ws.data_ptr()), need, sp)
             for k, v in pbufs]
    us_p = region(lambda i: check(lib.fd_decode(*pargs[i])), copies_p)
    del pbufs, pargs, ws
    torch.cuda.empty_cache()
    return {"workload": w.name, "prefix_len": CASCADE_PREFIX,
            "suffix_tokens": int(lens.sum()), "cascade_us_per_step": round(us_c, 2),
            "materialised_us_per_step": round(us_p, 2), "speedup": round(us_p / us_c, 3),
            "logical_kv_bytes": logical, "unique_kv_bytes": unique,
            "cascade_unique_GBps": round(unique / (us_c * 1e-6) / 1e9, 1),
            "cascade_logical_GBps": round(logical / (us_c * 1e-6) / 1e9, 1),
            "materialised_GBps": round(logical / (us_p * 1e-6) / 1e9, 1)}


SHARDS = 8
SHARD = workloads.Workload("mha_bf16_b1_h32_d128_n8192_shard_of_65536", batch=1, heads_q=32,
                           heads_kv=32, head_dim=128, max_kv_len=65536 // SHARDS, dtype="bf16",
                           out_dtype="f32", seed=9)


def time_shard(steps: int, warmup: int, dev: torch.device) -> dict:
    """One GPU's share of the 64K-context workload sharded over SHARDS GPUs
    along the sequence: fd_decode over 8192 tokens with fp32 (o, LSE) output
    (what that GPU would send to the rows' owner), and the owner's fd_combine
    over SHARDS such pairs per row.  The exchange itself is not measured."""
    p = Prepared(SHARD, dev)
    t = time_steps(p, steps, warmup)
    shard_us = t["wall_us_per_step"]
    batch, hq, d = SHARD.batch, SHARD.heads_q, SHARD.head_dim
    o_part = torch.zeros((batch, hq, SHARDS, d), dtype=torch.float32, device=dev)
    lse_part = torch.zeros((batch, hq, SHARDS), dtype=torch.float32, device=dev)
    o = torch.empty((batch, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    P = ctypes.c_void_p
    args = (P(o_part.data_ptr()), P(lse_part.data_ptr()), batch, hq, SHARDS, d, P(o.data_ptr()),
            fd.BF16, P(lse.data_ptr()), P(p.stream.cuda_stream))

    def comb(i):
        rc = p.lib.fd_combine(*args)
        if rc != fd.OK:
            raise fd.FDError(rc, fd.last_error())

    settle(comb)
    for i in range(warmup):
        comb(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(p.stream)
    for i in range(steps):
        comb(i)
    end.record(p.stream)
    torch.cuda.synchronize()
    comb_us = start.elapsed_time(end) / steps * 1e3
    out = {"workload": SHARD.name, "shards": SHARDS, "plan": p.plan, "num_splits": p.B,
           "shard_us_per_step": round(shard_us, 2),
           "shard_kv_GBps": round(p.kv_bytes / (shard_us * 1e-6) / 1e9, 1),
           "owner_combine_us": round(comb_us, 2),
           "exchange_bytes_per_gpu": batch * hq * (d + 1) * 4}
    p.free()
    return out


# Group sizes past one 16-query tile, up to multi-query attention (bf16/fp16
# on the matrix cores): the tiled kernel's fixed splits without lengths, the
# token-balanced plan with ragged lengths.
GROUPS = [
    workloads.Workload("mqa_bf16_b32_hq64_hkv1_d128_n8192", batch=32, heads_q=64, heads_kv=1,
                       head_dim=128, max_kv_len=8192, dtype="bf16", out_dtype="bf16", seed=8),
    workloads.Workload("gqa32_bf16_b16_hq64_hkv2_d128_n16384", batch=16, heads_q=64, heads_kv=2,
                       head_dim=128, max_kv_len=16384, dtype="bf16", out_dtype="bf16", seed=9),
    workloads.Workload("mqa_bf16_b32_hq128_hkv1_d128_ragged512_16384", batch=32, heads_q=128,
                       heads_kv=1, head_dim=128, max_kv_len=16384, dtype="bf16", out_dtype="bf16",
                       seed=10, ragged=(512, 16384)),
    workloads.Workload("gqa32_bf16_b16_hq64_hkv2_d128_ragged512_32768", batch=16, heads_q=64,
                       heads_kv=2, head_dim=128, max_kv_len=32768, dtype="bf16", out_dtype="bf16",
                       seed=11, ragged=(512, 32768)),
    workloads.Workload("mqa_f16_b32_hq64_hkv1_d64_ragged512_16384", batch=32, heads_q=64,
                       heads_kv=1, head_dim=64, max_kv_len=16384, dtype="f16", out_dtype="f16",
                       seed=12, ragged=(512, 16384)),
    workloads.Workload("mqa_f16_b32_hq64_hkv1_d64_n8192", batch=32, heads_q=64, heads_kv=1,
                       head_dim=64, max_kv_len=8192, dtype="f16", out_dtype="f16", seed=14),
]


def time_groups(steps: int, warmup: int, dev: torch.device) -> dict:
    """Decode steps of the large-group workloads, with the plan each takes."""
    out = {}
    res = {"workload": "query_groups_32_to_128", "cases": out}
    for w in GROUPS:
        p = Prepared(w, dev)
        t = time_steps(p, steps, warmup)
        su = time_split_kernel(p, steps, warmup)
        r = summarize(p, t, su)
        r["waves_per_group"] = p.dplan["waves_per_group"]
        r["query_tiles_per_group"] = p.dplan["query_tiles"]
        out[w.name] = r
        p.free()
        del p
        torch.cuda.empty_cache()
    return res


RAGGED_MHA = [
    workloads.Workload("mha_bf16_b8_h32_d128_ragged512_32768", batch=8, heads_q=32, heads_kv=32,
                       head_dim=128, max_kv_len=32768, dtype="bf16", out_dtype="bf16", seed=15,
                       ragged=(512, 32768)),
    workloads.Workload("mha_f16_b4_h16_d256_ragged1024_32768", batch=4, heads_q=16, heads_kv=16,
                       head_dim=256, max_kv_len=32768, dtype="f16", out_dtype="f16", seed=16,
                       ragged=(1024, 32768)),
]


def time_ragged_mha(steps: int, warmup: int, dev: torch.device) -> dict:
    """Decode steps of ragged multi-head batches: the library's plan (the
    token-balanced partition on the vector kernel) and, on the same inputs,
    the fixed splits the library picks for ragged lengths."""
    out = {}
    for w in RAGGED_MHA:
        p = Prepared(w, dev)
        t = time_steps(p, steps, warmup)
        su = time_split_kernel(p, steps, warmup)
        r = summarize(p, t, su)
        host, B = p.host, p.B
        p.free()
        del p
        torch.cuda.empty_cache()
        f = Prepared(w, dev, B, host=host)
        tf = time_steps(f, steps, warmup)
        r["fixed_splits"] = {"num_splits": f.B, "split_len": f.L,
                             "us_per_step": round(tf["wall_us_per_step"], 2)}
        r["speedup_vs_fixed_splits"] = round(tf["wall_us_per_step"] / t["wall_us_per_step"], 3)
        f.free()
        del f, host
        torch.cuda.empty_cache()
        out[w.name] = r
    return {"workload": "mha_ragged_bf16_d128_and_f16_d256", "cases": out}


def cpu_baseline(p: Prepared, budget_s: float) -> dict:
    """The fp64 oracle on the host cores, on whole decode steps of the same
    workload, repeated until about budget_s seconds of wall time."""
    import oracle  # test infrastructure: used only for this reported baseline

    w, inp = p.w, p.host
    lens = inp["kv_lens"]
    args = (w.dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]), workloads.raw(inp["v"]),
            None if lens is None else lens.numpy())
    threads = oracle.threads()
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.attention(*args, scale=w.scale)
        reps += 1
        if time.perf_counter() - t0 >= budget_s or reps >= 50:
            break
    wall = time.perf_counter() - t0
    us = wall / reps * 1e6
    out = {"value": round(p.kv_bytes / (us * 1e-6) / 1e9, 3), "unit": "GB/s", "cores": threads,
           "kind": "oracle", "us_per_step": round(us, 1),
           "sample": f"{reps} whole decode step(s) of {w.name} (every row, fp64, OpenMP over "
                     f"(sequence, head)), {wall:.1f} s wall"}
    # the same oracle on one thread, for reference, over the first sequences
    # of the batch up to >= 256 MiB of K/V (the whole step when smaller)
    nb, sample_bytes = 0, 0
    row = w.heads_kv * w.head_dim * 2 * inp["k"].element_size()
    while nb < w.batch and sample_bytes < (256 << 20):
        sample_bytes += row * (p.n_max if lens is None else int(lens[nb]))
        nb += 1
    sub = (w.dtype, workloads.raw(inp["q"][:nb]), workloads.raw(inp["k"][:nb]),
           workloads.raw(inp["v"][:nb]), None if lens is None else lens[:nb].numpy())
    oracle.set_threads(1)
    try:
        t1 = time.perf_counter()
        oracle.attention(*sub, scale=w.scale)
        one = time.perf_counter() - t1
    finally:
        oracle.set_threads(threads)
    what = (f"1 whole decode step of {w.name}" if nb == w.batch else
            f"sequences 0..{nb - 1} of one decode step of {w.name} ({sample_bytes} bytes of K/V)")
    out["one_thread"] = {"value": round(sample_bytes / one / 1e9, 3), "unit": "GB/s",
                         "us_per_step": round(one * 1e6 * p.kv_bytes / sample_bytes, 1),
                         "sample": f"{what} on 1 thread; us_per_step scaled to the whole step "
                                   "by K/V bytes"}
    return out


def cpu_baseline_workload(p: Prepared, one_thread: bool) -> dict:
    """Part of the cpu_baseline leg: the fp64 oracle over one whole decode step
    of p's workload, on the same host inputs, by wall clock, on the host cores
    and, when asked, on one thread (a reported baseline beside the GPU's step,
    never its target)."""
    import oracle  # test infrastructure: used only for this reported baseline

    w, inp = p.w, p.host
    lens = inp["kv_lens"]
    args = (w.dtype, workloads.raw(inp["q"]), workloads.raw(inp["k"]), workloads.raw(inp["v"]),
            None if lens is None else lens.numpy())
    threads = oracle.threads()
    t0 = time.perf_counter()
    oracle.attention(*args, scale=w.scale)
    wall = time.perf_counter() - t0
    out = {"us_per_step": round(wall * 1e6, 1), "cores": threads, "kind": "oracle",
           "kv_GBps": round(p.kv_bytes / wall / 1e9, 3)}
    if one_thread:
        oracle.set_threads(1)
        try:
            t1 = time.perf_counter()
            oracle.attention(*args, scale=w.scale)
            one = time.perf_counter() - t1
        finally:
            oracle.set_threads(threads)
        out["one_thread_us_per_step"] = round(one * 1e6, 1)
    return out


def traffic_from_profile(name: str) -> dict | None:
    """HBM bytes per split-kernel launch from a committed rocprofv3 counter
    summary, when it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != build.source_hash(rec.get("kernel", "")):
        return None
    return rec


def summarize(p: Prepared, t: dict, split_us: float | None) -> dict:
    us = t["wall_us_per_step"]
    out = {"us_per_step": round(us, 2), "event_us_median": round(t["event_us_median"], 2),
           "plan": p.plan, "route": p.dplan["route"], "split_kernel": p.dplan["kernel"],
           "kv_bytes": p.kv_bytes}
    if not p.balanced:
        out["num_splits"], out["split_len"] = p.B, p.L
    if p.copies > 1:
        gbs = p.kv_bytes / (us * 1e-6) / 1e9
        out["kv_GBps"] = round(gbs, 1)
        out["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    else:
        out["note"] = "cache-resident (0.5 MiB); µs only"
        # launch-bound: also the step's GPU-side time with the host overhead
        # taken out by graph replay
        out["graph_us_per_step"] = round(time_graph_steps(p, 200), 2)
    if split_us is not None:
        out["split_kernel_us"] = round(split_us, 2)
        out["split_kernel_GBps"] = round(p.split_bytes / (split_us * 1e-6) / 1e9, 1)
    prof = traffic_from_profile(p.w.name)
    if prof is not None:
        out["split_traffic_bytes_per_launch"] = prof["hbm_bytes_per_launch"]
        out["split_algorithmic_bytes_per_launch"] = p.split_bytes
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, help="headline workload (1-5)")
    ap.add_argument("--num-splits", type=int, default=0, help="override the split count")
    ap.add_argument("--only", action="store_true", help="time the headline workload only")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="oracle seconds (0: skip)")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--section", choices=("cascade", "paged", "shard", "groups", "ragged_mha"), default=None,
                    help="time only this section of the full run and print its JSON (profiling)")
    ap.add_argument("--library", default=None,
                    help="time a tuning variant (decode_attention_03_amd/variants/NAME.so, built "
                         "with python -m decode_attention_03_amd.build NAME -DKNOB=value) "
                         "instead of libfd.so; the JSON line names it")
    args = ap.parse_args()
    variant = None
    if args.library:
        rec = fd.use_variant(os.path.abspath(args.library))
        variant = {"path": os.path.relpath(os.path.abspath(args.library), ROOT),
                   "flags": rec.get("flags")}

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(each GPU would run its own independent decode); run with --gpus 1",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    # bring up the HIP runtime and this device's context before any threaded
    # CPU work (the input generator runs a thread pool)
    torch.cuda.init()
    torch.empty(1, device=dev)
    torch.cuda.synchronize(dev)

    if args.copy_probe:
        # a streaming elementwise kernel (out = -in) that reads and writes
        # exactly copy_probe bytes per dispatch: the scale for HBM counters
        n = args.copy_probe // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 5 dispatches reading and writing {args.copy_probe} bytes each")
        return 0

    if args.section:
        if args.section == "cascade":
            sec = time_cascade(args.steps, args.warmup, dev, materialised=False)
        elif args.section == "shard":
            sec = time_shard(args.steps, args.warmup, dev)
        elif args.section == "groups":
            sec = time_groups(args.steps, args.warmup, dev)
        elif args.section == "ragged_mha":
            sec = time_ragged_mha(args.steps, args.warmup, dev)
        else:  # the paged step of the ragged grouped workload, 16-token pages
            w = workloads.WORKLOADS[4]
            sec = {"workload": w.name, **time_paged(w, dev, 16, args.steps, args.warmup)}
        print(json.dumps({"section": args.section, "library_variant": variant, **sec}),
              flush=True)
        return 0

    head = workloads.WORKLOADS[args.config]
    p = Prepared(head, dev, args.num_splits)
    t = time_steps(p, args.steps, args.warmup)
    split_us = time_split_kernel(p, args.steps, args.warmup)
    log(f"[bench] {head.name}: {t}")
    us = t["wall_us_per_step"]
    gbs = p.kv_bytes / (us * 1e-6) / 1e9
    achieved = p.split_bytes / (split_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": f"split ({p.dplan['kernel']})", "kernel_us": round(split_us, 2),
                "algorithmic_bytes_per_launch": p.split_bytes}
    prof = traffic_from_profile(head.name)
    if prof is not None:
        roofline["traffic"] = prof.get("hbm_bytes_per_launch")
    cpu = cpu_baseline(p, args.cpu_budget) if args.cpu_budget > 0 else None
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": SETTLE_MS,
        "ms_per_step": round(us / 1e3, 5),
        "us_per_step": round(us, 2),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # storage and matrix-core operand type; every sum accumulates in fp32
        "dtype": head.dtype,
        "accumulate_dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head.name, "batch": head.batch, "heads_q": head.heads_q,
                   "heads_kv": head.heads_kv, "head_dim": head.head_dim,
                   "max_kv_len": p.n_max, "in_dtype": head.dtype, "out_dtype": head.out_dtype,
                   "plan": p.plan, "route": p.dplan["route"],
                   "split_kernel": p.dplan["kernel"], "num_splits": None if p.balanced else p.B,
                   "split_len": None if p.balanced else p.L, "kv_bytes_per_step": p.kv_bytes,
                   "input_copies": p.copies, "parallelism": "single-gpu"},
        "inputs_sha256": workloads.digest(p.host),
        "timing": {k: round(v, 2) for k, v in t.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if variant is not None:  # never the product library: say which build was timed
        result["library_variant"] = variant
    p.free()
    del p
    torch.cuda.empty_cache()
    if not args.only:
        others = {}

        def run_workload(c):
            w = workloads.WORKLOADS[c]
            q = Prepared(w, dev)
            tt = time_steps(q, args.steps, args.warmup)
            su = time_split_kernel(q, args.steps, args.warmup)
            others[w.name] = summarize(q, tt, su)
            others[w.name]["inputs_sha256"] = workloads.digest(q.host)
            log(f"[bench] {w.name}: {others[w.name]}")
            if cpu is not None:  # the oracle beside it: one step (one thread too up to 1 GiB)
                cw = cpu_baseline_workload(q, one_thread=q.kv_bytes <= (1 << 30))
                cpu.setdefault("workloads", {})[w.name] = cw
                log(f"[bench] oracle {w.name}: {cw}")
            q.free()
            del q
            torch.cuda.empty_cache()

        # The 8 GiB workload streams for over a second; sections timed right
        # after it ran up to 6-10 % slow for a few hundred milliseconds
        # (measured), so it runs last.
        late = [c for c in sorted(workloads.WORKLOADS)
                if c != args.config and workloads.WORKLOADS[c].max_kv_len >= 131072]
        for c in sorted(workloads.WORKLOADS):
            if c != args.config and c not in late:
                run_workload(c)
        result["workloads"] = others
        # the m/l/o partial format against the LSE pair, on the long-context
        # workload (16 splits per row, so the combine stage does real work)
        pf = time_partial_formats(workloads.WORKLOADS[3], dev, args.steps, args.warmup)
        log(f"[bench] partial formats: {pf}")
        result["partial_formats"] = pf
        torch.cuda.empty_cache()
        # the paged K/V cache (block-table indirection) on the multi-head and
        # the ragged grouped workloads, 16-token pages
        paged = {}
        for c in (2, 4):
            w = workloads.WORKLOADS[c]
            r = time_paged(w, dev, 16, args.steps, args.warmup)
            contiguous = (result if c == args.config else others[w.name])["us_per_step"]
            r["contiguous_us_per_step"] = contiguous
            paged[w.name] = r
            log(f"[bench] paged {w.name}: {r}")
            torch.cuda.empty_cache()
        result["paged"] = paged
        # shared-prefix decode against the same step over materialised caches
        casc = time_cascade(args.steps, args.warmup, dev)
        log(f"[bench] cascade: {casc}")
        result["cascade"] = casc
        torch.cuda.empty_cache()
        # one GPU's share of the long-context workload under sequence sharding
        shard = time_shard(args.steps, args.warmup, dev)
        log(f"[bench] shard: {shard}")
        result["shard"] = shard
        # groups past one matrix-core tile, up to multi-query attention
        groups = time_groups(args.steps, args.warmup, dev)
        log(f"[bench] groups: {groups}")
        result["groups"] = groups
        # ragged multi-head batches: balanced pieces on the vector kernel
        rm = time_ragged_mha(args.steps, args.warmup, dev)
        log(f"[bench] ragged_mha: {rm}")
        result["ragged_mha"] = rm
        for c in late:
            run_workload(c)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

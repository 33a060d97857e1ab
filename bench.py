#!/usr/bin/env python3
"""Benchmark: selected-cell INT8 decode attention (chunk + merge) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-batched] [--no-cpu]

Workload of the headline line: the pages' kernel point (Strata PR #2220,
"Kernel (chunk kernel + merge, synthetic INT8 pools, permuted page table,
200 calls)"): one sequence, one KV head, 12 query heads, head_dim 256,
32,768-cell INT8 pool behind a permuted page table, 2,051 selected cells,
chunk 256.  One step = four calls of sda_decode_attn_batch, one per query
count 1, 2, 3, 4 (the page's table axis), launched back to back on one
stream (each call: the chunk kernel, then the merge kernel).  Inputs are
generated on the host, uploaded, and resident in HBM before the timed
region.

Printed: one JSON line.  value = selected cells per second over the step;
roofline = the chunk kernel's algorithmic HBM bytes (520 B per selected cell,
4 B per touched page-table entry, the fp32 queries) over its mean duration,
timed with HIP events on the launch stream; cpu_baseline = the
fp64 CPU oracle on the same workload; "batched" = the three batched
workloads (256 x 2,051 cells x 4 q, 64 x 16,384 x 2 q, 32 x 131,072 x 4 q)
measured the same way with a cache flush between calls; the two passes are
also timed as separate calls for reference; "prompt_attention" = the prompt
workload of the same pages (32K-cell INT8 context, 2,048 causal queries x 12
heads) through sda_prompt_attn_batch, with its matrix-core roofline;
"kv_append" = the INT8 KV append of 64 x 2,048 new rows into 32K-cell pools
through sda_kv_append_batch, cold, with its HBM roofline; "qsa_selection" =
the QSA block scorer and top-k selection (64 instances x 512 blocks of 256
cells, top 64) through sda_qsa_block_scores and sda_qsa_select, cold, with
the scorer's HBM roofline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = ("selected KV cells/s and HBM GB/s (chunk+merge), µs/call at 2,051 cells "
          "× 1–4 q")
HBM_PEAK_GBS = 8000.0
# chunk + merge on RTX 2080 Ti (sm_75), attn_chunk_q8_v3_kernel, 2,051 cells (Strata PR #2220)
PAGES_V3_US = {1: 34.5, 2: 41.0, 3: 73.0, 4: 84.9}
PAGES_DEFAULT_US = {1: 51.6, 2: 78.5, 3: 110.0, 4: 145.6}
# the same table's 600-cell rows (same page and setup)
PAGES_600_V3_US = {1: 28.6, 2: 32.8, 3: 33.5, 4: 33.3}
PAGES_600_DEFAULT_US = {1: 45.9, 2: 74.6, 3: 105.5, 4: 136.9}


# HBM bytes per launch measured with two rocprofv3 counter runs (FETCH_SIZE,
# then WRITE_SIZE, caches evicted before each call), each scaled by what the
# counter reads for a plain 256 MiB device copy (FETCH_SIZE x 2.0,
# WRITE_SIZE x 1.0): the headline chunk kernel (n_q = 4), the prompt kernel
# and the KV append kernel.  The summaries with the commands are under
# profiles/.  A figure holds only for the kernel sources it was taken on
# (the SHA-256 of their code, comments left out); a changed source reports
# null.
MEASURED_TRAFFIC = {
    "chunk": {"sources": ("decode_attention_sparse_amd/csrc/chunk_mfma.hip",
                          "decode_attention_sparse_amd/csrc/sda_internal.h",
                          "decode_attention_sparse_amd/csrc/sda_api.hip"),
              "sources_sha256": "5725351ac2ccf994f9db0bb3ae2a8d48e30566c829987aa6caceea6f03324df4", "fetch_bytes": 1879040, "write_bytes": 1634688},
    "prompt": {"sources": ("decode_attention_sparse_amd/csrc/chunk_mfma.hip",
                           "decode_attention_sparse_amd/csrc/sda_internal.h",
                           "decode_attention_sparse_amd/csrc/sda_api.hip"),
               "sources_sha256": "5725351ac2ccf994f9db0bb3ae2a8d48e30566c829987aa6caceea6f03324df4", "fetch_bytes": 161506768, "write_bytes": 25264128},
    "append": {"sources": ("decode_attention_sparse_amd/csrc/kv_append.hip",
                           "decode_attention_sparse_amd/csrc/sda_internal.h",
                           "decode_attention_sparse_amd/csrc/sda_api.hip"),
               "sources_sha256": "95af2b33a412217f20e26e1ecd52a5cdb0672137219aa000e2f965bfc4de32d0", "fetch_bytes": 268717967, "write_bytes": 68157440},
    "qsa": {"sources": ("decode_attention_sparse_amd/csrc/qsa_select.hip",
                        "decode_attention_sparse_amd/csrc/sda_internal.h",
                        "decode_attention_sparse_amd/csrc/sda_api.hip"),
            "sources_sha256": "3d99c9d643b4c40526849f675eee0e985dba29066397c14714fb08fea6227f44", "fetch_bytes": 68185156, "write_bytes": 262517},
}


def sources_sha256(files) -> str:
    """SHA-256 of the sources' code: comments removed and white space
    collapsed, so that editing a comment keeps a measurement valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for f in files:
        with open(os.path.join(root, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()


def measured_traffic(kernel):
    """Measured HBM bytes per launch of `kernel` ("chunk", "prompt",
    "append", "qsa"), or None when its sources differ from those the counters
    were taken on."""
    m = MEASURED_TRAFFIC[kernel]
    if not m["sources_sha256"] or sources_sha256(m["sources"]) != m["sources_sha256"]:
        return None
    return m["fetch_bytes"] + m["write_bytes"]


def algorithmic_bytes(x) -> int:
    """Bytes the method must move for one chunk pass over inputs x: K and V
    code rows (256 B each), K and V scales (2 B each) and the list entry (4 B)
    per selected cell, 4 B per distinct page-table entry touched, and the
    fp32 query rows."""
    cells = int(np.sum(x.n_sel))
    pages = 0
    for i in range(x.sel.shape[0]):
        s = x.sel[i, : x.n_sel[i]]
        pages += int(np.unique(s >> 4).size)
    q_bytes = int(np.prod(x.q.shape)) * 4
    return cells * 520 + pages * 4 + q_bytes


def out_bytes(x) -> int:
    n_inst, n_q, nh, D = x.q.shape
    return n_inst * n_q * nh * (D + 1) * 4


class Case:
    """One workload resident on the GPU, with its buffers and timing hooks."""

    def __init__(self, x, chunk, interleave_scales=True):
        import torch
        from decode_attention_sparse_amd import api
        self.api, self.torch = api, torch
        self.x, self.chunk = x, chunk
        # the pool layout used for every measured workload: (K, V) scale pairs
        # interleaved per cell, so a gathered cell's two scales share a sector
        self.pool, self.dev = api.to_device(x, interleave_scales=interleave_scales)
        n_inst, n_q, nh, D = x.q.shape
        self.max_sel = int(x.sel.shape[1])
        self.out = torch.empty((n_inst, n_q, nh, D), device="cuda")
        self.lse = torch.empty((n_inst, n_q, nh), device="cuda")
        self.ws = api.workspace(n_inst, n_q, nh, self.max_sel, chunk)
        self.fused_chunk = api.fused_chunk_cells(n_inst, self.max_sel, chunk)
        # whether the call is one chunk-kernel launch that writes the outputs
        self.single_launch = api.fused_single_launch(n_inst, n_q, nh, self.max_sel, chunk)
        self.chunk_bytes = algorithmic_bytes(x)  # the chunk kernel's
        self.bytes = self.chunk_bytes + out_bytes(x)  # one whole call
        self.cells = int(np.sum(x.n_sel))

    def call(self):
        """The entry point a caller uses: sda_decode_attn_batch (chunk kernel,
        then merge kernel)."""
        d = self.dev
        self.api.decode_attn_batch(self.pool, d["page_table"], d["sel"], d["n_sel"], self.max_sel,
                                   d["q"], self.x.softmax_scale, self.chunk, self.out, self.lse,
                                   ws=self.ws)

    # The two kernels of a call, launched on their own exactly as the call
    # launches them: at the chunk size the call uses (finer than the
    # caller's for small grids, see sda_fused_chunk_cells).
    def chunk_pass(self, chunk=None):
        d = self.dev
        self.api.chunk_batch(self.pool, d["page_table"], d["sel"], d["n_sel"], self.max_sel, d["q"],
                             self.x.softmax_scale, chunk or self.fused_chunk, self.ws)

    def merge_pass(self, chunk=None):
        self.api.merge_batch(self.dev["n_sel"], self.max_sel, chunk or self.fused_chunk, self.ws,
                             self.out, self.lse)


def time_calls(cases, iters, flush=None):
    """Eager whole calls (Case.call): every case `iters` times, HIP events on
    the launch stream around each call, an optional cache flush before each
    call outside the events.  Returns per-case lists of ms."""
    import torch
    evs = []
    for _ in range(iters):
        row = []
        for c in cases:
            if flush is not None:
                flush()
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            c.call()
            e1.record()
            row.append((e0, e1))
        evs.append(row)
    torch.cuda.synchronize()
    res = [[] for _ in cases]
    for row in evs:
        for k, (e0, e1) in enumerate(row):
            res[k].append(e0.elapsed_time(e1))
    return res


def warm_up(cases, flush, min_ms=50.0):
    """Untimed cold calls until at least min_ms of them have run (at least
    five).  After setup, the first 10-20 ms of sustained HBM traffic run up to
    40 % slower (on the dense workload, cold calls start above 600 us and
    settle near 440 us after about 20 calls), so timing starts after that.
    Returns the number of calls run per case."""
    total, n = 0.0, 0
    while total < min_ms or n < 5:
        total += sum(sum(s) for s in time_calls(cases, 5, flush=flush))
        n += 5
    return n


def time_passes(cases, iters, flush=None):
    """The two kernels of a call as separate calls (sda_chunk_batch,
    sda_merge_batch), timed the same way.  Returns per-case lists of (chunk_ms, merge_ms)."""
    import torch
    evs = []
    for _ in range(iters):
        row = []
        for c in cases:
            if flush is not None:
                flush()
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record()
            c.chunk_pass()
            e1.record()
            c.merge_pass()
            e2.record()
            row.append((e0, e1, e2))
        evs.append(row)
    torch.cuda.synchronize()
    res = [[] for _ in cases]
    for row in evs:
        for k, (e0, e1, e2) in enumerate(row):
            res[k].append((e0.elapsed_time(e1), e1.elapsed_time(e2)))
    return res


def time_passes_at(cases, iters, chunk, flush=None):
    """time_passes at a given chunk size (the workload's stated one) instead
    of the call's."""
    import torch
    evs = []
    for _ in range(iters):
        row = []
        for c in cases:
            if flush is not None:
                flush()
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record()
            c.chunk_pass(chunk)
            e1.record()
            c.merge_pass(chunk)
            e2.record()
            row.append((e0, e1, e2))
        evs.append(row)
    torch.cuda.synchronize()
    return [[(e0.elapsed_time(e1), e1.elapsed_time(e2)) for (e0, e1, e2) in [r[k] for r in evs]]
            for k in range(len(cases))]


def graph_of(fn, reps):
    """Capture `reps` back-to-back calls of fn into one HIP graph, so that
    short kernels run without host launch gaps."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps):
    """Replay once untimed, then once between HIP events; ms per captured call."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def make_flush():
    """Cache eviction between timed calls: read a 1 GiB buffer (larger than
    L2 plus the 256 MB last-level cache).  The buffer is written once here;
    the flush itself only reads, so it leaves no dirty lines whose write-back
    would be charged to the next kernel."""
    import torch
    buf = torch.ones((1 << 30) // 4, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    buf.max()  # one read pass so the initial fill's dirty lines are gone
    torch.cuda.synchronize()

    def flush():
        buf.max()
    return flush


def summarize(case, calls, passes):
    tot = np.array(calls) * 1e3  # us per whole call
    ch = np.array([u[0] for u in passes]) * 1e3
    mg = np.array([u[1] for u in passes]) * 1e3
    med = float(np.median(tot))
    return {
        "us_per_call_median": round(med, 3),
        "us_per_call_p10": round(float(np.percentile(tot, 10)), 3),
        "us_per_call_p90": round(float(np.percentile(tot, 90)), 3),
        "chunk_us_mean": round(float(ch.mean()), 3),
        "merge_us_mean": round(float(mg.mean()), 3),
        "GBps_chunk_kernel": round(case.chunk_bytes / (ch.mean() * 1e-6) / 1e9, 1),
        "cells_per_s": round(case.cells / (med * 1e-6), 1),
        "GBps_algorithmic": round(case.bytes / (med * 1e-6) / 1e9, 1),
        "frac_hbm_peak": round(case.bytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }


def gather_ceiling():
    """Run probes/gather_ceiling (built with the library): cold-cache GB/s for
    random 256-byte rows, random 4 KB pages, sequential rows and a plain
    sequential read on this GPU.  None if the probe is not built."""
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode_attention_sparse_amd",
                       "probes", "gather_ceiling")
    if not os.path.exists(exe):
        print(f"# {exe} not built: no measured ceilings", file=sys.stderr)
        return None
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    if r.returncode != 0:
        print(f"# gather_ceiling failed ({r.returncode}): {r.stderr.strip()}", file=sys.stderr)
        return None
    return [json.loads(ln) for ln in r.stdout.splitlines() if ln.startswith("{")]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(xs, budget_s):
    """The fp64 oracle on the step's inputs, repeated for about budget_s."""
    import oracle
    cells, t0, reps = 0, time.perf_counter(), 0
    while True:
        for x in xs:
            oracle.attend(x)
            cells += int(np.sum(x.n_sel))
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(cells / el, 1), "unit": "selected cells/s", "cores": oracle.threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{reps} full steps of the headline workload (4 calls, n_q=1..4, "
                      f"2,051 cells each) in {el:.1f} s, fp64 C, OpenMP over query rows"}


# Prompt attention over the same pools (Strata PR #2220 page, closing note:
# the prompt attention parity test, INT8 32K context, 2,048 queries per
# prompt chunk, its reference the decode kernel): ms per chunk on the RTX
# 2080 Ti with the default and the v3 decode kernel (context, other hardware).
PROMPT_PAGES_MS = {"default": 71.5, "v3": 36.0}
INT8_MFMA_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix peak


def prompt_ops(x):
    """Algorithmic flops of one prompt call, and its (query row, visible
    cell) pairs: q.k and p.v take 2 * 256 flops each per pair."""
    limit = x.n_logical_pages * 16
    p = x.pos0[:, None].astype(np.int64) + np.arange(x.n_q)[None, :]
    pairs = int(np.clip(p + 1, 0, limit).sum()) * x.n_qheads
    return 4 * 256 * pairs, pairs


def prompt_case():
    import torch
    from decode_attention_sparse_amd import api, inputs
    x = inputs.make_prompt("prompt_int8_32k_2048q")
    pool, dev = api.to_device(x, interleave_scales=True)
    out = torch.empty(x.q.shape, device="cuda")
    lse = torch.empty(x.q.shape[:3], device="cuda")

    def call():
        api.prompt_attn_batch(pool, dev["page_table"], dev["pos0"], dev["q"], x.softmax_scale,
                              out, lse)
    return x, call


def prompt_section(reps, cpu_seconds):
    """The prompt workload: mean ms per call over a graph of `reps` calls
    (HIP events on the launch stream), its MFMA roofline, and the oracle on a
    bounded sample of positions."""
    x, call = prompt_case()
    for _ in range(3):
        call()
    g = graph_of(call, reps)
    ms = time_graph(g, reps)
    del g
    flops, pairs = prompt_ops(x)
    achieved = flops / (ms * 1e-3) / 1e12
    d = {
        "workload": x.workload,
        "config": {"instances": x.n_inst, "n_q": x.n_q, "n_qheads": x.n_qheads, "head_dim": 256,
                   "pool_cells": x.n_logical_pages * 16, "pos0": int(x.pos0[0]),
                   "mask": "causal: query t sees logical cells 0..pos0 + t",
                   "pool_layout": "int8 code rows; binary16 (K, V) scale pairs interleaved per cell"},
        "ms_per_call": round(ms, 4),
        "query_rows_x_visible_cells": pairs,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": INT8_MFMA_PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / INT8_MFMA_PEAK_TOPS, 4),
                     "traffic": measured_traffic("prompt"),
                     "kernel": "prompt_dma_kernel (96-row workgroups of eight compute waves, one per CU)",
                     "algorithmic_flops_per_launch": flops, "launch_ms_mean": round(ms, 4),
                     "note": "flops of the fp32-accurate products (q.k and p.v, 2 x 256 each per "
                             "row and visible cell) against the int8 matrix peak that runs them; "
                             "the digit splits issue 3 int8 products per q.k and 3 per p.v"},
        "pages_2080ti_ms_per_chunk": PROMPT_PAGES_MS,
        "speedup_vs_pages_v3": round(PROMPT_PAGES_MS["v3"] / ms, 2),
        "timing": f"{reps} calls captured in one HIP graph, HIP events around its replay",
    }
    if cpu_seconds > 0:
        import oracle
        t_ids = np.linspace(0, x.n_q - 1, 64).astype(np.int64)
        done, t0, k = 0, time.perf_counter(), 0
        while k < t_ids.size and time.perf_counter() - t0 < cpu_seconds:
            oracle.prompt_attend(x, 0, t_ids[k:k + 8])
            done += int(np.sum(np.minimum(int(x.pos0[0]) + t_ids[k:k + 8] + 1,
                                          x.n_logical_pages * 16))) * x.n_qheads
            k += 8
        el = time.perf_counter() - t0
        d["cpu_baseline"] = {
            "value": round(done / el, 1), "unit": "query rows x visible cells / s",
            "cores": oracle.threads(), "kind": "oracle",
            "ms_per_call_extrapolated": round(pairs / (done / el) * 1e3, 1),
            "sample": f"{k} of the {x.n_q} positions (12 rows each, evenly spaced) in {el:.1f} s, "
                      f"fp64 C, OpenMP over rows"}
    return d


def append_bytes(x) -> int:
    """Algorithmic bytes of one KV append: per new row the K and V values
    read (2 x 256 x 4 B) and the codes and scales written (2 x (256 + 2) B);
    4 B per touched page-table entry and per instance's pos0."""
    pages = 0
    for i in range(x.n_inst):
        c = int(x.pos0[i]) + np.arange(x.n_new)
        c = c[(c >= 0) & (c < x.page_table.shape[1] * 16)]
        pages += int(np.unique(c >> 4).size)
    return x.n_inst * x.n_new * (2 * 256 * 4 + 2 * 258) + pages * 4 + x.n_inst * 4


def append_case():
    import torch
    from decode_attention_sparse_amd import api, inputs
    x = inputs.make_append("kv_append_64inst_2048rows")
    cells = x.n_inst * x.pool_cells
    pool = api.Pool(torch.zeros((cells, 256), dtype=torch.int8, device="cuda"), None,
                    torch.zeros((cells, 256), dtype=torch.int8, device="cuda"), None,
                    scales=torch.zeros((cells, 2), dtype=torch.int16, device="cuda"))
    t = lambda a: torch.from_numpy(a).cuda()
    pt, pos0, kn, vn = t(x.page_table), t(x.pos0), t(x.k_new), t(x.v_new)

    def call():
        api.kv_append_batch(pool, pt, pos0, kn, vn)
    return x, call


def append_section(iters, flush):
    """The KV append workload: eager calls, caches evicted before each by the
    read flush, HIP events around the call on the launch stream."""
    import torch
    x, call = append_case()
    n_warm, t0 = 0, time.perf_counter()
    while n_warm < 5 or time.perf_counter() - t0 < 0.05:  # past the start-up transient
        flush()
        call()
        torch.cuda.synchronize()
        n_warm += 1
    evs = []
    for _ in range(iters):
        flush()
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        e0.record()
        call()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    med = float(np.median(us))
    nbytes = append_bytes(x)
    gbs = nbytes / (med * 1e-6) / 1e9
    return {
        "workload": x.workload,
        "config": {"instances": x.n_inst, "new_rows_per_instance": x.n_new,
                   "pool_cells_per_instance": x.pool_cells, "pos0": int(x.pos0[0]),
                   "rows": "float32 K and V rows, N(0, 1) x 2^U(-8, 8) per row",
                   "pool_layout": "int8 code rows; binary16 (K, V) scale pairs interleaved per cell"},
        "us_per_call_median": round(med, 3),
        "us_per_call_p10": round(float(np.percentile(us, 10)), 3),
        "us_per_call_p90": round(float(np.percentile(us, 90)), 3),
        "rows_per_s": round(x.n_inst * x.n_new / (med * 1e-6), 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("append"),
                     "kernel": "kv_append_kernel", "algorithmic_bytes_per_launch": nbytes,
                     "launch_us_median": round(med, 3)},
        "timing": f"{iters} eager calls after {n_warm} untimed ones, caches evicted before "
                  "each by reading a 1 GiB buffer",
    }


def qsa_bytes(x):
    """Algorithmic bytes of the scorer (the pooled keys of every block some
    row can use, the queries, dead flags and extents read, the scores
    written) and of the selection (the scores read, the cell list and counts
    written), for inputs x and the cell counts n_sel."""
    R = x.block_cells
    first = np.arange(x.max_blocks)[None, :] * R
    usable = (x.dead == 0) & (first < x.n_visible.max(axis=1)[:, None])
    hd = x.pooled.shape[2] * x.pooled.shape[3]
    n_scores = x.n_inst * x.n_rows * x.max_blocks
    scorer = (int(usable.sum()) * hd * 4 + x.q_idx.size * 4 + x.dead.size + x.n_visible.size * 4
              + n_scores * 4)
    return scorer, usable


def qsa_case():
    import torch
    from decode_attention_sparse_amd import api, inputs
    x = inputs.make_qsa("qsa_select_64inst_128k_2q")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    pooled, dead, q, vis = t(x.pooled), t(x.dead), t(x.q_idx), t(x.n_visible)
    scores = torch.empty((x.n_inst, x.n_rows, x.max_blocks), device="cuda")
    sel = torch.empty((x.n_inst, x.k_blocks * x.block_cells), dtype=torch.int32, device="cuda")
    n_sel = torch.empty((x.n_inst,), dtype=torch.int32, device="cuda")

    def score():
        api.qsa_block_scores(pooled, dead, q, vis, x.block_cells, scores)

    def select():
        api.qsa_select(scores, vis, x.block_cells, x.k_blocks, sel, n_sel)
    return x, score, select, n_sel


def qsa_section(iters, flush):
    """The QSA selection workload: the scorer and the top-k selection, each
    timed as eager calls with the caches evicted before each (HIP events on
    the launch stream), and the two back to back as one selection."""
    import torch
    x, score, select, n_sel = qsa_case()
    for _ in range(5):
        flush()
        score()
        select()
    torch.cuda.synchronize()
    t = {"scores": [], "select": [], "both": []}
    for _ in range(iters):
        for name, fns in (("scores", (score,)), ("select", (select,)), ("both", (score, select))):
            flush()
            e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record()
            for f in fns:
                f()
            e1.record()
            t[name].append((e0, e1))
    torch.cuda.synchronize()
    us = {k: float(np.median([a.elapsed_time(b) for a, b in v])) * 1e3 for k, v in t.items()}
    cells = int(n_sel.cpu().numpy().sum())
    scorer_bytes, usable = qsa_bytes(x)
    select_bytes = x.n_inst * x.n_rows * x.max_blocks * 4 + cells * 4 + x.n_inst * 4
    gbs = scorer_bytes / (us["scores"] * 1e-6) / 1e9
    return {
        "workload": x.workload,
        "config": {"instances": x.n_inst, "query_rows": x.n_rows, "indexer_heads":
                   int(x.pooled.shape[2]), "idx_dim": int(x.pooled.shape[3]),
                   "block_cells": x.block_cells, "blocks_per_instance": x.max_blocks,
                   "k_blocks": x.k_blocks, "visible_cells": [int(v) for v in x.n_visible[0]],
                   "dead_blocks": int(x.dead.sum())},
        "us_scores_median": round(us["scores"], 3),
        "us_select_median": round(us["select"], 3),
        "us_selection_median": round(us["both"], 3),
        "selected_cells": cells,
        "blocks_scored_per_s": round(x.n_inst * x.max_blocks / (us["both"] * 1e-6), 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("qsa"),
                     "kernel": "qsa_scores_kernel",
                     "algorithmic_bytes_per_launch": scorer_bytes,
                     "launch_us_median": round(us["scores"], 3),
                     "note": f"pooled keys of the {int(usable.sum())} blocks some row can use, "
                             "queries, flags and extents read, scores written"},
        "select_GBps_algorithmic": round(select_bytes / (us["select"] * 1e-6) / 1e9, 1),
        "timing": f"{iters} eager calls of each after 5 untimed ones, caches evicted before "
                  "each by reading a 1 GiB buffer, HIP events around the call",
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batched-iters", type=int, default=20)
    ap.add_argument("--no-batched", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--only-batched", action="store_true",
                    help="skip the headline workload (for profiling the batched kernels)")
    ap.add_argument("--configs", default="2,3,4", help="batched workloads to run")
    ap.add_argument("--chunk2", type=int, default=None,
                    help="chunk size for the 256-instance batched workload")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the measured HBM read ceilings (probes/gather_ceiling)")
    ap.add_argument("--no-prompt", action="store_true",
                    help="skip the prompt attention workload")
    ap.add_argument("--only-prompt", action="store_true",
                    help="only three eager prompt attention calls (for profiling)")
    ap.add_argument("--no-append", action="store_true", help="skip the KV append workload")
    ap.add_argument("--only-append", action="store_true",
                    help="only three eager KV append calls (for profiling)")
    ap.add_argument("--no-qsa", action="store_true", help="skip the QSA selection workload")
    ap.add_argument("--only-qsa", action="store_true",
                    help="only three eager QSA scorer + selection calls (for profiling)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size "
                         "reference dispatch for HBM byte counters)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print("bench.py measures one GPU: the path shards across GPUs without communication "
              "(instances are independent); run with --gpus 1", file=sys.stderr)
        return 2
    # measured read ceilings for the access shapes of the chunk pass; run as a
    # child process before this process touches the GPU
    ceiling = (None if (a.no_ceiling or a.only_batched or a.only_prompt or a.only_append
                        or a.only_qsa) else gather_ceiling())
    import torch
    from decode_attention_sparse_amd import api, inputs
    api.library()
    torch.cuda.init()
    dev_name = torch.cuda.get_device_name(0)
    if a.copy_probe_mib > 0:
        src = torch.ones(a.copy_probe_mib << 18, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if a.only_append:
        x, call = append_case()
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        print(json.dumps({"workload": x.workload, "calls": 3}), flush=True)
        return 0

    if a.only_qsa:
        x, score, select, _ = qsa_case()
        for _ in range(3):
            score()
            select()
        torch.cuda.synchronize()
        print(json.dumps({"workload": x.workload, "calls": 3}), flush=True)
        return 0

    if a.only_prompt:
        x, call = prompt_case()
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        print(json.dumps({"workload": x.workload, "calls": 3}), flush=True)
        return 0

    if a.only_batched:
        flush = make_flush()
        for cfg in [int(v) for v in a.configs.split(",") if v]:
            kw = {"chunk": a.chunk2} if (cfg == 2 and a.chunk2) else {}
            x = inputs.make(cfg, **kw)
            c = Case(x, x.chunk)
            time_calls([c], 3)
            d = summarize(c, time_calls([c], a.batched_iters, flush=flush)[0],
                          time_passes([c], a.batched_iters, flush=flush)[0])
            print(json.dumps({"workload": x.workload, "chunk": x.chunk, **d}), flush=True)
            del c, x
            torch.cuda.empty_cache()
        return 0

    # ---- headline workload: 2,051 cells, n_q = 1..4
    base = inputs.make(1)
    xs = [base.with_n_q(nq) for nq in (1, 2, 3, 4)]
    cases = [Case(x, base.chunk) for x in xs]
    time_calls(cases, a.warmup)  # W untimed eager steps

    def step():
        for c in cases:
            c.call()

    # the timed region: exactly K steps, captured into one graph and replayed
    g_steps = graph_of(step, a.steps)
    g_steps.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g_steps.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e0.elapsed_time(e1) / a.steps
    del g_steps
    # per-call means, each call alone in a graph of K launches, and the two
    # kernels of a call (sda_chunk_batch, sda_merge_batch at the chunk size
    # the call uses) timed the same way on their own: the chunk kernel's mean
    # launch duration feeds the roofline.  The two passes at the caller's
    # chunk size (256) are timed too, for reference.
    per_q = {}
    call_us_sum, bytes_sum = 0.0, 0
    for nq, c in zip((1, 2, 3, 4), cases):
        g_b = graph_of(c.call, a.steps)
        call_ms = time_graph(g_b, a.steps)
        del g_b
        g_c = graph_of(c.chunk_pass, a.steps)
        ch_ms = time_graph(g_c, a.steps)
        del g_c
        g_m = graph_of(c.merge_pass, a.steps)
        mg_ms = time_graph(g_m, a.steps)
        del g_m
        g_2 = graph_of(lambda: (c.chunk_pass(c.chunk), c.merge_pass(c.chunk)), a.steps)
        two_ms = time_graph(g_2, a.steps)
        del g_2
        per_q[f"q{nq}"] = {
            "us_per_call": round(call_ms * 1e3, 3), "call_chunk_cells": c.fused_chunk,
            "chunk_us": round(ch_ms * 1e3, 3), "merge_us": round(mg_ms * 1e3, 3),
            f"two_passes_at_chunk_{c.chunk}_us": round(two_ms * 1e3, 3),
            "cells_per_s": round(c.cells / (call_ms * 1e-3), 1),
            "GBps_algorithmic": round(c.bytes / (call_ms * 1e-3) / 1e9, 1),
            "pages_2080ti_v3_us": PAGES_V3_US[nq], "pages_2080ti_default_us": PAGES_DEFAULT_US[nq],
        }
        call_us_sum += call_ms * 1e3
        bytes_sum += c.bytes
    # the pages' 600-cell rows: config 0's pool and list (600 cells) with
    # 1-4 query positions, each call alone in a graph of K launches
    x600 = inputs.make(0, n_q=4)
    per_q600 = {}
    for nq in (1, 2, 3, 4):
        c6 = Case(x600.with_n_q(nq), x600.chunk)
        g6 = graph_of(c6.call, a.steps)
        us6 = time_graph(g6, a.steps) * 1e3
        del g6, c6
        per_q600[f"q{nq}"] = {"us_per_call": round(us6, 3),
                              "cells_per_s": round(600 / (us6 * 1e-6), 1),
                              "pages_2080ti_v3_us": PAGES_600_V3_US[nq],
                              "pages_2080ti_default_us": PAGES_600_DEFAULT_US[nq]}
    cells_step = sum(c.cells for c in cases)
    value = cells_step / (step_ms * 1e-3)
    pages_step_us = sum(PAGES_V3_US.values())
    # roofline of the dominant kernel: the chunk kernel of the n_q = 4 call
    c4, k4_us = cases[3], per_q["q4"]["chunk_us"]
    achieved = c4.chunk_bytes / (k4_us * 1e-6) / 1e9
    flush = make_flush()
    cold = time_calls(cases, 200, flush=flush)  # 200 calls per query count, as the pages' loop
    cold_us = {f"q{nq}": round(float(np.median(s_)) * 1e3, 3) for nq, s_ in zip((1, 2, 3, 4), cold)}
    cold_spread = {f"q{nq}": {"p10": round(float(np.percentile(s_, 10)) * 1e3, 3),
                              "p90": round(float(np.percentile(s_, 90)) * 1e3, 3)}
                   for nq, s_ in zip((1, 2, 3, 4), cold)}
    del cases
    torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "selected cells/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / (cells_step / (pages_step_us * 1e-6)), 3),
        "dtype": "i8 K/V codes, i8 MFMA with digit-split fp32 operands, fp32 softmax",
        "data": "synthetic (seeded PCG64; int8 codes uniform [-127,127], fp16 scales U[0.002,0.02], q N(0,1))",
        "config": {"workload": base.workload, "instances": 1, "n_qheads": 12, "head_dim": 256,
                   "queries": [1, 2, 3, 4], "selected_cells": 2051, "pool_cells": 32768,
                   "chunk": base.chunk, "calls_per_step": 4, "device": dev_name,
                   "pool_layout": "int8 K and V code rows [cells][256]; binary16 (K, V) scale pairs interleaved per cell",
                   "timing": "K steps captured in one HIP graph, HIP events around its replay; back-to-back calls with warm caches, as the pages' 200-call loop"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                     "traffic": measured_traffic("chunk"),
                     "kernel": f"{'chunk_tile_kernel' if c4.fused_chunk == 64 else 'chunk_mfma_kernel'}"
                               f", the n_q = 4 call of the step "
                               f"({c4.fused_chunk}-cell chunks: "
                               f"{-(-c4.max_sel // c4.fused_chunk)} chunks, one workgroup per "
                               f"chunk and 16-row group)",
                     "algorithmic_bytes_per_launch": c4.chunk_bytes,
                     "launch_us_mean": k4_us,
                     "note": "latency-bound: one instance, 2,051 cells; "
                             "traffic = HBM bytes per launch (cold, counters), null if the "
                             "kernel changed since they were taken: 1.88 MB fetched (the "
                             "1.05 MB of code rows once, the query rows and the page-table row "
                             "once per XCD that holds a workgroup of the instance, the scales' "
                             "sectors) and 1.63 MB of chunk partials written (33 chunks x 48 "
                             "rows x 1 KB), which the merge reads back; the launch's duration "
                             "is set by its round trips, not by these bytes",
                     "bytes_per_step": bytes_sum, "call_us_per_step": round(call_us_sum, 3)},
        "per_query_count": per_q,
        "pages_600_cells_per_query_count": per_q600,
        "value_cold": round(cells_step / (sum(cold_us.values()) * 1e-6), 1),
        "ms_per_step_cold": round(sum(cold_us.values()) * 1e-3, 6),
        "cold_us_per_call_median": cold_us,
        "cold_us_per_call_p10_p90": cold_spread,
        "cold_note": "200 eager calls per query count, caches evicted before each by reading a "
                     "1 GiB buffer, HIP events around each call; value_cold = the step's cells "
                     "over the sum of the four cold medians (value: K back-to-back steps, warm, "
                     "as the pages' 200-call loop)",
        "hbm_read_ceiling_measured": ceiling,
        "vs_baseline_ref": "pages' v3 kernel on RTX 2080 Ti, sum over q=1..4 of chunk+merge us (context, other hardware)",
        "wall_s_timed_region": round(wall, 3),
    }

    # ---- batched workloads (HBM-scale), cold caches between calls
    if not a.no_batched:
        batched = {}
        for cfg in [int(v) for v in a.configs.split(",") if v]:
            kw = {}
            if cfg == 2 and a.chunk2:
                kw["chunk"] = a.chunk2
            x = inputs.make(cfg, **kw)
            c = Case(x, x.chunk)
            n_warm = warm_up([c], flush)
            d = summarize(c, time_calls([c], a.batched_iters, flush=flush)[0],
                          time_passes([c], a.batched_iters, flush=flush)[0])
            st = time_passes_at([c], a.batched_iters, x.chunk, flush=flush)[0]
            d[f"two_passes_at_stated_chunk_{x.chunk}_us"] = {
                "chunk_us_median": round(float(np.median([u[0] for u in st])) * 1e3, 3),
                "merge_us_median": round(float(np.median([u[1] for u in st])) * 1e3, 3),
                "sum_us_median": round(float(np.median([u[0] + u[1] for u in st])) * 1e3, 3)}
            nch = -(-int(x.sel.shape[1]) // c.fused_chunk)
            d.update({"instances": x.n_inst, "n_q": x.n_q, "selected_cells_per_instance":
                      int(x.sel.shape[1]), "chunk": x.chunk, "call_chunk_cells": c.fused_chunk,
                      "call_launches": ("one chunk_mfma_kernel launch: " +
                                        ("two gather pipelines per workgroup, " if nch == 2 else "")
                                        + "outputs merged and written in place")
                                       if c.single_launch else "chunk_mfma_kernel, then merge kernel",
                      "two_pass_note": "chunk_us_mean / merge_us_mean: sda_chunk_batch and "
                                       "sda_merge_batch at the call's chunk size, timed as "
                                       "separate calls",
                      "warmup_calls": n_warm,
                      "timing": f"{a.batched_iters} eager calls after {n_warm} untimed ones, "
                                "caches evicted before each by reading a 1 GiB buffer, HIP "
                                "events around the call on the launch stream; median",
                      "bytes_algorithmic": c.bytes, "partials_bytes_written":
                      0 if c.single_launch else int(x.n_inst * nch * x.n_q * 12 * 258 * 4)})
            batched[x.workload] = d
            print(f"# {x.workload}: {d['us_per_call_median']} us/call, "
                  f"{d['GBps_algorithmic']} GB/s ({d['frac_hbm_peak']*100:.1f}% of HBM peak)",
                  file=sys.stderr, flush=True)
            del c, x
            torch.cuda.empty_cache()
        result["batched"] = batched

    # ---- prompt attention over the same pools (the next workload on the pages)
    if not a.no_prompt:
        d = prompt_section(20, 0.0 if a.no_cpu else a.cpu_seconds / 2)
        result["prompt_attention"] = d
        print(f"# {d['workload']}: {d['ms_per_call']} ms/call, {d['roofline']['achieved']} "
              f"TFLOP/s ({d['roofline']['frac']*100:.1f}% of the int8 matrix peak)",
              file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    # ---- INT8 KV append into the same pool layout
    if not a.no_append:
        d = append_section(a.batched_iters, flush)
        result["kv_append"] = d
        print(f"# {d['workload']}: {d['us_per_call_median']} us/call, {d['roofline']['achieved']} "
              f"GB/s ({d['roofline']['frac']*100:.1f}% of HBM peak)", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    # ---- QSA block scoring and top-k selection (the step before the path)
    if not a.no_qsa:
        d = qsa_section(a.batched_iters, flush)
        result["qsa_selection"] = d
        print(f"# {d['workload']}: scores {d['us_scores_median']} us ({d['roofline']['achieved']} "
              f"GB/s, {d['roofline']['frac']*100:.1f}% of HBM peak), select "
              f"{d['us_select_median']} us", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()

    if not a.no_cpu:
        result["cpu_baseline"] = cpu_baseline(xs, a.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

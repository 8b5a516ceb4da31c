#!/usr/bin/env python3
"""Decode-step benchmark of the quantized paged KV cache on one MI355X.

One step = the decode hot path of one full-attention layer: the T new rows of
every sequence are quantized into the pool, then paged decode attention runs
over the whole context (paged_decode_step: the split kernel quantizes the new
rows it holds, then the log-sum-exp merge).  The same step as the two calls
kv_append_quant + paged_decode_attn is timed beside it.
The headline workload is the MTP3 verify step at 131,072 tokens (B=1, T=4,
Hq=24, Hkv=4, D=256, INT8 group-64 KV); the JSON line also carries the 32K
(T=1) and 262,144-token (T=1, INT8 and FP8-row) depths of the metric.

Inputs are seeded synthetic data (kvq_synth) already resident in HBM.  Steps
rotate over several copies of the page pool so the 256 MB Infinity Cache never
holds the pool a step reads: every timed byte comes from HBM.

Prints ONE JSON line.  --gpus N > 1 exits: the library runs on one GPU (multi-GPU sharding is a design only).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak, vendor figure
HEADLINE = "mtp128k"
DEPTHS = ["qwen32k", "mtp128k", "c8", "full256k_int8", "full256k_fp8", "mtp128k_rk8v4", "mtp128k_rk4v4", "mtp128k_bf16",
          "full256k_bf16", "full256k_rk8v4", "full256k_rk4v4"]
SETTLE_S = 0.2  # seconds of untimed back-to-back steps before the warmup steps
FLUSH_BYTES = 1.5 * 2 ** 30  # bytes read between two reads of one pool copy (> 256 MB MALL)
KERNEL_SOURCES = ("internal.h", "shape.h", "quant_row.h", "attn_kernels.h")  # what the split kernel is built from


def kernel_sources_sha256():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_attention_quantized_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """HBM bytes per split-kernel launch from the committed counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE passes, each scaled by what the same counter
    reads for a copy kernel of known size).  None when there is no summary or the
    kernel sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"attn_split_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith((" ", "#")):
                k, v = line.split("=", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        return int(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu():
    model = platform.processor()
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
    except OSError:
        pass
    return model, os.cpu_count()


class Run:
    """One workload: data on the device, n_copies pools, timed steps."""

    def __init__(self, K, S, H, torch, name, device):
        self.K, self.S, self.H, self.torch = K, S, H, torch
        self.name, self.dev = (name if isinstance(name, str) else name.name), device
        w = S.make(name)
        self.w = w
        s = w.shape
        cache = H.new_cache(K, w, device, poison=True)
        self.bt = H.fill_gpu(K, w, cache, device, chunk=65536)
        pool_bytes = cache.nbytes()
        self.n_copies = int(min(64, max(2, math.ceil(FLUSH_BYTES / max(1, w.kv_bytes())) + 1)))
        self.caches = [cache]
        for _ in range(self.n_copies - 1):
            c = K.Cache(s.fmt, w.num_blocks, s.Hkv, s.D, device=device)
            for a, b in zip(cache.tensors(), c.tensors()):
                b.copy_(a)
            self.caches.append(c)
        self.pool_bytes = pool_bytes
        self.q = H.src_tensor(w.q, s.src, device)
        self.k_new = H.src_tensor(w.new_rows("k"), s.src, device)
        self.v_new = H.src_tensor(w.new_rows("v"), s.src, device)
        self.start = torch.from_numpy(w.seq_lens - s.T).to(device)
        self.sl = torch.from_numpy(w.seq_lens).to(device)
        self.out = torch.empty(self.q.shape, dtype=torch.float32, device=device)
        if s.chunk and s.B == 1:
            # the last prefill chunk (s.chunk rows before the T decode rows), for the append measurement
            L = int(w.seq_lens[0])
            c0 = L - s.T - s.chunk
            self.chunk_k = H.src_tensor(w.rows("k", 0, c0, c0 + s.chunk), s.src, device)
            self.chunk_v = H.src_tensor(w.rows("v", 0, c0, c0 + s.chunk), s.src, device)
            self.chunk_start = torch.tensor([c0], dtype=torch.int32, device=device)
        self.ws = K.alloc_workspace(cache, s.B, s.T, s.Hq, w.max_seq_len, device=device)
        self.n_splits, self.tps = K.num_splits(s.B, s.T, s.Hq, s.Hkv, s.D, w.max_seq_len)
        torch.cuda.synchronize()

    def attn_args(self, i):
        w = self.w
        return (self.caches[i % self.n_copies], self.q, self.bt, self.sl, w.max_seq_len, w.softmax_scale, self.out,
                self.ws)

    def step(self, i):
        """One decode step on pool copy i, one call: append the T new rows and attend
        (split kernel with the rows quantized in, then the merge)."""
        c, q, bt, sl, L, scale, out, ws = self.attn_args(i)
        self.K.paged_decode_step(c, self.k_new, self.v_new, q, bt, sl, L, scale, out, ws)

    def step_two_calls(self, i):
        """The same step as kv_append_quant followed by paged_decode_attn (3 kernels)."""
        c = self.caches[i % self.n_copies]
        self.K.kv_append_quant(c, self.k_new, self.v_new, self.bt, self.start)
        self.K.paged_decode_attn(*self.attn_args(i))

    def _graph(self, fn, idx):
        g = self.torch.cuda.CUDAGraph()
        with self.torch.cuda.graph(g):
            for i in idx:
                fn(i)
        return g

    def build_graphs(self):
        """HIP graphs (torch.cuda.CUDAGraph): one step per pool copy, all copies' steps
        in order, the same for the two-call step, and the split kernel alone."""
        torch = self.torch
        for i in range(self.n_copies):  # eager warm-up of every copy before capture
            self.step(i)
            self.step_two_calls(i)
        torch.cuda.synchronize()
        allc = range(self.n_copies)
        self.g_one = [self._graph(self.step, [i]) for i in allc]
        self.g_all = self._graph(self.step, allc)
        self.g_all_two = self._graph(self.step_two_calls, allc)
        self.g_split = self._graph(lambda i: self.K.paged_decode_attn_split(*self.attn_args(i)), allc)
        self.g_attn = self._graph(lambda i: self.K.paged_decode_attn(*self.attn_args(i)), allc)
        # the first replay of a graph also uploads it to the device: do that for every graph
        # here, so no timed region pays it
        for g in self.g_one + [self.g_all, self.g_all_two, self.g_split, self.g_attn]:
            g.replay()
        torch.cuda.synchronize()

    def measure_eager(self, steps, warmup):
        """Plain stream launches, no graphs (for counter runs): every kernel is its own dispatch."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(warmup + i)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(self.n_copies):
            self.K.paged_decode_attn_split(*self.attn_args(i))
        e1.record()
        torch.cuda.synchronize()
        return wall_ms / steps, [e0.elapsed_time(e1) / self.n_copies], None

    def _events(self, g, reps, per):
        torch = self.torch
        out = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) / (reps * per))
        return sorted(out)

    def measure(self, steps, warmup, eager=False):
        torch = self.torch
        if eager:
            return self.measure_eager(steps, warmup)
        self.build_graphs()
        # the GPU reaches its steady clocks only after tens of ms of sustained load: run
        # back-to-back steps for SETTLE_S seconds, then the W warmup steps, untimed
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < SETTLE_S:
            self.g_all.replay()
            torch.cuda.synchronize()
        wfull, wrest = divmod(warmup, self.n_copies)
        for _ in range(wfull):
            self.g_all.replay()
        for i in range(wrest):
            self.g_one[i].replay()
        torch.cuda.synchronize()
        full, rest = divmod(steps, self.n_copies)
        # exactly `steps` steps, synchronized on both sides; GPU time from events on the
        # replay stream, host wall time beside it (the host launch cadence of Python graph
        # replays can trail the GPU)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(full):
            self.g_all.replay()
        for i in range(rest):
            self.g_one[i].replay()
        e1.record()
        torch.cuda.synchronize()
        self.wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        gpu_ms = e0.elapsed_time(e1)
        reps = max(1, steps // self.n_copies)
        # the split kernel alone: events on the replay stream around back-to-back launches
        split_ms = self._events(self.g_split, reps, self.n_copies)
        two_ms = self._events(self.g_all_two, reps, self.n_copies)
        # the whole paged_decode_attn call (split + merge), no append
        self.attn_ms = self._events(self.g_attn, reps, self.n_copies)
        # the distribution: each step timed alone (events around one replay of one step)
        self.step_pct_us = self.step_percentiles(steps)
        return gpu_ms / steps, split_ms, two_ms

    def step_percentiles(self, steps):
        """p10 / p50 / p90 of the steps of a back-to-back run: an event between every two
        consecutive one-step graph replays, all enqueued before one synchronization."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            self.g_one[i % self.n_copies].replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        t = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(steps))
        q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
        return {"p10": round(q(0.1), 2), "p50": round(q(0.5), 2), "p90": round(q(0.9), 2)}

    def _launcher(self, fn, eager):
        """Something with replay() that runs fn(i) once per pool copy: a HIP graph, or (eager)
        the plain launches, each its own dispatch (for counter collection)."""
        if not eager:
            return self._graph(fn, range(self.n_copies))

        class _Eager:
            def replay(_self):
                for i in range(self.n_copies):
                    fn(i)
        return _Eager()

    def measure_chunk_append(self, reps=20, eager=False):
        """kv_append_quant of the last prefill chunk (rewriting the same rows with the same
        values), events around a graph of one append per pool copy (or the plain launches).
        Returns (ms per call, bytes read + written by definition)."""
        if not hasattr(self, "chunk_k"):
            return None, None
        K, torch = self.K, self.torch

        def app(i):
            K.kv_append_quant(self.caches[i % self.n_copies], self.chunk_k, self.chunk_v, self.bt, self.chunk_start)

        for i in range(self.n_copies):
            app(i)
        torch.cuda.synchronize()
        g = self._launcher(app, eager)
        g.replay()
        torch.cuda.synchronize()
        ms = self._events(g, reps, self.n_copies)[1]
        s = self.w.shape
        rows = self.chunk_k.shape[1] * s.Hkv
        src = 2 * rows * s.D * self.chunk_k.element_size()
        dst = 2 * rows * (s.D + (2 * s.D // 64 if s.fmt == 0 else 4))
        return ms, src + dst

    def measure_prefill_chunk(self, reps=2, eager=False):
        """paged_prefill_attn of the last prefill chunk where it sits in the context: its
        rows (seeded queries, N(0,1) in the source dtype) see every earlier key and the
        chunk's own rows up to themselves.  Events around a graph of one call per pool copy
        (or the plain launches).
        Returns (ms per call, flops by definition: 4 * D per visible (row, key) pair)."""
        if not hasattr(self, "chunk_k"):
            return None, None
        K, torch, S = self.K, self.torch, self.S
        s = self.w.shape
        n = s.chunk
        Lc = int(self.chunk_start.item()) + n
        g = torch.Generator().manual_seed(S.seed_of(self.name) + 77)
        q = torch.randn((1, n, s.Hq, s.D), generator=g, dtype=torch.float32)
        q = q.to(self.dev).to(torch.bfloat16 if s.src == S.SRC_BF16 else torch.float32)
        sl = torch.tensor([Lc], dtype=torch.int32, device=self.dev)
        out = torch.empty(q.shape, dtype=torch.float32, device=self.dev)
        ws = K.alloc_prefill_workspace(self.caches[0], 1, n, s.Hq, Lc, device=self.dev)

        def pf(i):
            K.paged_prefill_attn(self.caches[i % self.n_copies], q, self.bt, sl, Lc, self.w.softmax_scale, out, ws)

        for i in range(self.n_copies):
            pf(i)
        torch.cuda.synchronize()
        gr = self._launcher(pf, eager)
        gr.replay()
        torch.cuda.synchronize()
        ms = self._events(gr, reps, self.n_copies)[1]
        pairs = n * (Lc - n) + n * (n + 1) // 2
        return ms, 4 * s.D * s.Hq * pairs

    def algorithmic_split_bytes(self):
        """Bytes the split kernel must move by definition: every visible key and value
        (codes + scales), the block-table entries and the queries."""
        s = self.w.shape
        pages = sum(math.ceil(int(L) / 64) for L in self.w.seq_lens)
        q_bytes = self.q.numel() * self.q.element_size()
        return self.w.kv_bytes() + pages * 4 + q_bytes


def cpu_baseline(S, H, name, rows_target_s=12.0):
    """The oracle as it stands (plain C, fp64) on the same workload, two ways:
    - one thread on a bounded sample of query rows (each row re-reads its KV head's whole
      context, as the oracle does for every row), scaled to the whole call;
    - every query row of the call over all host cores, one oracle call per row on a pool
      of threads (the oracle releases the interpreter while it runs), timed whole.
    Returns the all-cores figure with the one-thread figure beside it."""
    import concurrent.futures as cf

    import numpy as np
    import oracle as O

    w = S.make(name)
    s = w.shape
    pool = H.oracle_pool(O, w)
    total_rows = s.B * s.T * s.Hq

    def one(r):
        pool.paged_attn(w.q, s.src, s.T, s.Hq, w.block_table, w.seq_lens, w.softmax_scale,
                        rows=np.array([r], np.int32))

    t_sum, n1 = 0.0, 0
    for r in range(total_rows):  # one thread (also builds any lazily made tables first)
        t0 = time.perf_counter()
        one(r)
        t_sum += time.perf_counter() - t0
        n1 += 1
        if t_sum >= rows_target_s:
            break
    call_1 = t_sum / n1 * total_rows
    cores = min(os.cpu_count() or 1, total_rows)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(cores) as ex:
        list(ex.map(one, range(total_rows)))
    call_all = time.perf_counter() - t0
    kv = w.kv_bytes()
    return {"value": round(kv / call_all / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"all {total_rows} query rows of {name} (the whole call), fp64 oracle, one oracle call per "
                      f"row on {cores} threads: {call_all:.1f} s",
            "tok_per_s": round(s.B * s.T / call_all, 4),
            "single_thread": {"value": round(kv / call_1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{n1} of {total_rows} query rows ({t_sum / n1:.2f} s/row), scaled to the "
                                        f"whole call ({call_1:.1f} s)"}}


def hbm_probe(K, torch, dev, mib=2048, reps=20):
    """Measured streaming ceilings of this GPU on a 2 GiB buffer, each the median of `reps`
    timed runs (events): the library's streaming-read probe kernel (kvq_probe.h) at several
    grid sizes (the best is the read ceiling) and torch's copy (read + write bytes)."""
    n = mib * 2 ** 20
    a = torch.empty(n // 4, dtype=torch.float32, device=dev)
    b = torch.empty(n // 4, dtype=torch.float32, device=dev)
    a.fill_(1.0)
    sink = torch.empty(4096, dtype=torch.int32, device=dev)
    out = {}
    probes = [(f"read_wg{wg}", (lambda wg=wg: K.hbm_read_probe(a, wg, sink)), n) for wg in (256, 512, 1024, 2048)]
    for kind, fn, nbytes in probes + [("copy", lambda: b.copy_(a), 2 * n)]:
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e-3)
        t.sort()
        out[f"{kind}_gbs"] = round(nbytes / t[len(t) // 2] / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    out["read_gbs"] = max(v for k, v in out.items() if k.startswith("read_wg"))
    out["buffer_mib"] = mib
    out["kernels"] = ("kvq_hbm_read_probe (non-temporal 16-byte loads, 256-thread workgroups) at 256..2048 "
                      "workgroups; torch copy_ (read+write bytes); median of 20 each")
    return out


def depth_sweep(K, S, H, torch, dev, steps):
    """Split-kernel time against context depth (INT8 group-64, B=1, Hq=24, Hkv=4, D=256, 64
    chunks per KV head at every depth): T=1 and T=4 at 32K..256K, and the least-squares line
    us = fixed + per_page * pages per team (pages a 4-wave team streams = L / 64 / 64 / 2)."""
    res = {}
    for T in (1, 4):
        pts = []
        for L in (32768, 65536, 131072, 196608, 262144):
            shp = dataclasses.replace(S.shape("mtp128k"), T=T, lens=[L], name=f"sweep_t{T}_{L}")
            print(f"[bench] depth sweep T={T} L={L}", file=sys.stderr, flush=True)
            run = Run(K, S, H, torch, shp, dev)
            run.build_graphs()
            t0 = time.perf_counter()  # settle the clocks, as the main measurement does
            while time.perf_counter() - t0 < SETTLE_S:
                run.g_split.replay()
                torch.cuda.synchronize()
            ms = run._events(run.g_split, max(1, steps // run.n_copies), run.n_copies)[1]
            pts.append((L // 64 // 64 // 2, ms * 1e3))
            del run
            torch.cuda.empty_cache()
        n = len(pts)
        mx = sum(p for p, _ in pts) / n
        my = sum(u for _, u in pts) / n
        slope = sum((p - mx) * (u - my) for p, u in pts) / sum((p - mx) ** 2 for p, _ in pts)
        res[f"T={T}"] = {"split_us_by_context": {str(p * 8192): round(u, 2) for p, u in pts},
                         "per_page_us": round(slope, 3), "fixed_us": round(my - slope * mx, 2)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=["tiny", "qwen32k", "mtp128k", "mtp128k_rk8v4", "mtp128k_rk4v4", "mtp128k_bf16", "full256k_bf16",
                                                             "full256k_rk8v4", "full256k_rk4v4", "c8",
                                                             "full256k_int8",
                                                             "full256k_fp8"])
    ap.add_argument("--headline-only", action="store_true", help="skip the other depths")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch without HIP graphs (for counter collection)")
    ap.add_argument("--depth-sweep", action="store_true",
                    help="also time the split kernel against context depth (T=1 and T=4, 32K..256K)")
    ap.add_argument("--no-hbm-probe", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a known-size kernel for counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design only)", file=sys.stderr)
        sys.exit(2)

    import torch

    import kvq_synth as S
    import paged_attention_quantized_kv_amd as K
    from tests import gpu_harness as H

    dev = "cuda:0"
    if args.copy_probe_mib:
        n = args.copy_probe_mib * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    names = [args.workload] if args.headline_only else [args.workload] + [d for d in DEPTHS if d != args.workload]
    results = {}
    for name in names:
        print(f"[bench] {name}: generating and appending the context", file=sys.stderr, flush=True)
        run = Run(K, S, H, torch, name, dev)
        ms, split_ms, two_ms = run.measure(args.steps, args.warmup, eager=args.eager)
        w = run.w
        s = w.shape
        split_avg = sum(split_ms) / len(split_ms)
        chunk_ms, chunk_bytes = run.measure_chunk_append(eager=args.eager)
        pf_ms, pf_flops = run.measure_prefill_chunk(eager=args.eager)
        alg = run.algorithmic_split_bytes()
        results[name] = {
            "ms_per_step": ms,
            "kv_gbs": w.kv_bytes() / (ms * 1e-3) / 1e9,
            "tok_per_s": s.B * s.T / (ms * 1e-3),
            "split_ms_avg": split_avg,
            "split_ms_min": split_ms[0],
            "split_ms_max": split_ms[-1],
            "split_alg_bytes": alg,
            "split_gbs": alg / (split_avg * 1e-3) / 1e9,
            "kv_bytes": w.kv_bytes(),
            "n_copies": run.n_copies,
            "n_splits": run.n_splits,
            "tokens_per_split": run.tps,
            "two_call_ms": (sum(two_ms) / len(two_ms)) if two_ms else None,
            "attn_ms": (sum(run.attn_ms) / len(run.attn_ms)) if getattr(run, "attn_ms", None) else None,
            "step_pct_us": getattr(run, "step_pct_us", None),
            "wall_ms": getattr(run, "wall_ms", None),
            "chunk_ms": chunk_ms,
            "chunk_bytes": chunk_bytes,
            "prefill_ms": pf_ms,
            "prefill_flops": pf_flops,
        }
        print(f"[bench] {name}: {ms * 1e3:.1f} us/step, split {split_avg * 1e3:.1f} us "
              f"({results[name]['split_gbs']:.0f} GB/s), {run.n_copies} pool copies", file=sys.stderr, flush=True)
        del run
        torch.cuda.empty_cache()

    head = results[args.workload]
    shp = S.shape(args.workload)
    model, ncpu = host_cpu()
    line = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) and tok/s at 32K/128K/256K",
        "value": round(head["kv_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={shp.B} T={shp.T} Hq={shp.Hq} Hkv={shp.Hkv} D={shp.D} "
                               f"L={shp.lens[0] if shp.B == 1 else 'ragged'} page=64 "
                               f"{ {0: 'INT8 g64', 1: 'FP8 E4M3 row', 2: 'rk8v4', 3: 'rk4v4', 4: 'BF16'}[shp.fmt]} KV",
                   "global_batch": shp.B * shp.T, "seq_len": shp.lens[0] if shp.B == 1 else max(shp.lens),
                   "step": "paged_decode_step: append of the T new rows + paged decode attention (2 kernels)",
                   "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * head["kv_gbs"] / HBM_PEAK_GBS, 2),
        "tok_per_s": round(head["tok_per_s"], 1),
        "roofline": {"bound": "hbm", "achieved": round(head["split_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(head["split_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(args.workload),
                     "kernel": "attn_split_kernel", "launch_avg_us": round(head["split_ms_avg"] * 1e3, 2),
                     "alg_bytes_per_launch": head["split_alg_bytes"],
                     # the whole paged_decode_attn call (split + merge kernels, no append)
                     "attn_call_us": round(head["attn_ms"] * 1e3, 2) if head["attn_ms"] else None,
                     "attn_call_frac": round(head["split_alg_bytes"] / (head["attn_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                     if head["attn_ms"] else None},
        "depths": {n: {"kv_gbs": round(r["kv_gbs"], 1), "pct_hbm_peak": round(100 * r["kv_gbs"] / HBM_PEAK_GBS, 2),
                       "tok_per_s": round(r["tok_per_s"], 1), "us_per_step": round(r["ms_per_step"] * 1e3, 2),
                       "split_us": round(r["split_ms_avg"] * 1e3, 2), "split_gbs": round(r["split_gbs"], 1),
                       "us_per_step_two_calls": round(r["two_call_ms"] * 1e3, 2) if r["two_call_ms"] else None,
                       "us_per_step_pct": r["step_pct_us"],
                       "attn_call_us": round(r["attn_ms"] * 1e3, 2) if r["attn_ms"] else None,
                       "us_per_step_host_wall": round(r["wall_ms"] * 1e3, 2) if r["wall_ms"] else None,
                       "n_splits": r["n_splits"], "pool_copies": r["n_copies"],
                       **({"append_chunk_rows": 4096, "append_chunk_us": round(r["chunk_ms"] * 1e3, 2),
                           "append_chunk_gbs": round(r["chunk_bytes"] / (r["chunk_ms"] * 1e-3) / 1e9, 1)}
                          if r["chunk_ms"] else {}),
                       **({"prefill_chunk_us": round(r["prefill_ms"] * 1e3, 1),
                           "prefill_chunk_tflops": round(r["prefill_flops"] / (r["prefill_ms"] * 1e-3) / 1e12, 1),
                           "prefill_chunk_frac_f16_mfma": round(r["prefill_flops"] / (r["prefill_ms"] * 1e-3)
                                                                / (MFMA_F16_PEAK_TFLOPS * 1e12), 4)}
                          if r["prefill_ms"] else {})} for n, r in results.items()},
        "host": {"cpu": model, "nproc": ncpu},
        "step_us_pct": head["step_pct_us"],
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(S, H, args.workload)
    if not args.no_hbm_probe and not args.eager:
        print("[bench] HBM read/copy probe", file=sys.stderr, flush=True)
        line["hbm_probe"] = hbm_probe(K, torch, dev)
    if args.depth_sweep:
        line["depth_sweep"] = depth_sweep(K, S, H, torch, dev, args.steps)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Helpers shared by the GPU parity tests, smoke() and bench.py.

They move seeded workloads (kvq_synth) to the device, fill a page pool through
kv_append_quant, and build the oracle's pool from the same source rows.  No
value produced here on the GPU ever feeds the oracle.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import kvq_synth as S

POISON_CODE = 0x7F
POISON_F16 = 0x7E00  # fp16 NaN


def src_tensor(a: np.ndarray, src: int, device) -> torch.Tensor:
    """Source rows / queries (float32 array, or uint16 bf16 bits) -> device tensor."""
    if src == S.SRC_BF16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def new_cache(K, w: S.Workload, device, poison: bool = True):
    s = w.shape
    cache = K.Cache(s.fmt, w.num_blocks, s.Hkv, s.D, device=device)
    if poison and s.fmt == S.FMT_BF16:  # every element a bf16 NaN
        cache.k_codes.view(torch.int16).fill_(-1)
        cache.v_codes.view(torch.int16).fill_(-1)
    elif poison:
        cache.k_codes.fill_(POISON_CODE)
        cache.v_codes.fill_(POISON_CODE)
        if s.fmt in (S.FMT_INT8_G64, S.FMT_RK8V4, S.FMT_RK4V4):  # fp16 scales
            cache.k_scales.view(torch.int16).fill_(POISON_F16)
            cache.v_scales.view(torch.int16).fill_(POISON_F16)
        else:
            cache.k_scales.fill_(float("nan"))
            cache.v_scales.fill_(float("nan"))
    return cache


def fill_gpu(K, w: S.Workload, cache, device, chunk: int = 8192, decode_rows: bool = True):
    """Append every context row of every sequence: prefill chunks of `chunk` rows
    (the last prefill chunk is w.shape.chunk rows if set), then the T decode rows
    of all sequences in one batched call."""
    s = w.shape
    bt = torch.from_numpy(w.block_table).to(device)
    for b in range(s.B):
        L = int(w.seq_lens[b])
        stop = L - s.T if decode_rows else L
        edges = list(range(0, stop, chunk))
        if s.chunk and stop > s.chunk:
            edges = list(range(0, stop - s.chunk, chunk)) + [stop - s.chunk]
        edges.append(stop)
        for a0, a1 in zip(edges[:-1], edges[1:]):
            if a1 <= a0:
                continue
            k = src_tensor(w.rows("k", b, a0, a1), s.src, device)
            v = src_tensor(w.rows("v", b, a0, a1), s.src, device)
            sp = torch.tensor([a0], dtype=torch.int32, device=device)
            K.kv_append_quant(cache, k, v, bt[b:b + 1].contiguous(), sp)
    if decode_rows:
        k = src_tensor(w.new_rows("k"), s.src, device)
        v = src_tensor(w.new_rows("v"), s.src, device)
        sp = torch.from_numpy(w.seq_lens - s.T).to(device)
        K.kv_append_quant(cache, k, v, bt, sp)
    return bt


def oracle_pool(O, w: S.Workload):
    s = w.shape
    pool = O.Pool(s.fmt, w.num_blocks, s.Hkv, s.D, fill=0xFF if s.fmt == S.FMT_BF16 else POISON_CODE)
    if s.fmt == S.FMT_BF16:
        for b in range(s.B):
            L = int(w.seq_lens[b])
            pool.append(w.rows("k", b, 0, L), w.rows("v", b, 0, L), s.src, w.block_table[b:b + 1],
                        np.array([0], np.int32))
        return pool
    if s.fmt in (S.FMT_INT8_G64, S.FMT_RK8V4, S.FMT_RK4V4):
        pool.k_scales[:] = POISON_F16
        pool.v_scales[:] = POISON_F16
    else:
        pool.k_scales[:] = np.nan
        pool.v_scales[:] = np.nan
    for b in range(s.B):
        L = int(w.seq_lens[b])
        pool.append(w.rows("k", b, 0, L), w.rows("v", b, 0, L), s.src, w.block_table[b:b + 1],
                    np.array([0], np.int32))
    return pool


def oracle_attn(pool, w: S.Workload, rows=None, q=None, threads: int = 16) -> np.ndarray:
    """The oracle's attention rows (all, or the given output rows), computed on several host
    threads: rows are independent, and the C oracle releases the interpreter while it runs.
    The first row runs alone, since the oracle fills its lookup tables on first use."""
    s = w.shape
    q = w.q if q is None else q
    rows = np.arange(s.B * s.T * s.Hq, dtype=np.int32) if rows is None else np.asarray(rows, np.int32)

    def call(r):
        return pool.paged_attn(q, s.src, s.T, s.Hq, w.block_table, w.seq_lens, w.softmax_scale, rows=r)

    if rows.size <= 1:
        return call(rows)
    first = call(rows[:1])
    parts = np.array_split(rows[1:], min(threads, os.cpu_count() or 1, rows.size - 1))
    with ThreadPoolExecutor(len(parts)) as ex:
        return np.concatenate([first] + list(ex.map(call, parts)))


def pool_equal(cache, pool) -> dict:
    """Byte-exact comparison of the device pool with the oracle's pool; returns mismatch counts."""
    res = {}
    for name in ("k_codes", "v_codes", "k_scales", "v_scales"):
        if name.endswith("scales") and cache.format == S.FMT_BF16:  # the BF16 pool has no scales
            res[name] = 0
            continue
        g = getattr(cache, name).contiguous().view(torch.uint8).cpu().numpy()
        o = getattr(pool, name).view(np.uint8)
        res[name] = int(np.count_nonzero(g != o)) if g.size == o.size else -1
    return res


def run_attn(K, w: S.Workload, cache, bt, device, q=None, stream=None, prefill=False):
    """paged_decode_attn (or paged_prefill_attn) of the workload's queries."""
    s = w.shape
    q = src_tensor(w.q, s.src, device) if q is None else q
    sl = torch.from_numpy(w.seq_lens).to(device)
    out = torch.empty(q.shape, dtype=torch.float32, device=device)
    if prefill:
        ws = K.alloc_prefill_workspace(cache, s.B, s.T, s.Hq, w.max_seq_len, device=device)
        K.paged_prefill_attn(cache, q, bt, sl, w.max_seq_len, w.softmax_scale, out, ws, stream=stream)
    else:
        ws = K.alloc_workspace(cache, s.B, s.T, s.Hq, w.max_seq_len, device=device)
        K.paged_decode_attn(cache, q, bt, sl, w.max_seq_len, w.softmax_scale, out, ws, stream=stream)
    return out

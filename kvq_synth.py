"""Seeded synthetic inputs shared by the tests, smoke() and bench.py.

This module only draws random numbers and builds index tables.  It holds none
of the method's arithmetic (no quantization, no attention), so the oracle and
the HIP path can both consume what it produces without sharing code.

Workloads (one full-attention layer of a 27B-class hybrid model, page = 64
tokens; shapes after NInfer-4090 README "What this fork changes", d256-h24-kv4):

  tiny        B=1 T=1 Hq=8  Hkv=1 D=128 L=2048, fp32 K/V/Q ~ N(0,1)
  qwen32k     B=1 T=1 Hq=24 Hkv=4 D=256 L=32768, bf16 K/V ~ N(0,1) with 4 outlier
              channels per (KV head, K|V) scaled x20; Q bf16 ~ N(0,1)
  mtp128k     as qwen32k, T=4 (MTP3 verify: 3 drafted + 1), L=131072
  c8          B=8 T=4, L_b ~ U[4096, 65536] (seeded), pages of all sequences
              interleaved in one pool by a shuffled block table
  full256k    B=1 T=1 L=262144, INT8 (A) or row-scaled FP8 (B); the last
              4096 context rows form one prefill chunk
  mtp128k_rk8v4  mtp128k's data in the rk8v4 format (rotated INT8 keys,
              4-bit group-32 values)
  mtp128k_rk4v4  the same in the rk4v4 format (4-bit Lloyd-Max keys)
  mtp128k_bf16, full256k_bf16  the same data in the BF16 reference format
  full256k_rk8v4, full256k_rk4v4  full256k's data (T=1) in the rotated formats

Every pool starts filled with poison (code bytes 0x7F, NaN scales), so a read of
a slot that was never appended shows up as NaN in the output.  Block-table
entries past a sequence's last page point at a poison page.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

PAGE = 64
FMT_INT8_G64 = 0
FMT_FP8_ROW = 1
FMT_RK8V4 = 2
FMT_RK4V4 = 3
FMT_BF16 = 4
SRC_F32 = 0
SRC_BF16 = 1

CONFIG_NAMES = ["tiny", "qwen32k", "mtp128k", "c8", "full256k_int8", "full256k_fp8"]
_SEED_INDEX = {"tiny": 0, "qwen32k": 1, "mtp128k": 2, "c8": 3, "full256k_int8": 4, "full256k_fp8": 4,
               "mtp128k_rk8v4": 2, "mtp128k_rk4v4": 2, "mtp128k_bf16": 2, "full256k_bf16": 4,
               "full256k_rk8v4": 4, "full256k_rk4v4": 4}


@dataclasses.dataclass
class Shape:
    name: str
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    lens: list
    src: int
    fmt: int
    outliers: bool
    chunk: int = 0  # size of the last prefill chunk before the decode rows (0: none)


def shape(name: str, **over) -> Shape:
    if name == "tiny":
        s = Shape(name, 1, 1, 8, 1, 128, [2048], SRC_F32, FMT_INT8_G64, False)
    elif name == "qwen32k":
        s = Shape(name, 1, 1, 24, 4, 256, [32768], SRC_BF16, FMT_INT8_G64, True)
    elif name == "mtp128k":
        s = Shape(name, 1, 4, 24, 4, 256, [131072], SRC_BF16, FMT_INT8_G64, True)
    elif name == "c8":
        g = torch.Generator().manual_seed(seed_of(name) + 7)
        lens = torch.randint(4096, 65536 + 1, (8,), generator=g).tolist()
        s = Shape(name, 8, 4, 24, 4, 256, lens, SRC_BF16, FMT_INT8_G64, True)
    elif name == "full256k_int8":
        s = Shape(name, 1, 1, 24, 4, 256, [262144], SRC_BF16, FMT_INT8_G64, True, chunk=4096)
    elif name == "mtp128k_rk8v4":
        s = Shape(name, 1, 4, 24, 4, 256, [131072], SRC_BF16, FMT_RK8V4, True)
    elif name == "mtp128k_bf16":
        s = Shape(name, 1, 4, 24, 4, 256, [131072], SRC_BF16, FMT_BF16, True)
    elif name == "full256k_bf16":
        s = Shape(name, 1, 1, 24, 4, 256, [262144], SRC_BF16, FMT_BF16, True)
    elif name == "full256k_rk8v4":
        s = Shape(name, 1, 1, 24, 4, 256, [262144], SRC_BF16, FMT_RK8V4, True)
    elif name == "full256k_rk4v4":
        s = Shape(name, 1, 1, 24, 4, 256, [262144], SRC_BF16, FMT_RK4V4, True)
    elif name == "mtp128k_rk4v4":
        s = Shape(name, 1, 4, 24, 4, 256, [131072], SRC_BF16, FMT_RK4V4, True)
    elif name == "full256k_fp8":
        s = Shape(name, 1, 1, 24, 4, 256, [262144], SRC_BF16, FMT_FP8_ROW, True, chunk=4096)
    else:
        raise KeyError(name)
    return dataclasses.replace(s, **over)


def seed_of(name: str) -> int:
    return 0x5EED0000 + _SEED_INDEX.get(name.split("@")[0], 9)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bfloat16 bit patterns of a bf16 tensor as uint16."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class Workload:
    shape: Shape
    k_src: list  # per sequence: [L_b, Hkv, D]  float32 ndarray, or uint16 bf16 bits
    v_src: list
    q: np.ndarray  # [B, T, Hq, D] float32 or uint16 bf16 bits
    block_table: np.ndarray  # [B, max_blocks] int32
    seq_lens: np.ndarray  # [B] int32
    num_blocks: int
    poison_block: int
    softmax_scale: float

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max())

    def rows(self, which: str, b: int, start: int, stop: int) -> np.ndarray:
        """Source rows [start, stop) of sequence b as [1, n, Hkv, D] (the append input)."""
        src = self.k_src if which == "k" else self.v_src
        return np.ascontiguousarray(src[b][start:stop][None])

    def new_rows(self, which: str) -> np.ndarray:
        """The T decode rows of every sequence as [B, T, Hkv, D]."""
        s = self.shape
        src = self.k_src if which == "k" else self.v_src
        return np.ascontiguousarray(np.stack([src[b][int(self.seq_lens[b]) - s.T:int(self.seq_lens[b])]
                                              for b in range(s.B)]))

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode call reads: every visible key and value, codes + scales."""
        s = self.shape
        if s.fmt == FMT_RK8V4:  # INT8 keys with fp16 group-64 scales, 4-bit values with fp16 group-32 scales
            per_tok_head = (s.D + 2 * (s.D // 64)) + (s.D // 2 + 2 * (s.D // 32))
        elif s.fmt == FMT_BF16:  # two bytes per element, no scales
            per_tok_head = 2 * 2 * s.D
        elif s.fmt == FMT_RK4V4:  # 4-bit keys with fp16 group-64 scales, rk8v4 values
            per_tok_head = (s.D // 2 + 2 * (s.D // 64)) + (s.D // 2 + 2 * (s.D // 32))
        else:
            per_tok_head = 2 * (s.D + (2 * (s.D // 64) if s.fmt == FMT_INT8_G64 else 4))
        return int(self.seq_lens.sum()) * s.Hkv * per_tok_head


def _source(gen: torch.Generator, L: int, Hkv: int, D: int, src: int, outliers: bool,
            out_ch: np.ndarray) -> np.ndarray:
    x = torch.randn((L, Hkv, D), generator=gen, dtype=torch.float32)
    if outliers:
        for h in range(Hkv):
            x[:, h, torch.from_numpy(out_ch[h])] *= 20.0
    if src == SRC_BF16:
        return bf16_bits(x.to(torch.bfloat16))
    return x.numpy()


def make(name_or_shape, seed: int | None = None, extra_blocks: int = 4) -> Workload:
    s = shape(name_or_shape) if isinstance(name_or_shape, str) else name_or_shape
    seed = seed_of(s.name) if seed is None else seed
    gen = torch.Generator().manual_seed(seed)
    # outlier channels: per (K|V, KV head), 4 distinct channels from a seeded permutation
    k_ch = np.stack([torch.randperm(s.D, generator=gen)[:4].numpy() for _ in range(s.Hkv)])
    v_ch = np.stack([torch.randperm(s.D, generator=gen)[:4].numpy() for _ in range(s.Hkv)])
    k_src, v_src = [], []
    for b in range(s.B):
        k_src.append(_source(gen, s.lens[b], s.Hkv, s.D, s.src, s.outliers, k_ch))
        v_src.append(_source(gen, s.lens[b], s.Hkv, s.D, s.src, s.outliers, v_ch))
    q = torch.randn((s.B, s.T, s.Hq, s.D), generator=gen, dtype=torch.float32)
    q = bf16_bits(q.to(torch.bfloat16)) if s.src == SRC_BF16 else q.numpy()
    return _with_tables(s, gen, k_src, v_src, q, extra_blocks)


def make_sink(s: Shape, gap_nats: float = 13.0, stride: int = 4096, seed: int = 0, v_mean: float = 1.0,
              v_sd: float = 0.2, k_sd: float = 0.05, extra_blocks: int = 4) -> Workload:
    """Inputs whose softmax has attention sinks: a few dominant keys over many near-uniform ones.

    Every query row of KV head h is the same seeded +-1 pattern u_h.  Keys are
    N(0, k_sd^2) except one key every `stride` positions (positions 0, stride, ...),
    which is u_h * gap_nats / sqrt(D): with the softmax scale 1/sqrt(D) its logit lies
    gap_nats above the others, whose logits are ~N(0, k_sd^2).  Values are
    v_mean + v_sd * N(0, 1): a nonzero mean and small group scales, so the many tiny
    weights of the near-uniform keys carry a visible share of the output.  s.outliers
    is ignored.
    """
    gen = torch.Generator().manual_seed(0x51C0 + seed)
    u = torch.randint(0, 2, (s.Hkv, s.D), generator=gen).to(torch.float32) * 2.0 - 1.0
    a = gap_nats / math.sqrt(s.D)
    k_src, v_src = [], []
    for b in range(s.B):
        L = s.lens[b]
        k = torch.randn((L, s.Hkv, s.D), generator=gen, dtype=torch.float32) * k_sd
        k[0:L:stride] = u * a
        v = v_mean + v_sd * torch.randn((L, s.Hkv, s.D), generator=gen, dtype=torch.float32)
        if s.src == SRC_BF16:
            k_src.append(bf16_bits(k.to(torch.bfloat16)))
            v_src.append(bf16_bits(v.to(torch.bfloat16)))
        else:
            k_src.append(k.numpy())
            v_src.append(v.numpy())
    G = s.Hq // s.Hkv
    q = u.repeat_interleave(G, dim=0)[None, None].expand(s.B, s.T, s.Hq, s.D).contiguous()
    q = bf16_bits(q.to(torch.bfloat16)) if s.src == SRC_BF16 else q.numpy()
    return _with_tables(s, gen, k_src, v_src, q, extra_blocks)


def make_wide(s: Shape, span_log2: float = 8.0, seed: int = 0, small_run: int | None = None,
              extra_blocks: int = 4) -> Workload:
    """Inputs whose rows span a wide range of magnitudes.

    Keys and queries ~ N(0, 1); each value row (token, KV head) is N(0, 1) times
    2^u with u ~ U(-span_log2, span_log2) drawn per row, so the V scales of one
    page differ by up to 2^(2 span_log2) and the largest of them falls on any slot.
    With small_run = r (0..3), u is instead -span_log2 for the positions j with
    (j % 16) // 4 == r and +span_log2 elsewhere: every 16-slot run of a page has
    the same four small rows.  s.outliers is ignored.
    """
    gen = torch.Generator().manual_seed(0x3D0E + seed)
    k_src, v_src = [], []
    for b in range(s.B):
        L = s.lens[b]
        k = torch.randn((L, s.Hkv, s.D), generator=gen, dtype=torch.float32)
        u = (torch.rand((L, s.Hkv, 1), generator=gen, dtype=torch.float32) * 2.0 - 1.0) * span_log2
        if small_run is not None:
            small = ((torch.arange(L) % 16) // 4 == small_run).to(torch.float32)[:, None, None]
            u = span_log2 * (1.0 - 2.0 * small) + 0.0 * u
        v = torch.randn((L, s.Hkv, s.D), generator=gen, dtype=torch.float32) * torch.exp2(u)
        if s.src == SRC_BF16:
            k_src.append(bf16_bits(k.to(torch.bfloat16)))
            v_src.append(bf16_bits(v.to(torch.bfloat16)))
        else:
            k_src.append(k.numpy())
            v_src.append(v.numpy())
    q = torch.randn((s.B, s.T, s.Hq, s.D), generator=gen, dtype=torch.float32)
    q = bf16_bits(q.to(torch.bfloat16)) if s.src == SRC_BF16 else q.numpy()
    return _with_tables(s, gen, k_src, v_src, q, extra_blocks)


def _with_tables(s: Shape, gen: torch.Generator, k_src, v_src, q, extra_blocks: int) -> Workload:
    # shared pool: every (sequence, page) pair gets a shuffled physical block id
    pages = [math.ceil(L / PAGE) for L in s.lens]
    total = sum(pages)
    num_blocks = total + extra_blocks
    perm = torch.randperm(num_blocks, generator=gen).numpy().astype(np.int32)
    poison_block = int(perm[total])  # first spare block: target of unused table entries
    max_blocks = max(pages)
    bt = np.full((s.B, max_blocks), poison_block, np.int32)
    k = 0
    for b in range(s.B):
        for p in range(pages[b]):
            bt[b, p] = perm[k]
            k += 1
    return Workload(s, k_src, v_src, q, bt, np.asarray(s.lens, np.int32), num_blocks, poison_block,
                    float(np.float32(1.0 / math.sqrt(s.D))))


def tiny_shape(B=1, T=1, Hq=8, Hkv=1, D=128, lens=(200,), src=SRC_F32, fmt=FMT_INT8_G64,
               outliers=False, name="custom") -> Shape:
    """A small custom shape for parity and edge-case tests."""
    return Shape(name, B, T, Hq, Hkv, D, list(lens), src, fmt, outliers)

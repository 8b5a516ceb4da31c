"""Pins of the oracle's BF16 KV format, the unquantized reference (CPU only).

BF16 (NInfer-3090 README, "Choosing a KV format": 65,536 B/token on the 27B): each K
and V element is stored as bfloat16, rounded to nearest even, with no scales.  The
rounding is pinned against torch at every rounding edge; the size against the pages'
table; the cache against the source rows (a bf16 source is stored exactly, so attention
over the cache is attention over the source).
"""
import os

import numpy as np
import torch

import kvq_synth as S
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def test_bf16_rounding_matches_torch_at_every_rounding_edge():
    h = np.arange(0, 0x7F80, dtype=np.uint32)  # every finite non-negative bf16
    v = (h << 16).view(np.float32)
    nxt = ((h + 1) << 16).view(np.float32)
    mid = ((h << 16) + 0x8000).view(np.float32)  # exactly halfway (exact in binary32)
    probes = np.concatenate([v, mid, mid.view(np.uint32).__sub__(1).view(np.float32),
                             mid.view(np.uint32).__add__(1).view(np.float32), nxt])
    x = np.concatenate([probes, -probes])
    assert np.array_equal(O.f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_bf16_special_values():
    x = np.array([np.inf, -np.inf, 0.0, -0.0, 3.4e38, -3.4e38, 1e-45], np.float32)
    assert np.array_equal(O.f32_to_bf16_bits(x), _torch_bf16_bits(x))
    n = O.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (n & 0x7F80) == 0x7F80 and (n & 0x7F) != 0


def test_bf16_bytes_per_token_match_the_pages_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "kv_format_table.txt")):
        f = line.split("#")[0].split()
        if f:
            rows[f[0]] = [float(v) for v in f[1:]]
    layers, heads, D = int(rows["layers"][0]), int(rows["kv_heads"][0]), int(rows["head_dim"][0])
    p = O.Pool(O.FMT_BF16, num_blocks=3, num_kv_heads=heads, head_dim=D)
    per_tok_layer = (p.k_codes.nbytes + p.v_codes.nbytes) / (3 * 64)
    assert per_tok_layer * layers == rows["bf16"][0]


def _pool(w):
    s = w.shape
    pool = O.Pool(s.fmt, w.num_blocks, s.Hkv, s.D, fill=0xFF)  # 0xFFFF: a bf16 NaN
    for b in range(s.B):
        L = int(w.seq_lens[b])
        pool.append(w.rows("k", b, 0, L), w.rows("v", b, 0, L), s.src, w.block_table[b:b + 1],
                    np.array([0], np.int32))
    return pool


def test_append_stores_bf16_of_the_source_in_the_int8_element_order():
    w = S.make(S.tiny_shape(B=2, T=1, Hq=4, Hkv=2, D=128, lens=(150, 70), src=S.SRC_F32, fmt=S.FMT_BF16), seed=51)
    pool = _pool(w)
    k16 = pool.k_codes.view(np.uint16)
    for b in range(2):
        L = int(w.seq_lens[b])
        xk = w.rows("k", b, 0, L)[0]
        xv = w.rows("v", b, 0, L)[0]
        bk, bv = O.f32_to_bf16_bits(xk), O.f32_to_bf16_bits(xv)
        for j in (0, 1, 63, 64, L - 1):
            blk, slot = w.block_table[b, j // 64], j % 64
            for h in range(2):
                for d in (0, 5, 17, 64, 127):
                    assert pool.dequant(0, blk, h, slot, d) == float(O.bf16_bits_to_f32(bk[j, h, d:d + 1])[0])
                    assert pool.dequant(1, blk, h, slot, d) == float(O.bf16_bits_to_f32(bv[j, h, d:d + 1])[0])
                    page = blk * 2 + h
                    assert k16[page * 64 * 128 + O.k_byte(slot, d, 128)] == bk[j, h, d]


def test_attention_over_a_bf16_source_is_attention_over_the_source_rows():
    w = S.make(S.tiny_shape(B=1, T=3, Hq=4, Hkv=2, D=128, lens=(140,), src=S.SRC_BF16, fmt=S.FMT_BF16,
                            outliers=True), seed=52)
    pool = _pool(w)
    out = pool.paged_attn(w.q, S.SRC_BF16, 3, 4, w.block_table, w.seq_lens, w.softmax_scale).reshape(3, 4, 128)
    qf = O.bf16_bits_to_f32(w.q).astype(np.float64)
    K = O.bf16_bits_to_f32(w.rows("k", 0, 0, 140))[0].astype(np.float64)
    V = O.bf16_bits_to_f32(w.rows("v", 0, 0, 140))[0].astype(np.float64)
    for kvh in range(2):
        for t in range(3):
            for h in (2 * kvh, 2 * kvh + 1):
                ref = O.dense_attn(qf[0, t, h][None], K[:, kvh], V[:, kvh], float(np.float32(w.softmax_scale)),
                                   np.array([140 - 3 + t], np.int32))
                assert np.array_equal(out[t, h], ref[0])

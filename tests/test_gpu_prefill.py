"""Parity of paged_prefill_attn (chunked-prefill attention over the quantized paged
cache) with the CPU oracle, through the C ABI.

Each case appends its context with kv_append_quant (the chunk's own rows last, as one
batch), checks the pool byte for byte, then compares the prefill attention with the
oracle's fp64 result element by element (max-abs <= 2e-3).  Small cases cover both
launch modes (chunked with a merge, and one chunk per row block written directly),
row blocks with a ragged tail, prefill from an empty cache (causal all the way), both
KV formats and both query dtypes; the 4096-row chunk at the 262,144-token context is
checked on sampled rows.
"""
import dataclasses

import numpy as np
import pytest
import torch

import kvq_synth as S
from tests import gpu_harness as H
from tests.test_gpu_parity import DEV, K, TOL, check, say  # noqa: F401  (K is a fixture)

pytestmark = pytest.mark.gpu

PREFILL = {
    "pf_b2_t100_d128": S.tiny_shape(B=2, T=100, Hq=8, Hkv=2, D=128, lens=(300, 180), src=S.SRC_BF16,
                                    outliers=True),
    "pf_scratch_d256": S.tiny_shape(B=1, T=200, Hq=12, Hkv=2, D=256, lens=(200,), src=S.SRC_BF16, outliers=True),
    "pf_fp8_f32_g6": S.tiny_shape(B=1, T=37, Hq=24, Hkv=4, D=256, lens=(1000,), src=S.SRC_F32,
                                  fmt=S.FMT_FP8_ROW),
    "pf_t1_mha": S.tiny_shape(B=3, T=1, Hq=2, Hkv=2, D=128, lens=(1, 64, 1000), src=S.SRC_F32),
    "pf_int8_f32_long": S.tiny_shape(B=1, T=70, Hq=16, Hkv=2, D=128, lens=(5000,), src=S.SRC_F32),
    "pf_fp8_scratch_bf16": S.tiny_shape(B=2, T=130, Hq=24, Hkv=4, D=256, lens=(130, 333), src=S.SRC_BF16,
                                        fmt=S.FMT_FP8_ROW, outliers=True),
    # bf16 queries over INT8 / FP8 pools take the prefill kernel (128-row blocks): a D=128 FP8 case,
    # rows that end mid-tile (T*G = 3*50 = 150), and a page-aligned context end
    "pf_fp8_d128_g3": S.tiny_shape(B=1, T=50, Hq=6, Hkv=2, D=128, lens=(700,), src=S.SRC_BF16, fmt=S.FMT_FP8_ROW,
                                   outliers=True),
    "pf_int8_b3_ragged": S.tiny_shape(B=3, T=33, Hq=8, Hkv=1, D=256, lens=(33, 64, 1025), src=S.SRC_BF16,
                                      outliers=True),
}


def _direct(K, s, L):
    """One chunk per row block (rows written by the split kernel, no merge)."""
    return K.prefill_workspace_bytes(s.B, s.T, s.Hq, s.Hkv, s.D, L) == 256


def _prefill_rows(w, ts, n_heads, seed=11):
    s = w.shape
    g = np.random.default_rng(seed)
    rows = set()
    for b in range(s.B):
        for t in ts:
            t = min(max(t, 0), s.T - 1)
            for h in g.choice(s.Hq, size=min(n_heads, s.Hq), replace=False):
                rows.add((b * s.T + t) * s.Hq + int(h))
    return np.array(sorted(rows), np.int32)


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_small(K, name):
    w = S.make(PREFILL[name], seed=S.seed_of("tiny") + 500 + list(PREFILL).index(name))
    assert not _direct(K, w.shape, w.max_seq_len)
    check(K, w, chunk=100, prefill=True)


@pytest.mark.parametrize("fmt", [S.FMT_INT8_G64, S.FMT_FP8_ROW])
def test_prefill_direct_rows(K, fmt):
    """8192 query rows per KV head: 64 row blocks of 128 x 2 KV heads x 2 sequences fill
    the chip with one chunk each, so the kernel writes the rows itself."""
    shp = S.tiny_shape(B=2, T=1024, Hq=16, Hkv=2, D=128, lens=(1100, 1500), src=S.SRC_BF16, fmt=fmt,
                       outliers=True, name="pf_direct")
    w = S.make(shp, seed=S.seed_of("tiny") + 600 + fmt)
    assert _direct(K, w.shape, w.max_seq_len)
    check(K, w, rows=_prefill_rows(w, (0, 1, 15, 16, 17, 255, 480, 1023), 5), chunk=300, prefill=True)


@pytest.mark.parametrize("name", ["full256k_int8", "full256k_fp8"])
def test_prefill_chunk_at_full_context_sampled(K, name):
    """The 4096-row prefill chunk whose rows end the 262,144-token context: appended as
    one batch, then its attention (each row sees the 258,048 earlier keys and the chunk's
    rows up to itself)."""
    shp = dataclasses.replace(S.shape(name), T=4096, chunk=0, name=name + "@prefill")
    w = S.make(shp, seed=S.seed_of(name))
    assert _direct(K, w.shape, w.max_seq_len)
    check(K, w, rows=_prefill_rows(w, (0, 1, 2047, 4094, 4095), 2), chunk=65536, prefill=True)


@pytest.mark.parametrize("fmt", [S.FMT_INT8_G64, S.FMT_FP8_ROW])
def test_prefill_chunk_in_rounds_sampled(K, fmt):
    """A 512-row chunk ending a 65,536-token context: 24 row blocks of 128 rows x 4 KV
    heads, so each row block's context is cut into 8 chunks (768 workgroups, three full
    rounds) and merged, with the row blocks dispatched last rows first.  Sampled rows
    over the whole chunk, the first and last rows of row blocks among them."""
    shp = S.tiny_shape(B=1, T=512, Hq=24, Hkv=4, D=256, lens=(65536,), src=S.SRC_BF16, fmt=fmt, outliers=True,
                       name="pf_rounds")
    w = S.make(shp, seed=S.seed_of("tiny") + 700 + fmt)
    assert not _direct(K, w.shape, w.max_seq_len)
    check(K, w, rows=_prefill_rows(w, (0, 1, 21, 22, 255, 490, 511), 3), chunk=8192, prefill=True)


def test_prefill_t_le_8_matches_decode(K):
    """For T <= 8 the prefill call computes what paged_decode_attn computes."""
    w = S.make(S.tiny_shape(B=2, T=4, Hq=24, Hkv=4, D=256, lens=(3000, 515), src=S.SRC_BF16, outliers=True),
               seed=21)
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV)
    dec = H.run_attn(K, w, cache, bt, DEV)
    pre = H.run_attn(K, w, cache, bt, DEV, prefill=True)
    # the two kernels sum in different orders (chunks, wave ownership); both are deterministic,
    # and on this seeded case they differ by 7.6e-6 at most: the bound leaves 4x room for a
    # change of summation order, far inside the 2e-3 bar each holds against the oracle
    diff = float((dec - pre).abs().max())
    say(f"[prefill vs decode] T=4 max-abs difference {diff:.3e}")
    assert diff <= 3e-5


def test_prefill_repeat_is_bit_identical(K):
    w = S.make(PREFILL["pf_b2_t100_d128"], seed=22)
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV)
    a = H.run_attn(K, w, cache, bt, DEV, prefill=True)
    b = H.run_attn(K, w, cache, bt, DEV, prefill=True)
    assert torch.equal(a, b)


@pytest.mark.parametrize("direct", [False, True])
def test_prefill_bad_tables_give_nan_rows_without_touching_others(K, direct):
    T = 1024 if direct else 40
    w = S.make(S.tiny_shape(B=3, T=T, Hq=16, Hkv=2, D=128, lens=(T + 200, T + 300, T + 100), src=S.SRC_BF16),
               seed=23)
    s = w.shape
    assert _direct(K, s, w.max_seq_len) == direct
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV)
    good = H.run_attn(K, w, cache, bt, DEV, prefill=True)
    q = H.src_tensor(w.q, s.src, DEV)
    bt_bad = bt.clone()
    bt_bad[1, 0] = w.num_blocks + 7  # the first page of sequence 1: every row sees it
    sl = torch.tensor([T + 200, T + 300, 10 ** 6], dtype=torch.int32, device=DEV)  # sequence 2 too long
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    L = w.max_seq_len
    ws = K.alloc_prefill_workspace(cache, s.B, s.T, s.Hq, L, device=DEV)
    K.paged_prefill_attn(cache, q, bt_bad, sl, L, w.softmax_scale, out, ws)
    torch.cuda.synchronize()
    say(f"[prefill bad tables] direct={direct}")
    assert torch.equal(out[0], good[0])
    assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all()


def _ragged(seed, B, lo, hi):
    return tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, size=B))


MANY_PF = {
    # 40 sequences x 2 row blocks x 4 KV heads: one chunk per row block, rows written directly
    "pf_b40_direct": dict(B=40, T=40, Hq=24, Hkv=4, D=256, lens=(40,) + _ragged(81, 39, 40, 900)),
    # 8 sequences x 2 row blocks x 1 KV head: chunked contexts and a merge
    "pf_b8_merged": dict(B=8, T=20, Hq=8, Hkv=1, D=128, lens=(20,) + _ragged(82, 7, 20, 3000)),
}


@pytest.mark.parametrize("fmt", [S.FMT_INT8_G64, S.FMT_FP8_ROW, S.FMT_RK8V4])
@pytest.mark.parametrize("name", list(MANY_PF))
def test_prefill_many_sequences(K, name, fmt):
    """Prefill batches of many sequences with ragged contexts (lengths down to T, so some
    sequences prefill from an empty cache): chunks are sized from the longest context and
    the short sequences' later chunks are skipped; both launch modes, sampled rows."""
    shp = S.tiny_shape(src=S.SRC_BF16, fmt=fmt, outliers=True, name=name, **MANY_PF[name])
    w = S.make(shp, seed=S.seed_of("tiny") + 700 + 10 * list(MANY_PF).index(name) + fmt)
    assert _direct(K, w.shape, w.max_seq_len) == name.endswith("direct")
    check(K, w, rows=_prefill_rows(w, (0, 1, shp.T - 1), 2), chunk=128, prefill=True)

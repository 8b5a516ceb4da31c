"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Codes and scales: byte-exact against the oracle's pool.  Attention: max-abs
error <= 2e-3 against the oracle's fp64 result, element by element, on the
same seeded inputs.  Small shapes cover several tiles and ragged tails; the
full-size workloads compare the whole pool and sampled output rows.
"""
import sys

import numpy as np
import pytest
import torch

import kvq_synth as S
import oracle as O
from tests import gpu_harness as H

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import paged_attention_quantized_kv_amd as K
    return K


def check(K, w, rows=None, chunk=8192, prefill=False):
    s = w.shape
    say(f"[parity] {s.name} B={s.B} T={s.T} Hq={s.Hq} Hkv={s.Hkv} D={s.D} lens={s.lens[:8]} fmt={s.fmt} src={s.src}"
        f" prefill={prefill}")
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV, chunk=chunk)
    out = H.run_attn(K, w, cache, bt, DEV, prefill=prefill)
    torch.cuda.synchronize()
    pool = H.oracle_pool(O, w)
    mism = H.pool_equal(cache, pool)
    assert mism == {"k_codes": 0, "v_codes": 0, "k_scales": 0, "v_scales": 0}, mism
    got = out.cpu().numpy().reshape(-1, s.D)
    ref = H.oracle_attn(pool, w, rows)
    if rows is not None:
        got = got[np.asarray(rows)]
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - ref).max())
    say(f"[parity] {s.name}: max-abs err {err:.3e} over {got.size} outputs")
    assert err <= TOL
    return cache, bt, out, err


SMALL = {
    "tiny": S.shape("tiny"),
    "g6_t1_d256_bf16": S.tiny_shape(B=1, T=1, Hq=24, Hkv=4, D=256, lens=(1000,), src=S.SRC_BF16, outliers=True),
    "g6_t4_d256_bf16": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(777,), src=S.SRC_BF16, outliers=True),
    "ragged_b3_t4": S.tiny_shape(B=3, T=4, Hq=12, Hkv=2, D=256, lens=(4, 65, 300), src=S.SRC_BF16, outliers=True),
    "mha_len1": S.tiny_shape(B=2, T=1, Hq=2, Hkv=2, D=256, lens=(1, 130), src=S.SRC_BF16),
    "fp8_d128_f32": S.tiny_shape(B=2, T=2, Hq=8, Hkv=2, D=128, lens=(129, 64), src=S.SRC_F32, fmt=S.FMT_FP8_ROW),
    "fp8_g6_t4_bf16": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(1500,), src=S.SRC_BF16,
                                   fmt=S.FMT_FP8_ROW, outliers=True),
    "rows32_d128": S.tiny_shape(B=2, T=8, Hq=8, Hkv=2, D=128, lens=(513, 70), src=S.SRC_BF16, outliers=True),
    "g8_t2_d256_f32": S.tiny_shape(B=1, T=2, Hq=8, Hkv=1, D=256, lens=(2049,), src=S.SRC_F32),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_shapes(K, name):
    w = S.make(SMALL[name], seed=S.seed_of("tiny") + 100 + list(SMALL).index(name))
    check(K, w, chunk=100)


def _sample_rows(w, n_per_kv=1):
    """Output rows (b, t, h) for every sequence b and every query row t, with n_per_kv query
    heads drawn from the group of each KV head, so every KV head of every row is compared."""
    s = w.shape
    G = s.Hq // s.Hkv
    g = np.random.default_rng(7)
    rows = []
    for b in range(s.B):
        for t in range(s.T):
            for kvh in range(s.Hkv):
                hs = kvh * G + g.choice(G, size=min(n_per_kv, G), replace=False)
                rows += [(b * s.T + t) * s.Hq + int(h) for h in hs]
    return np.array(sorted(set(rows)), np.int32)


def test_qwen32k_full(K):
    check(K, S.make("qwen32k"))


def test_mtp128k_sampled(K):
    w = S.make("mtp128k")
    check(K, w, rows=_sample_rows(w, 2))


def test_cohort_c8_sampled(K):
    w = S.make("c8")
    check(K, w, rows=_sample_rows(w, 1))


@pytest.mark.parametrize("name", ["full256k_int8", "full256k_fp8"])
def test_full_native_context_sampled(K, name):
    w = S.make(name)
    check(K, w, rows=_sample_rows(w, 2), chunk=65536)


def test_repeat_and_page_placement_are_bit_identical(K):
    w = S.make(S.tiny_shape(B=2, T=4, Hq=24, Hkv=4, D=256, lens=(900, 333), src=S.SRC_BF16, outliers=True), seed=5)
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV)
    a = H.run_attn(K, w, cache, bt, DEV)
    b = H.run_attn(K, w, cache, bt, DEV)
    assert torch.equal(a, b)
    # move every page to another physical block and rewrite the table
    n, hkv, D = w.num_blocks, w.shape.Hkv, w.shape.D
    perm = torch.roll(torch.arange(n), 5)
    moved = H.new_cache(K, w, DEV)
    for src_t, dst_t in zip(cache.tensors(), moved.tensors()):
        per = src_t.numel() // n
        dst_t.view(n, per)[perm.to(DEV)] = src_t.view(n, per)
    bt2 = perm.to(DEV)[bt.long()].to(torch.int32).contiguous()
    c = H.run_attn(K, w, moved, bt2, DEV)
    assert torch.equal(a, c)


def test_two_phase_equals_one_call_and_side_stream(K):
    w = S.make(S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(2000,), src=S.SRC_BF16, outliers=True), seed=6)
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV)
    one = H.run_attn(K, w, cache, bt, DEV)
    s = w.shape
    q = H.src_tensor(w.q, s.src, DEV)
    sl = torch.from_numpy(w.seq_lens).to(DEV)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        ws = K.alloc_workspace(cache, s.B, s.T, s.Hq, w.max_seq_len, device=DEV)
        K.paged_decode_attn_split(cache, q, bt, sl, w.max_seq_len, w.softmax_scale, out, ws)
        K.paged_decode_attn_merge(cache, q, bt, sl, w.max_seq_len, w.softmax_scale, out, ws)
    st.synchronize()
    assert torch.equal(one, out)


def test_verify_rows_match_decode_at_shorter_lengths(K):
    w = S.make(S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(1234,), src=S.SRC_BF16, outliers=True), seed=8)
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV)
    out4 = H.run_attn(K, w, cache, bt, DEV).cpu()
    q = H.src_tensor(w.q, w.shape.src, DEV)
    for t in range(4):
        L = 1234 - 4 + t + 1
        sl = torch.tensor([L], dtype=torch.int32, device=DEV)
        q1 = q[:, t:t + 1].contiguous()
        out1 = torch.empty(q1.shape, dtype=torch.float32, device=DEV)
        ws = K.alloc_workspace(cache, 1, 1, 24, L, device=DEV)
        K.paged_decode_attn(cache, q1, bt, sl, L, w.softmax_scale, out1, ws)
        assert float((out1.cpu()[0, 0] - out4[0, t]).abs().max()) <= 1e-5


def test_bad_table_values_give_nan_rows_without_touching_others(K):
    w = S.make(S.tiny_shape(B=3, T=1, Hq=8, Hkv=2, D=128, lens=(200, 300, 100), src=S.SRC_BF16), seed=9)
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV)
    good = H.run_attn(K, w, cache, bt, DEV)
    s = w.shape
    q = H.src_tensor(w.q, s.src, DEV)
    bt_bad = bt.clone()
    bt_bad[1, 2] = w.num_blocks + 7  # block id out of range in sequence 1
    sl = torch.tensor([200, 300, 10 ** 6], dtype=torch.int32, device=DEV)  # sequence 2 too long
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = K.alloc_workspace(cache, s.B, s.T, s.Hq, 300, device=DEV)
    K.paged_decode_attn(cache, q, bt_bad, sl, 300, w.softmax_scale, out, ws)
    assert torch.equal(out[0], good[0])
    assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all()
    # appends with an out-of-range position or block id write nothing
    before = [t.clone() for t in cache.tensors()]
    k = torch.ones((1, 1, 2, 128), dtype=torch.bfloat16, device=DEV)
    K.kv_append_quant(cache, k, k, bt[0:1].contiguous(), torch.tensor([10 ** 7], dtype=torch.int32, device=DEV))
    bt_neg = torch.full((1, 4), -3, dtype=torch.int32, device=DEV)
    K.kv_append_quant(cache, k, k, bt_neg, torch.tensor([0], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    for a, b in zip(before, cache.tensors()):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_fp8_code_conversion_is_exact_for_every_code(K):
    """Each finite E4M3FN code, stored as the single key of its own sequence with a
    unit row scale, must come back exactly (one key: softmax weight 1)."""
    D = 128
    vals = O.e4m3fn_to_f32(np.arange(256, dtype=np.uint16).astype(np.uint8))
    vals = vals[np.isfinite(vals)]
    n = vals.size
    shape = S.tiny_shape(B=n, T=1, Hq=1, Hkv=1, D=D, lens=(1,) * n, src=S.SRC_F32, fmt=S.FMT_FP8_ROW)
    w = S.make(shape, seed=1)
    for b in range(n):
        row = np.zeros((1, 1, D), np.float32)
        row[0, 0, 0] = 448.0  # absmax 448: the row scale is exactly 1
        row[0, 0, 1] = vals[b]
        w.v_src[b] = row
        w.k_src[b] = np.zeros_like(row)
    w.q[:] = 0
    _, _, out, _ = check(K, w)
    got = out.cpu().numpy()[:, 0, 0, :2]
    assert np.array_equal(got[:, 0], np.full(n, 448.0, np.float32))
    assert np.array_equal(got[:, 1], vals)


def _fused_check(K, w, rows=None):
    """Fill all but the T decode rows, then one paged_decode_step call; the pool must
    equal the oracle's and the outputs must match it."""
    s = w.shape
    say(f"[fused] {s.name} B={s.B} T={s.T} lens={s.lens[:8]} fmt={s.fmt}")
    cache = H.new_cache(K, w, DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    for b in range(s.B):
        L = int(w.seq_lens[b])
        if L - s.T > 0:
            k = H.src_tensor(w.rows("k", b, 0, L - s.T), s.src, DEV)
            v = H.src_tensor(w.rows("v", b, 0, L - s.T), s.src, DEV)
            K.kv_append_quant(cache, k, v, bt[b:b + 1].contiguous(), torch.tensor([0], dtype=torch.int32, device=DEV))
    q = H.src_tensor(w.q, s.src, DEV)
    kn = H.src_tensor(w.new_rows("k"), s.src, DEV)
    vn = H.src_tensor(w.new_rows("v"), s.src, DEV)
    sl = torch.from_numpy(w.seq_lens).to(DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = K.alloc_workspace(cache, s.B, s.T, s.Hq, w.max_seq_len, device=DEV)
    K.paged_decode_step(cache, kn, vn, q, bt, sl, w.max_seq_len, w.softmax_scale, out, ws)
    torch.cuda.synchronize()
    pool = H.oracle_pool(O, w)
    mism = H.pool_equal(cache, pool)
    assert mism == {"k_codes": 0, "v_codes": 0, "k_scales": 0, "v_scales": 0}, mism
    got = out.cpu().numpy().reshape(-1, s.D)
    ref = H.oracle_attn(pool, w, rows)
    if rows is not None:
        got = got[np.asarray(rows)]
    err = float(np.abs(got - ref).max())
    say(f"[fused] {s.name}: max-abs err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL
    # the same step through the two separate calls gives bit-identical outputs
    two = H.run_attn(K, w, cache, bt, DEV)
    assert torch.equal(two, out)


@pytest.mark.parametrize("name", ["tiny", "g6_t4_d256_bf16", "ragged_b3_t4", "mha_len1", "fp8_d128_f32",
                                  "rows32_d128"])
def test_fused_step_small(K, name):
    _fused_check(K, S.make(SMALL[name], seed=S.seed_of("tiny") + 200 + list(SMALL).index(name)))


def test_fused_step_mtp128k_and_cohort(K):
    w = S.make("mtp128k")
    _fused_check(K, w, rows=_sample_rows(w, 2))
    w = S.make("c8")
    _fused_check(K, w, rows=_sample_rows(w, 1))


@pytest.mark.parametrize("fmt", [S.FMT_INT8_G64, S.FMT_FP8_ROW])
def test_fused_step_late_rows_straddling_pages(K, fmt):
    """New rows deep inside a chunk (the last page of a 16-page chunk), where the fused
    step quantizes them while the chunk's first page is processed, and rows that straddle
    into the first page of the next chunk, which that chunk writes up front."""
    L0 = 64 * 336 + 2  # rows 21502..21505: page 335 (last of chunk 20) and page 336 (first of chunk 21)
    shp = S.tiny_shape(B=2, T=4, Hq=24, Hkv=4, D=128, lens=(L0, 32768), src=S.SRC_BF16, fmt=fmt, outliers=True,
                       name="late_rows")
    n_splits, tps = K.num_splits(shp.B, shp.T, shp.Hq, shp.Hkv, shp.D, max(shp.lens))
    assert tps == 16 * 64, tps
    assert (L0 - shp.T) // 64 == 16 * 20 + 15 and (L0 - 1) // 64 == 16 * 21
    w = S.make(shp, seed=S.seed_of("tiny") + 300 + fmt)
    _fused_check(K, w, rows=_sample_rows(w, 6))


def test_check_tables_counts_bad_lengths_and_block_ids(K):
    w = S.make(SMALL["ragged_b3_t4"], seed=S.seed_of("tiny") + 400)
    s = w.shape
    cache = H.new_cache(K, w, DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    sl = torch.from_numpy(w.seq_lens).to(DEV)
    res = K.check_tables(cache, s.T, bt, sl, w.max_seq_len)
    torch.cuda.synchronize()
    assert res.tolist() == [0, 0]
    bad_bt = w.block_table.copy()
    bad_bt[2, 0] = -1                      # used page of sequence 2
    bad_bt[2, 1] = w.num_blocks            # used page of sequence 2
    bad_bt[0, bad_bt.shape[1] - 1] = -7    # beyond sequence 0's 4 keys: unused, not counted
    bad_sl = w.seq_lens.copy()
    bad_sl[1] = s.T - 1                    # fewer keys than query rows
    res = K.check_tables(cache, s.T, torch.from_numpy(bad_bt).to(DEV), torch.from_numpy(bad_sl).to(DEV),
                         w.max_seq_len)
    torch.cuda.synchronize()
    assert res.tolist() == [1, 2]


def test_cohort_member_matches_its_own_single_sequence_run(K):
    """Sequence b of a ragged cohort sharing one pool (pages interleaved by the shuffled
    table) gives, to within summation order, what it gives run alone."""
    w = S.make(S.tiny_shape(B=4, T=4, Hq=24, Hkv=4, D=256, lens=(900, 3000, 64, 1777), src=S.SRC_BF16,
                            outliers=True), seed=61)
    s = w.shape
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV)
    cohort = H.run_attn(K, w, cache, bt, DEV)
    q = H.src_tensor(w.q, s.src, DEV)
    for b in range(s.B):
        L = int(w.seq_lens[b])
        sl = torch.tensor([L], dtype=torch.int32, device=DEV)
        qb = q[b:b + 1].contiguous()
        out = torch.empty(qb.shape, dtype=torch.float32, device=DEV)
        ws = K.alloc_workspace(cache, 1, s.T, s.Hq, L, device=DEV)
        K.paged_decode_attn(cache, qb, bt[b:b + 1].contiguous(), sl, L, w.softmax_scale, out, ws)
        torch.cuda.synchronize()
        err = float((out[0] - cohort[b]).abs().max())
        say(f"[cohort] seq {b} L={L}: max-abs difference {err:.2e}")
        assert err <= 1e-4


def _lens(seed, B, lo, hi):
    return tuple(int(x) for x in np.random.default_rng(seed).integers(lo, hi + 1, size=B))


MANY = {
    "b64_t4_int8": S.tiny_shape(B=64, T=4, Hq=24, Hkv=4, D=256, lens=_lens(73, 64, 4, 3000), src=S.SRC_BF16,
                                outliers=True, name="b64_t4_int8"),
    "b300_t1_int8": S.tiny_shape(B=300, T=1, Hq=24, Hkv=4, D=256, lens=_lens(71, 300, 1, 400), src=S.SRC_BF16,
                                 outliers=True, name="b300_t1_int8"),
    "b1024_t2_fp8": S.tiny_shape(B=1024, T=2, Hq=8, Hkv=2, D=128, lens=_lens(72, 1024, 2, 150), src=S.SRC_F32,
                                 fmt=S.FMT_FP8_ROW, name="b1024_t2_fp8"),
    "b600_t1_bf16": S.tiny_shape(B=600, T=1, Hq=8, Hkv=1, D=128, lens=_lens(74, 600, 1, 300), src=S.SRC_BF16,
                                 fmt=S.FMT_BF16, name="b600_t1_bf16"),
}


@pytest.mark.parametrize("name", list(MANY))
def test_many_sequences(K, name):
    """Cohorts up to the 1024-sequence limit with ragged contexts (lengths down to T):
    B * Hkv reaches or passes the 256 workgroups a launch aims for, so each (sequence,
    KV head) is one chunk; both the two-call path and paged_decode_step, which past 512
    split workgroups (b300, b1024, b600) appends with the row kernel before the split."""
    shp = MANY[name]
    n_splits, _ = K.num_splits(shp.B, shp.T, shp.Hq, shp.Hkv, shp.D, max(shp.lens))
    assert n_splits == 1
    w = S.make(shp, seed=S.seed_of("tiny") + 500 + list(MANY).index(name))
    rows = _sample_rows(w, 1)  # one head per KV head of every row of every sequence
    check(K, w, rows=rows)
    _fused_check(K, w, rows=rows)


@pytest.mark.parametrize("shp,chunks", [
    (S.tiny_shape(B=1, T=2, Hq=8, Hkv=1, D=128, lens=(20000,), src=S.SRC_F32, name="splits157_f32"), 157),
    (S.tiny_shape(B=1, T=4, Hq=16, Hkv=2, D=256, lens=(12000,), src=S.SRC_BF16, outliers=True,
                  name="splits94_kv2"), 94),
    (S.tiny_shape(B=2, T=1, Hq=4, Hkv=1, D=128, lens=(40000, 9000), src=S.SRC_BF16, fmt=S.FMT_FP8_ROW,
                  outliers=True, name="splits105_fp8"), 157),
], ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_merge_of_more_than_64_chunks(K, shp, chunks):
    """Few KV heads and long contexts: more than 64 chunks per (sequence, KV head).  157
    chunks in one sequence take four merge waves per slice (the last one idle), 94 take
    two; the balanced two-sequence call (157 chunks for its long sequence, chunk count set
    on the device) takes the one-wave merge through three batches, and its short second
    sequence's rows stop early among them.  Both the two-call path and the fused step."""
    n_splits, _ = K.num_splits(shp.B, shp.T, shp.Hq, shp.Hkv, shp.D, max(shp.lens))
    if shp.B == 1:
        assert n_splits == chunks
    else:  # balanced: the long sequence's chunks, from the device-side rule (pages / even page count)
        pages = [(L + 63) // 64 for L in shp.lens]
        pp = max(2, -(-sum(pages) * shp.Hkv // 256))
        pp += pp % 2
        assert -(-pages[0] // pp) == chunks
    w = S.make(shp, seed=S.seed_of("tiny") + 800 + shp.B)
    check(K, w)
    _fused_check(K, w)


def test_merge_past_256_chunks_at_4m_tokens(K):
    """One KV head at 4,210,688 tokens (65,792 pages): the chunk cap of 256 pages gives 257
    chunks, so the four-wave merge takes chunk 256 in a second round of batches (wave 0,
    slots 256..319).  Every output row against the oracle."""
    L = 257 * 256 * 64
    assert K.num_splits(1, 1, 4, 1, 128, L) == (257, 256 * 64)
    w = S.make(S.tiny_shape(B=1, T=1, Hq=4, Hkv=1, D=128, lens=(L,), src=S.SRC_BF16, name="mqa_4m"), seed=41)
    check(K, w, chunk=1 << 20)


BALANCED = {
    "skew_b8": S.tiny_shape(B=8, T=1, Hq=24, Hkv=4, D=256, lens=(131072, 64, 65, 100, 200, 1, 2, 3000),
                            src=S.SRC_BF16, outliers=True, name="skew_b8"),
    "b32_t4": S.tiny_shape(B=32, T=4, Hq=12, Hkv=2, D=128, lens=tuple(int(x) for x in
                                                                     np.random.default_rng(9).integers(4, 9000, 32)),
                           src=S.SRC_F32, fmt=S.FMT_FP8_ROW, name="b32_t4"),
    "b2_t4_rk8v4": S.tiny_shape(B=2, T=4, Hq=24, Hkv=4, D=256, lens=(30000, 29000), src=S.SRC_BF16,
                                fmt=S.FMT_RK8V4, outliers=True, name="b2_t4_rk8v4"),
    "b48_t2_kv2": S.tiny_shape(B=48, T=2, Hq=8, Hkv=2, D=128, lens=tuple(int(x) for x in
                                                                      np.random.default_rng(10).integers(2, 12000, 48)),
                               src=S.SRC_BF16, outliers=True, name="b48_t2_kv2"),
}


@pytest.mark.parametrize("name", list(BALANCED))
def test_balanced_chunking(K, name):
    """Cohorts of 2..64 sequences with fewer than 256 (sequence, KV head) pairs: chunks of
    one common length set on the device from the actual lengths, so a sequence's chunk
    count follows its own length (a 131,072-token sequence beside tiny ones takes nearly
    all the workgroups).  Parity with the oracle, the two phases called apart equal to the
    one call bit for bit, and the fused step."""
    shp = BALANCED[name]
    w = S.make(shp, seed=S.seed_of("tiny") + 900 + list(BALANCED).index(name))
    rows = _sample_rows(w, 2)
    cache, bt, out, _ = check(K, w, rows=rows)
    s = w.shape
    q = H.src_tensor(w.q, s.src, DEV)
    sl = torch.from_numpy(w.seq_lens).to(DEV)
    two = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = K.alloc_workspace(cache, s.B, s.T, s.Hq, w.max_seq_len, device=DEV)
    K.paged_decode_attn_split(cache, q, bt, sl, w.max_seq_len, w.softmax_scale, two, ws)
    K.paged_decode_attn_merge(cache, q, bt, sl, w.max_seq_len, w.softmax_scale, two, ws)
    torch.cuda.synchronize()
    assert torch.equal(two, out)
    _fused_check(K, w, rows=rows)

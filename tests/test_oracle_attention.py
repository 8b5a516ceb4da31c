"""Pins of the oracle's attention (CPU only).

Closed forms of softmax attention, reductions between call shapes and
invariances fix what the oracle must return without re-deriving it from its
own formula: a dropped max-shift, a wrong GQA head mapping, an off-by-one
causal bound, a transposed page index or a lost scale each break one of them.
"""
import math

import numpy as np
import pytest

import oracle as O
import kvq_synth as S


def _pool_from(w: S.Workload):
    s = w.shape
    pool = O.Pool(s.fmt, w.num_blocks, s.Hkv, s.D, fill=0x7F)
    # poison scales too: an unwritten slot that leaks into an output shows up as NaN
    if s.fmt == O.FMT_INT8_G64:
        pool.k_scales[:] = 0x7E00
        pool.v_scales[:] = 0x7E00
    else:
        pool.k_scales[:] = np.nan
        pool.v_scales[:] = np.nan
    for b in range(s.B):
        bt = w.block_table[b:b + 1]
        pool.append(w.rows("k", b, 0, int(w.seq_lens[b])), w.rows("v", b, 0, int(w.seq_lens[b])), s.src, bt,
                    np.array([0], np.int32))
    return pool


def _dequant_seq(pool, w, b, kvh, n):
    K = np.array([[pool.dequant(0, w.block_table[b, j // 64], kvh, j % 64, d) for d in range(w.shape.D)]
                  for j in range(n)])
    V = np.array([[pool.dequant(1, w.block_table[b, j // 64], kvh, j % 64, d) for d in range(w.shape.D)]
                  for j in range(n)])
    return K, V


# ------------------------------------------------------------------ dense closed forms
def test_dense_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(0)
    L, D = 37, 128
    k, v = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    q = np.zeros((3, D))
    last = np.array([0, 10, 36], np.int32)
    out = O.dense_attn(q, k, v, 0.1, last)
    for r in range(3):
        np.testing.assert_allclose(out[r], v[:last[r] + 1].mean(0), rtol=0, atol=1e-14)


def test_dense_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((1, 64)) * 50, rng.standard_normal((5, 64)), rng.standard_normal((5, 64))
    out = O.dense_attn(q, k, v, 1.0, np.array([0], np.int32))
    assert np.array_equal(out[0], v[0])


def test_dense_two_keys_with_log3_gap_weigh_three_to_one():
    D = 64
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k = np.zeros((2, D))
    k[0, 0] = math.log(3.0)  # logit ln 3 vs 0 -> weights 3/4 and 1/4
    v = np.zeros((2, D))
    v[0, :] = 4.0
    v[1, :] = -8.0
    out = O.dense_attn(q, k, v, 1.0, np.array([1], np.int32))
    np.testing.assert_allclose(out[0], 0.75 * 4.0 + 0.25 * -8.0, rtol=0, atol=1e-14)


def test_dense_dominant_logit_selects_its_value_and_max_shift_prevents_overflow():
    rng = np.random.default_rng(2)
    D, L = 128, 50
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((L, D)) * 0.01
    k[17] = q[0] * 1000.0  # logit ~ 1000 * |q|^2: exp() of it alone overflows binary64
    v = rng.standard_normal((L, D))
    out = O.dense_attn(q, k, v, 1.0, np.array([L - 1], np.int32))
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0], v[17], rtol=0, atol=1e-12)


def test_dense_identical_keys_average_values_and_key_shift_is_invisible():
    rng = np.random.default_rng(3)
    D, L = 64, 20
    q = rng.standard_normal((2, D))
    k = np.tile(rng.standard_normal(D), (L, 1))
    v = rng.standard_normal((L, D))
    out = O.dense_attn(q, k, v, 0.3, np.array([L - 1, 7], np.int32))
    np.testing.assert_allclose(out[0], v.mean(0), atol=1e-14)
    np.testing.assert_allclose(out[1], v[:8].mean(0), atol=1e-14)
    # adding one vector c to every key shifts each row's logits by q.c: softmax is unchanged
    k2 = rng.standard_normal((L, D))
    c = rng.standard_normal(D) * 3
    a = O.dense_attn(q, k2, v, 0.3, np.array([L - 1, 7], np.int32))
    b = O.dense_attn(q, k2 + c, v, 0.3, np.array([L - 1, 7], np.int32))
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_dense_scale_and_query_scaling_commute_and_scale_sharpens():
    rng = np.random.default_rng(4)
    D, L = 64, 30
    q, k, v = rng.standard_normal((1, D)), rng.standard_normal((L, D)), rng.standard_normal((L, D))
    last = np.array([L - 1], np.int32)
    a = O.dense_attn(q, k, v, 0.125, last)
    b = O.dense_attn(q * 0.125, k, v, 1.0, last)
    np.testing.assert_allclose(a, b, atol=1e-13)
    # scale -> 0 tends to the mean; a large scale tends to the arg-max key's value
    z = (k @ q[0])
    np.testing.assert_allclose(O.dense_attn(q, k, v, 1e-12, last)[0], v.mean(0), atol=1e-10)
    np.testing.assert_allclose(O.dense_attn(q, k, v, 1e4, last)[0], v[int(np.argmax(z))], atol=1e-10)


def test_dense_rejects_bad_last():
    with pytest.raises(ValueError):
        O.dense_attn(np.zeros((1, 8)), np.zeros((4, 8)), np.zeros((4, 8)), 1.0, np.array([4], np.int32))


# ------------------------------------------------------------------ paged oracle
def _small(**kw):
    return S.make(S.tiny_shape(**kw), seed=11)


@pytest.mark.parametrize("fmt", [S.FMT_INT8_G64, S.FMT_FP8_ROW])
def test_paged_equals_dense_over_the_gathered_dequantized_cache(fmt):
    w = _small(B=2, T=2, Hq=4, Hkv=2, D=128, lens=(130, 77), src=S.SRC_BF16, fmt=fmt, outliers=True)
    pool = _pool_from(w)
    out = pool.paged_attn(w.q, w.shape.src, 2, 4, w.block_table, w.seq_lens, w.softmax_scale)
    out = out.reshape(2, 2, 4, 128)
    qf = O.bf16_bits_to_f32(w.q).astype(np.float64)
    for b in range(2):
        L = int(w.seq_lens[b])
        for kvh in range(2):
            K, V = _dequant_seq(pool, w, b, kvh, L)
            for t in range(2):
                for h in (2 * kvh, 2 * kvh + 1):
                    ref = O.dense_attn(qf[b, t, h][None], K, V, float(np.float32(w.softmax_scale)),
                                       np.array([L - 2 + t], np.int32))
                    assert np.array_equal(out[b, t, h], ref[0])


def test_paged_is_invariant_to_physical_page_placement():
    w = _small(B=1, T=1, Hq=8, Hkv=1, D=128, lens=(300,))
    pool = _pool_from(w)
    ref = pool.paged_attn(w.q, w.shape.src, 1, 8, w.block_table, w.seq_lens, w.softmax_scale)
    # move every page to a different physical block, rewrite the table, recompute
    n = w.num_blocks
    perm = np.roll(np.arange(n), 3)
    moved = O.Pool(w.shape.fmt, n, 1, 128)
    for arr_src, arr_dst, per in ((pool.k_codes, moved.k_codes, 64 * 128), (pool.v_codes, moved.v_codes, 64 * 128),
                                  (pool.k_scales, moved.k_scales, 128), (pool.v_scales, moved.v_scales, 128)):
        for blk in range(n):
            arr_dst[perm[blk] * per:(perm[blk] + 1) * per] = arr_src[blk * per:(blk + 1) * per]
    bt2 = perm[w.block_table].astype(np.int32)
    got = moved.paged_attn(w.q, w.shape.src, 1, 8, bt2, w.seq_lens, w.softmax_scale)
    assert np.array_equal(got, ref)


def test_paged_zero_query_is_the_mean_of_dequantized_values_up_to_the_causal_bound():
    w = _small(B=1, T=4, Hq=2, Hkv=1, D=128, lens=(131,))
    w.q[:] = 0
    pool = _pool_from(w)
    out = pool.paged_attn(w.q, w.shape.src, 4, 2, w.block_table, w.seq_lens, w.softmax_scale).reshape(4, 2, 128)
    _, V = _dequant_seq(pool, w, 0, 0, 131)
    for t in range(4):
        np.testing.assert_allclose(out[t, 0], V[:131 - 4 + t + 1].mean(0), atol=1e-13)
        np.testing.assert_allclose(out[t, 1], out[t, 0], atol=0)


def test_verify_row_t_equals_decode_at_shorter_length():
    w = _small(B=1, T=4, Hq=4, Hkv=2, D=128, lens=(200,), src=S.SRC_BF16, outliers=True)
    pool = _pool_from(w)
    out4 = pool.paged_attn(w.q, w.shape.src, 4, 4, w.block_table, w.seq_lens, w.softmax_scale).reshape(4, 4, 128)
    for t in range(4):
        q1 = np.ascontiguousarray(w.q[:, t:t + 1])
        out1 = pool.paged_attn(q1, w.shape.src, 1, 4, w.block_table, np.array([200 - 4 + t + 1], np.int32),
                               w.softmax_scale)
        assert np.array_equal(out1.reshape(4, 128), out4[t])


def test_cohort_sequence_equals_its_own_single_sequence_call():
    w = _small(B=3, T=2, Hq=4, Hkv=2, D=128, lens=(70, 190, 129), src=S.SRC_BF16)
    pool = _pool_from(w)
    out = pool.paged_attn(w.q, w.shape.src, 2, 4, w.block_table, w.seq_lens, w.softmax_scale).reshape(3, 2, 4, 128)
    for b in range(3):
        one = pool.paged_attn(np.ascontiguousarray(w.q[b:b + 1]), w.shape.src, 2, 4, w.block_table[b:b + 1],
                              w.seq_lens[b:b + 1], w.softmax_scale)
        assert np.array_equal(one.reshape(2, 4, 128), out[b])


def test_gqa_heads_read_kv_head_h_over_group_size():
    # KV head 1 holds one constant value (127/256 quantizes exactly: scale 2^-8, code 127):
    # query heads 2 and 3 (h // 2 == 1) must return it; heads 0 and 1 must not
    c = 127.0 / 256.0
    w = _small(B=1, T=1, Hq=4, Hkv=2, D=128, lens=(96,))
    w.v_src[0][:, 1, :] = c
    pool = _pool_from(w)
    out = pool.paged_attn(w.q, w.shape.src, 1, 4, w.block_table, w.seq_lens, w.softmax_scale).reshape(4, 128)
    np.testing.assert_allclose(out[2], c, atol=1e-14)
    np.testing.assert_allclose(out[3], c, atol=1e-14)
    assert np.abs(out[0] - c).max() > 0.1 and np.abs(out[1] - c).max() > 0.1


def test_rows_subset_matches_full_call_and_invalid_rows_raise():
    w = _small(B=2, T=1, Hq=4, Hkv=1, D=128, lens=(64, 65))
    pool = _pool_from(w)
    full = pool.paged_attn(w.q, w.shape.src, 1, 4, w.block_table, w.seq_lens, w.softmax_scale)
    rows = np.array([7, 0, 5], np.int32)
    sub = pool.paged_attn(w.q, w.shape.src, 1, 4, w.block_table, w.seq_lens, w.softmax_scale, rows=rows)
    assert np.array_equal(sub, full[rows])
    with pytest.raises(ValueError):
        pool.paged_attn(w.q, w.shape.src, 1, 4, w.block_table, w.seq_lens, w.softmax_scale,
                        rows=np.array([8], np.int32))


def test_outputs_are_finite_although_unwritten_slots_hold_nan():
    w = _small(B=2, T=4, Hq=8, Hkv=2, D=256, lens=(67, 130), src=S.SRC_BF16, fmt=S.FMT_FP8_ROW, outliers=True)
    pool = _pool_from(w)
    out = pool.paged_attn(w.q, w.shape.src, 4, 8, w.block_table, w.seq_lens, w.softmax_scale)
    assert np.all(np.isfinite(out))

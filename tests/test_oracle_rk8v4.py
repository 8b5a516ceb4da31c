"""Pins of the oracle's rk8v4 format (CPU only).

rk8v4 (NInfer-3090 README, "RotorQuant KV (rk8v4)"): keys rotated per 64-dim group
by H64 and stored in the INT8 group-64 encoding; values not rotated, signed 4-bit
codes (15 levels) two per byte over one fp16 scale per 32 dims.  The rotation is
pinned against scipy's Hadamard construction and its closed forms; the 4-bit
quantizer against hand-built ties and its error bound; the layout against a
bijection and hand-worked offsets; the bytes per token against the pages' table;
attention against dense attention over the un-rotated dequantized keys.
"""
import os

import numpy as np
import pytest
import scipy.linalg

import kvq_synth as S
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
H64 = scipy.linalg.hadamard(64).astype(np.float64)  # Sylvester construction


def f16(h):
    return O.f16_bits_to_f32(np.asarray(h, np.uint16)).astype(np.float64)


# ------------------------------------------------------------------ rotation
def test_rotation_matches_scipy_hadamard_over_8():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((200, 64)).astype(np.float32)
    # bf16-representable inputs: the binary64 sum is exact, so the result is the
    # correctly rounded binary32 of the exact rotation
    x = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    want = (x.astype(np.float64) @ H64.T / 8.0).astype(np.float32)
    assert np.array_equal(O.h64_rotate(x), want)


def test_rotation_closed_forms():
    # a unit vector e_i rotates to column i of H64 / 8: +-1/8 with the sign (-1)^popcount(i & j)
    for i in (0, 1, 5, 63):
        e = np.zeros(64, np.float32)
        e[i] = 1.0
        y = O.h64_rotate(e)
        sign = np.array([(-1) ** bin(i & j).count("1") for j in range(64)], np.float64)
        assert np.array_equal(y.astype(np.float64), sign / 8.0)
    # a Hadamard row rotates to 8 e_j; rotating twice is the identity (H64/8 is its own inverse)
    for j in (0, 3, 40):
        y = O.h64_rotate(H64[j].astype(np.float32))
        want = np.zeros(64)
        want[j] = 8.0
        assert np.array_equal(y.astype(np.float64), want)
    x = (np.arange(64, dtype=np.float32) - 20.0) / 4.0  # dyadic: every step exact
    assert np.array_equal(O.h64_rotate(O.h64_rotate(x)), x)
    # orthonormal: the norm is kept
    rng = np.random.default_rng(2)
    z = rng.standard_normal(64).astype(np.float32)
    assert abs(np.linalg.norm(O.h64_rotate(z).astype(np.float64)) - np.linalg.norm(z.astype(np.float64))) < 1e-5


def test_rk8v4_keys_are_the_int8_encoding_of_the_rotated_row():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 256)).astype(np.float32) * np.float32(3.0)
    ck, sk = O.quant_rows(O.FMT_RK8V4, x)
    ci, si = O.quant_rows(O.FMT_INT8_G64, O.h64_rotate(x))
    assert np.array_equal(ck, ci) and np.array_equal(sk, si)
    # a one-hot key at the first dim of a group spreads evenly: every rotated entry is a/8,
    # so every code of that group is +127
    e = np.zeros((1, 128), np.float32)
    e[0, 64] = 5.0
    c, s = O.quant_rows(O.FMT_RK8V4, e)
    assert np.all(c[0, 64:] == 127) and np.all(c[0, :64] == 0)
    assert s[0, 1] == O.f32_to_f16_bits(np.float32(0.625) / np.float32(127.0)) and s[0, 0] == 0


def test_rk8v4_key_round_trip_bound_in_the_original_domain():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    x[:, 7] *= 20  # an outlier channel
    c, s = O.quant_rows(O.FMT_RK8V4, x)
    for g in range(2):
        sc = f16(s[:, g])[:, None]
        yhat = c[:, 64 * g:64 * g + 64].astype(np.float64) * sc           # rotated domain
        xhat = yhat @ H64 / 8.0                                            # un-rotate (H64/8 symmetric, own inverse)
        err = np.linalg.norm(xhat - x[:, 64 * g:64 * g + 64].astype(np.float64), axis=1)
        # each rotated coordinate is off by at most s/2 (plus the fp16 scale's rounding at
        # the clamp), and the rotation keeps the norm
        assert np.all(err <= 8 * (sc[:, 0] / 2) * (1 + 1e-3) + 1e-6)


# ------------------------------------------------------------------ 4-bit values
def test_int4_textbook_ties_with_unit_scale():
    # absmax 7 -> scale fp16(7/7) = 1 exactly; codes are plain round-half-even of x
    x = np.zeros((1, 32), np.float32)
    vals = [7.0, 2.5, 3.5, -2.5, 0.5, 1.5, -7.0, 6.5, -0.5, 4.49]
    x[0, :len(vals)] = vals
    c, s = O.quant_int4_g32(x)
    assert s[0, 0] == 0x3C00  # fp16 1.0
    assert list(c[0, :len(vals)]) == [7, 2, 4, -2, 0, 2, -7, 6, 0, 4]


def test_int4_round_trip_bound_range_and_group_32():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((400, 256)).astype(np.float32)
    x[:, 40] = 40.0  # an outlier in the second 32-dim group only
    c, s = O.quant_int4_g32(x)
    assert c.min() >= -7 and c.max() <= 7
    sc = f16(s)  # [400, 8]
    xhat = c.astype(np.float64) * np.repeat(sc, 32, axis=1)
    err = np.abs(xhat - x.astype(np.float64))
    amax = np.abs(x).reshape(400, 8, 32).max(-1)
    # |x - c s| <= s/2, except at the clamp where the fp16 scale's rounding adds |a - 7 s|
    bound = np.repeat(sc / 2 + np.maximum(0.0, amax - 7 * sc), 32, axis=1)
    assert np.all(err <= bound * (1 + 1e-6))
    idx = np.abs(x.reshape(400, 8, 32)).argmax(-1)
    assert np.all(np.abs(np.take_along_axis(c.reshape(400, 8, 32), idx[..., None], -1)) == 7)
    # the outlier sets only its own group's scale
    assert np.all(sc[:, 1] == f16(O.f32_to_f16_bits(np.float32(40.0) / np.float32(7.0))))
    assert np.all(np.delete(sc, 1, axis=1) < 1.0)


def test_int4_zero_group():
    x = np.zeros((1, 64), np.float32)
    x[0, 40] = 1.0
    c, s = O.quant_int4_g32(x)
    assert s[0, 0] == 0 and np.all(c[0, :32] == 0) and c[0, 40] == 7


# ------------------------------------------------------------------ layout and size
@pytest.mark.parametrize("D", [128, 256])
def test_v4_layout_is_a_bijection_onto_the_page_nibbles(D):
    bits = {O.v4_bit(s, d, D) for s in range(64) for d in range(D)}
    assert bits == set(range(0, 64 * D * 4, 4))
    vs = {O.scale_elem(O.FMT_RK8V4, 1, s, g, D) for s in range(64) for g in range(D // 32)}
    assert vs == set(range(64 * D // 32))
    ks = {O.scale_elem(O.FMT_RK8V4, 0, s, g, D) for s in range(64) for g in range(D // 64)}
    assert ks == {O.scale_elem(O.FMT_INT8_G64, 0, s, g, D) for s in range(64) for g in range(D // 64)}


def test_v4_layout_matches_the_worked_examples():
    """tests/golden/page_layout.txt, rows v4 and vs_rk8v4: worked by hand from include/kvq.h."""
    n = 0
    for line in open(os.path.join(GOLDEN, "page_layout.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        kind, D, sl, dg, off = line.split()
        if kind == "v4":
            assert O.v4_bit(int(sl), int(dg), int(D)) == int(off), line
            n += 1
        elif kind == "vs_rk8v4":
            assert O.scale_elem(O.FMT_RK8V4, 1, int(sl), int(dg), int(D)) == int(off), line
            n += 1
    assert n >= 12


def test_rk8v4_bytes_per_token_match_the_pages_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "kv_format_table.txt")):
        line = line.split("#")[0].split()
        if line:
            rows[line[0]] = [float(v) for v in line[1:]]
    layers, heads, D = int(rows["layers"][0]), int(rows["kv_heads"][0]), int(rows["head_dim"][0])
    p = O.Pool(O.FMT_RK8V4, num_blocks=3, num_kv_heads=heads, head_dim=D)
    per_tok_layer = (p.k_codes.nbytes + p.v_codes.nbytes + p.k_scales.nbytes + p.v_scales.nbytes) / (3 * 64)
    assert per_tok_layer * layers == rows["rk8v4"][0]
    assert per_tok_layer * layers * 2048 / 2 ** 20 == rows["rk8v4"][1]


# ------------------------------------------------------------------ append and attention
def _pool(w):
    s = w.shape
    pool = O.Pool(s.fmt, w.num_blocks, s.Hkv, s.D, fill=0x77)
    pool.k_scales[:] = 0x7E00
    pool.v_scales[:] = 0x7E00
    for b in range(s.B):
        L = int(w.seq_lens[b])
        pool.append(w.rows("k", b, 0, L), w.rows("v", b, 0, L), s.src, w.block_table[b:b + 1],
                    np.array([0], np.int32))
    return pool


def _widen(w, which, b, L):
    x = w.rows(which, b, 0, L)
    return (O.bf16_bits_to_f32(x) if w.shape.src == S.SRC_BF16 else x).astype(np.float32)


def test_append_stores_rotated_keys_and_4bit_values():
    w = S.make(S.tiny_shape(B=2, T=1, Hq=4, Hkv=2, D=128, lens=(150, 70), src=S.SRC_BF16, fmt=S.FMT_RK8V4,
                            outliers=True), seed=31)
    pool = _pool(w)
    for b in range(2):
        L = int(w.seq_lens[b])
        ck, sk = O.quant_rows(O.FMT_RK8V4, _widen(w, "k", b, L)[0])
        cv, sv = O.quant_int4_g32(_widen(w, "v", b, L)[0])
        for j in (0, 1, 63, 64, L - 1):
            blk, slot = w.block_table[b, j // 64], j % 64
            for h in range(2):
                for d in (0, 17, 31, 32, 64, 127):
                    assert pool.dequant(0, blk, h, slot, d) == ck[j, h, d] * f16(sk[j, h, d // 64])
                    assert pool.dequant(1, blk, h, slot, d) == cv[j, h, d] * f16(sv[j, h, d // 32])
    # the nibble of an unwritten slot keeps its poison half-byte
    blk = w.block_table[1, 1]  # second page of sequence 1: slots 6..63 unwritten
    bit = O.v4_bit(40, 3, 128)
    assert (pool.v_codes[blk * 2 * 64 * 64 + bit // 8] >> (bit % 8)) & 0xF == 0x7


def test_attention_equals_dense_attention_over_the_unrotated_keys():
    """The oracle rotates q; the plain definition un-rotates the dequantized keys.  The
    two must agree (a transposed or unnormalized rotation on either side breaks it)."""
    w = S.make(S.tiny_shape(B=1, T=3, Hq=4, Hkv=2, D=128, lens=(140,), src=S.SRC_BF16, fmt=S.FMT_RK8V4,
                            outliers=True), seed=32)
    pool = _pool(w)
    out = pool.paged_attn(w.q, S.SRC_BF16, 3, 4, w.block_table, w.seq_lens, w.softmax_scale).reshape(3, 4, 128)
    qf = O.bf16_bits_to_f32(w.q).astype(np.float64)
    L = 140
    for kvh in range(2):
        Kr = np.array([[pool.dequant(0, w.block_table[0, j // 64], kvh, j % 64, d) for d in range(128)]
                       for j in range(L)])
        V = np.array([[pool.dequant(1, w.block_table[0, j // 64], kvh, j % 64, d) for d in range(128)]
                      for j in range(L)])
        K = np.concatenate([Kr[:, 64 * g:64 * g + 64] @ H64 / 8.0 for g in range(2)], axis=1)
        for t in range(3):
            for h in (2 * kvh, 2 * kvh + 1):
                ref = O.dense_attn(qf[0, t, h][None], K, V, float(np.float32(w.softmax_scale)),
                                   np.array([L - 3 + t], np.int32))
                np.testing.assert_allclose(out[t, h], ref[0], rtol=0, atol=1e-12)


def test_attention_closed_forms_in_rk8v4():
    w = S.make(S.tiny_shape(B=1, T=1, Hq=2, Hkv=1, D=128, lens=(90,), src=S.SRC_BF16, fmt=S.FMT_RK8V4),
               seed=33)
    w.q[:] = 0  # zero query: the mean of the dequantized values
    pool = _pool(w)
    out = pool.paged_attn(w.q, S.SRC_BF16, 1, 2, w.block_table, w.seq_lens, w.softmax_scale)
    V = np.array([[pool.dequant(1, w.block_table[0, j // 64], 0, j % 64, d) for d in range(128)] for j in range(90)])
    np.testing.assert_allclose(out[0], V.mean(0), atol=1e-13)
    # one key: its value, whatever the query
    w1 = S.make(S.tiny_shape(B=1, T=1, Hq=2, Hkv=1, D=128, lens=(1,), src=S.SRC_BF16, fmt=S.FMT_RK8V4), seed=34)
    p1 = _pool(w1)
    o1 = p1.paged_attn(w1.q, S.SRC_BF16, 1, 2, w1.block_table, w1.seq_lens, w1.softmax_scale)
    v0 = np.array([p1.dequant(1, w1.block_table[0, 0], 0, 0, d) for d in range(128)])
    assert np.array_equal(o1[0], v0) and np.array_equal(o1[1], v0)

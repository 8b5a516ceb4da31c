"""Pins of the oracle's rk4v4 format (CPU only).

rk4v4 (NInfer-3090 README, "Lloyd-Max 4-bit keys (rk4v4)"): rk8v4's values; each
rotated key dimension is a 4-bit index into the 16-level Lloyd-Max quantizer for a
Gaussian, whose levels carry fixed INT8 codes, with one fp16 scale per 64 dims.  The
levels are pinned against the optimality conditions (each level the N(0,1) mean of its
cell, computed with scipy; thresholds at midpoints) and against Max's published table;
the quantizer against a brute-force nearest-level search and hand-built ties; the
layout against a bijection and hand-worked offsets; the size against the pages' table.
"""
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.stats

import kvq_synth as S
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
H64 = scipy.linalg.hadamard(64).astype(np.float64)


def _golden(kind):
    out = []
    for line in open(os.path.join(GOLDEN, "lloyd_max16.txt")):
        f = line.split("#")[0].split()
        if f and f[0] == kind:
            out.append(float(f[1]))
    return np.array(out)


def f16(h):
    return O.f16_bits_to_f32(np.asarray(h, np.uint16)).astype(np.float64)


# ------------------------------------------------------------------ the codebook
def test_lloyd_max_levels_satisfy_the_optimality_conditions():
    L = O.lloyd_max16()
    assert np.all(np.diff(L) > 0) and np.allclose(L, -L[::-1], atol=1e-12)
    t = np.concatenate([[-np.inf], (L[:-1] + L[1:]) / 2, [np.inf]])
    for i in range(16):
        mean = scipy.stats.truncnorm.mean(t[i], t[i + 1])  # N(0,1) restricted to the cell
        assert abs(mean - L[i]) < 1e-9


def test_lloyd_max_levels_and_error_match_max_1960():
    L = O.lloyd_max16()
    assert np.allclose(L[8:], _golden("level"), atol=1e-4)
    t = np.concatenate([[-np.inf], (L[:-1] + L[1:]) / 2, [np.inf]])
    mse = sum(scipy.integrate.quad(lambda x, c=L[i]: (x - c) ** 2 * scipy.stats.norm.pdf(x), t[i], t[i + 1])[0]
              for i in range(16))
    # Max's 1960 figures carry the precision of their computation (about 4 digits):
    # the exact fixed point gives 0.0095010
    assert abs(mse - _golden("mse")[0]) < 1e-5


def test_level_codes_match_the_hand_worked_table():
    c = O.rk4_codes().astype(int)
    want = _golden("code").astype(int)
    assert list(c[8:]) == list(want) and list(c[:8]) == list(-want[::-1])


# ------------------------------------------------------------------ the key quantizer
def _unrotate(y):
    """x with rotate(x) = y (H64/8 is its own inverse); exact for dyadic y."""
    return (y.reshape(-1, 64) @ H64 / 8.0).reshape(y.shape).astype(np.float32)


def test_key_index_is_the_nearest_level_code_with_ties_to_the_lower():
    c = O.rk4_codes().astype(np.float64)
    # rotated values chosen directly (multiples of 1/2, so the inverse rotation is exact):
    # absmax 127 gives the scale fp16(127/127) = 1, so u = y
    y = np.zeros(64)
    y[:12] = [127, 12, 0, -24.5, 6, 18, -127, 85.5, -12.25, 1, -1, 111.75]
    idx, s = O.quant_rk4v4_keys(_unrotate(y)[None])
    assert s[0, 0] == 0x3C00
    # ties at the midpoints 12 (6|18), 0 (-6|6), -24.5 (-31|-18), 85.5 (75|96) go to the lower level
    want = [15, 8, 7, 5, 8, 9, 0, 13, 6, 8, 7, 15]
    assert list(idx[0, :12]) == want
    assert np.all(c[idx[0, 12:]] == -6)  # the zeros sit on the -6|6 midpoint


def test_key_index_brute_force_and_absmax_lands_on_the_extreme_level():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((300, 256)).astype(np.float32)
    x[:, 5] *= 20
    idx, s = O.quant_rk4v4_keys(x)
    y = O.h64_rotate(x).astype(np.float64)
    c = O.rk4_codes().astype(np.float64)
    sc = np.repeat(f16(s), 64, axis=1)
    u = np.where(sc != 0, (y.astype(np.float32) / sc.astype(np.float32)).astype(np.float64), 0.0)
    dist = np.abs(u[..., None] - c)  # [300, 256, 16]
    best = dist.min(-1)
    assert np.allclose(dist[np.arange(300)[:, None], np.arange(256)[None], idx], best, atol=0)
    am = np.abs(y.reshape(300, 4, 64)).argmax(-1)
    ext = np.take_along_axis(idx.reshape(300, 4, 64), am[..., None], -1)[..., 0]
    assert np.all((ext == 0) | (ext == 15))


# ------------------------------------------------------------------ layout and size
@pytest.mark.parametrize("D", [128, 256])
def test_k4_layout_is_a_bijection_onto_the_page_nibbles(D):
    bits = {O.k4_bit(s, d, D) for s in range(64) for d in range(D)}
    assert bits == set(range(0, 64 * D * 4, 4))


def test_k4_layout_matches_the_worked_examples():
    n = 0
    for line in open(os.path.join(GOLDEN, "page_layout.txt")):
        if line.startswith("k4 "):
            _, D, sl, d, off = line.split()
            assert O.k4_bit(int(sl), int(d), int(D)) == int(off), line
            n += 1
    assert n >= 10


def test_rk4v4_bytes_per_token_match_the_pages_table():
    rows = {}
    for line in open(os.path.join(GOLDEN, "kv_format_table.txt")):
        f = line.split("#")[0].split()
        if f:
            rows[f[0]] = [float(v) for v in f[1:]]
    layers, heads, D = int(rows["layers"][0]), int(rows["kv_heads"][0]), int(rows["head_dim"][0])
    p = O.Pool(O.FMT_RK4V4, num_blocks=3, num_kv_heads=heads, head_dim=D)
    per_tok_layer = (p.k_codes.nbytes + p.v_codes.nbytes + p.k_scales.nbytes + p.v_scales.nbytes) / (3 * 64)
    assert per_tok_layer * layers == rows["rk4v4"][0]
    assert per_tok_layer * layers * 2048 / 2 ** 20 == rows["rk4v4"][1]


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


def test_append_stores_level_codes_and_rk8v4_values():
    w = S.make(S.tiny_shape(B=2, T=1, Hq=4, Hkv=2, D=128, lens=(150, 70), src=S.SRC_BF16, fmt=S.FMT_RK4V4,
                            outliers=True), seed=41)
    pool = _pool(w)
    c = O.rk4_codes().astype(np.float64)
    for b in range(2):
        L = int(w.seq_lens[b])
        xk = O.bf16_bits_to_f32(w.rows("k", b, 0, L))[0]
        xv = O.bf16_bits_to_f32(w.rows("v", b, 0, L))[0]
        ik, sk = O.quant_rk4v4_keys(xk)
        cv, sv = O.quant_int4_g32(xv)
        for j in (0, 1, 63, 64, L - 1):
            blk, slot = w.block_table[b, j // 64], j % 64
            for h in range(2):
                for d in (0, 3, 4, 8, 17, 64, 127):
                    assert pool.dequant(0, blk, h, slot, d) == c[ik[j, h, d]] * f16(sk[j, h, d // 64])
                    assert pool.dequant(1, blk, h, slot, d) == cv[j, h, d] * f16(sv[j, h, d // 32])


def test_attention_equals_dense_attention_over_the_unrotated_keys():
    w = S.make(S.tiny_shape(B=1, T=2, Hq=4, Hkv=2, D=128, lens=(140,), src=S.SRC_BF16, fmt=S.FMT_RK4V4,
                            outliers=True), seed=42)
    pool = _pool(w)
    out = pool.paged_attn(w.q, S.SRC_BF16, 2, 4, w.block_table, w.seq_lens, w.softmax_scale).reshape(2, 4, 128)
    qf = O.bf16_bits_to_f32(w.q).astype(np.float64)
    L = 140
    for kvh in range(2):
        Kr = np.array([[pool.dequant(0, w.block_table[0, j // 64], kvh, j % 64, d) for d in range(128)]
                       for j in range(L)])
        V = np.array([[pool.dequant(1, w.block_table[0, j // 64], kvh, j % 64, d) for d in range(128)]
                      for j in range(L)])
        K = np.concatenate([Kr[:, 64 * g:64 * g + 64] @ H64 / 8.0 for g in range(2)], axis=1)
        for t in range(2):
            for h in (2 * kvh, 2 * kvh + 1):
                ref = O.dense_attn(qf[0, t, h][None], K, V, float(np.float32(w.softmax_scale)),
                                   np.array([L - 2 + t], np.int32))
                np.testing.assert_allclose(out[t, h], ref[0], rtol=0, atol=1e-12)

"""Pins of the oracle's number formats, quantizers and page layout (CPU only).

Each test checks the oracle against something other than itself: a library
conversion (numpy float16, torch bfloat16 / float8_e4m3fn), a hand-built tie
case, an invariant of the quantizer, or the pages' bytes-per-token table.
"""
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ binary16
def _f16_boundary_probes():
    """For every finite binary16 value: itself, and the binary32 values at and
    one ulp either side of the midpoint to its successor (the rounding edges)."""
    h = np.arange(0, 0x7C00, dtype=np.uint16)  # all finite non-negative halves
    v = h.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65536.0)  # successor (2^16 past the largest finite)
    mid = ((v + nxt) / 2).astype(np.float32)  # exact: midpoints need <= 12 significant bits
    probes = [v.astype(np.float32), mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))]
    x = np.concatenate(probes)
    return np.concatenate([x, -x])


def test_f16_from_f32_matches_numpy_at_every_rounding_edge():
    x = _f16_boundary_probes()
    got = O.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_from_f32_matches_numpy_random_and_special():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(1000),
        (rng.standard_normal(200000) * 1e-5).astype(np.float32),
        (rng.standard_normal(100000) * 1e-7).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.996, 65520, 1e-45, 2.0 ** -25, 2.0 ** -24,
                  3 * 2.0 ** -26], np.float32),
    ])
    got = O.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    nan = O.f32_to_f16_bits(np.array([np.nan], np.float32))
    assert (nan[0] & 0x7C00) == 0x7C00 and (nan[0] & 0x3FF) != 0


def test_f16_to_f32_all_patterns_match_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.f16_bits_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
    assert np.isnan(got[~fin]).all()


def test_bf16_to_f32_all_patterns_match_torch():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_bits_to_f32(b)
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    fin = ~np.isnan(want)
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
    assert np.isnan(got[~fin]).all()


# ------------------------------------------------------------------ E4M3FN
def test_e4m3fn_decode_all_codes_match_torch():
    c = np.arange(256, dtype=np.uint16).astype(np.uint8)
    got = O.e4m3fn_to_f32(c)
    want = torch.from_numpy(c).view(torch.float8_e4m3fn).float().numpy()
    fin = ~np.isnan(want)
    assert fin.sum() == 254  # 0x7F and 0xFF are the only NaNs
    assert np.array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))
    assert np.isnan(got[~fin]).all()
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3fn_encode_matches_torch_in_range():
    mags = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = (mags[:-1] + mags[1:]) / 2
    edge = np.concatenate([mags, mids]).astype(np.float32)
    edge = np.concatenate([edge, np.nextafter(edge, np.float32(0)), np.nextafter(edge, np.float32(1e9))])
    rng = np.random.default_rng(2)
    rnd = np.concatenate([rng.uniform(-448, 448, 200000), rng.standard_normal(100000) * 0.01]).astype(np.float32)
    x = np.concatenate([edge, -edge, rnd])
    x = x[np.abs(x) <= 448]
    got = O.f32_to_e4m3fn(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_e4m3fn_encode_saturates_and_keeps_sign():
    x = np.array([449.0, 463.9, 464.0, 500.0, 1e30, np.inf, -449.0, -1e30, -np.inf, -0.0, -1e-30, np.nan],
                 np.float32)
    got = O.f32_to_e4m3fn(x)
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0xFE, 0x80, 0x80, 0x7F]


# ------------------------------------------------------------------ INT8 group-64
def test_int8_g64_textbook_ties_with_unit_scale():
    # absmax 127 -> s32 = 1 exactly -> s16 = 1.0, so code = rint(x): ties go to even
    x = np.zeros(64, np.float32)
    x[:10] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -126.5, -0.5, 125.5, -3.5]
    codes, scales = O.quant_rows(O.FMT_INT8_G64, x[None])
    assert scales[0, 0] == 0x3C00  # fp16 1.0
    assert codes[0, :10].tolist() == [127, 2, 4, -2, 0, 2, -126, 0, 126, -4]


def test_int8_g64_round_trip_bound_and_absmax_code():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2000, 256)).astype(np.float32)
    x[:, [3, 70, 130, 200]] *= 20.0
    x[5] *= 0.05
    codes, scales = O.quant_rows(O.FMT_INT8_G64, x)
    s = O.f16_bits_to_f32(scales).astype(np.float64)  # [n, 4]
    xg = x.reshape(2000, 4, 64).astype(np.float64)
    cg = codes.reshape(2000, 4, 64).astype(np.float64)
    a = np.abs(xg).max(-1)
    # stored scale is within fp16 rounding of absmax/127 (all scales here are fp16-normal)
    assert np.all(s >= 2.0 ** -14)
    assert np.all(np.abs(s - a / 127) <= a / 127 * 2.0 ** -11)
    # |x - c*s| <= s/2 (+ the fp32 rounding of the quotient)
    err = np.abs(xg - cg * s[..., None])
    assert np.all(err <= s[..., None] / 2 + np.abs(xg) * 2.0 ** -23)
    # the absmax element of each group lands on +-127
    idx = np.abs(xg).argmax(-1)
    top = np.take_along_axis(cg, idx[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 127)
    assert codes.min() >= -127 and codes.max() <= 127


def test_int8_g64_zero_and_subnormal_groups():
    x = np.zeros((3, 128), np.float32)
    x[1, 64:] = np.float32(3e-5)  # a/127 is below fp16's normal range
    x[1, 64] = np.float32(4e-5)
    x[2] = -x[1]
    codes, scales = O.quant_rows(O.FMT_INT8_G64, x)
    assert scales[0].tolist() == [0, 0] and not codes[0].any()
    assert scales[1, 0] == 0 and not codes[1, :64].any()
    s = O.f16_bits_to_f32(scales[1, 1:2])[0]
    assert 0 < s < 2.0 ** -14  # subnormal fp16 scale
    # 4e-5 / s = 134.2 with the subnormal scale 5 * 2^-24: the code clamps to +-127 (the
    # range is symmetric, -128 never appears)
    assert abs(4e-5 / s - 134.2) < 0.1
    assert int(codes[1, 64]) == 127 and int(codes[2, 64]) == -127
    assert np.all(np.abs(codes[1:, 64:].astype(int)) <= 127)
    assert np.array_equal(codes[2].astype(int), -codes[1].astype(int)) and np.array_equal(scales[2], scales[1])


# ------------------------------------------------------------------ FP8 row
def test_fp8_row_round_trip_bound():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((500, 256)).astype(np.float32)
    x[:, [1, 2, 3, 4]] *= 20
    codes, scales = O.quant_rows(O.FMT_FP8_ROW, x)
    a = np.abs(x).max(-1).astype(np.float64)
    assert np.all(np.abs(scales - a / 448) <= a / 448 * 2.0 ** -23)
    dq = O.e4m3fn_to_f32(codes).astype(np.float64) * scales[:, None]
    xs = np.abs(x / scales[:, None])
    normal = xs >= 2.0 ** -6
    err = np.abs(dq - x)
    assert np.all(err[normal] <= np.abs(x[normal]) * 2.0 ** -4 * (1 + 2.0 ** -20))
    assert np.all(err[~normal] <= (2.0 ** -10) * np.broadcast_to(scales[:, None], x.shape)[~normal] * (1 + 1e-6))
    idx = np.abs(x).argmax(-1)
    assert np.all((codes[np.arange(500), idx] & 0x7F) == 0x7E)  # absmax lands on 448


# ------------------------------------------------------------------ layout
@pytest.mark.parametrize("D", [128, 256])
def test_page_layout_is_a_bijection(D):
    k = {O.k_byte(s, d, D) for s in range(64) for d in range(D)}
    v = {O.v_byte(s, d, D) for s in range(64) for d in range(D)}
    assert k == set(range(64 * D)) and v == set(range(64 * D))
    for which in (0, 1):
        si = {O.scale_elem(O.FMT_INT8_G64, which, s, g, D) for s in range(64) for g in range(D // 64)}
        assert si == set(range(64 * D // 64))
        sf = {O.scale_elem(O.FMT_FP8_ROW, which, s, 0, D) for s in range(64)}
        assert sf == set(range(64))


def _golden_table():
    rows = {}
    with open(os.path.join(GOLDEN, "kv_format_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                rows[line[0]] = [float(v) for v in line[1:]]
    return rows


def test_page_layout_matches_the_worked_examples():
    """tests/golden/page_layout.txt: offsets worked by hand from the layout in include/kvq.h."""
    path = os.path.join(os.path.dirname(__file__), "golden", "page_layout.txt")
    n = 0
    for line in open(path):
        if not line.strip() or line.startswith("#"):
            continue
        kind, D, sl, dg, off = line.split()
        D, sl, dg, off = int(D), int(sl), int(dg), int(off)
        if kind in ("v4", "vs_rk8v4", "k4"):  # checked in test_oracle_rk8v4.py / test_oracle_rk4v4.py
            continue
        if kind == "k":
            got = O.k_byte(sl, dg, D)
        elif kind == "v":
            got = O.v_byte(sl, dg, D)
        elif kind == "ks_int8":
            got = O.scale_elem(O.FMT_INT8_G64, 0, sl, dg, D)
        elif kind == "vs_int8":
            got = O.scale_elem(O.FMT_INT8_G64, 1, sl, dg, D)
        else:
            got = O.scale_elem(O.FMT_FP8_ROW, 0, sl, 0, D)
            assert O.scale_elem(O.FMT_FP8_ROW, 1, sl, 0, D) == got
        assert got == off, line
        n += 1
    assert n >= 40


def test_bytes_per_token_match_the_pages_table():
    t = _golden_table()
    layers, heads, D = int(t["layers"][0]), int(t["kv_heads"][0]), int(t["head_dim"][0])
    # INT8 g64: the pool's bytes per (token, layer, KV head) over K and V, times the model
    p = O.Pool(O.FMT_INT8_G64, num_blocks=3, num_kv_heads=heads, head_dim=D)
    per_tok_layer = (p.k_codes.nbytes + p.v_codes.nbytes + p.k_scales.nbytes + p.v_scales.nbytes) / (3 * 64)
    assert per_tok_layer * layers == t["int8"][0]
    assert per_tok_layer * layers * 2048 / 2 ** 20 == t["int8"][1]
    # FP8: the code bytes reproduce the table; the scale is one fp32 per token per KV head
    # (32 bytes more per token than the table's total, which implies 2-byte row scales)
    f = O.Pool(O.FMT_FP8_ROW, num_blocks=3, num_kv_heads=heads, head_dim=D)
    code_bytes = (f.k_codes.nbytes + f.v_codes.nbytes) / (3 * 64) * layers
    assert code_bytes == 32768 and t["fp8"][0] - code_bytes == 256
    # bf16 for scale: 2 bytes per element, K and V
    assert 2 * 2 * heads * D * layers == t["bf16"][0]


# ------------------------------------------------------------------ append
@pytest.mark.parametrize("fmt", [O.FMT_INT8_G64, O.FMT_FP8_ROW])
def test_append_scatters_quantized_rows_through_the_block_table(fmt):
    rng = np.random.default_rng(5)
    H, D, nblk = 2, 128, 6
    pool = O.Pool(fmt, nblk, H, D, fill=0x7F)
    bt = np.array([[4, 1, 5], [0, 3, 2]], np.int32)
    x_k = rng.standard_normal((2, 70, H, D)).astype(np.float32)
    x_v = rng.standard_normal((2, 70, H, D)).astype(np.float32)
    start = np.array([10, 100], np.int32)
    pool.append(x_k, x_v, O.SRC_F32, bt, start)
    ck, sk = O.quant_rows(fmt, x_k)
    cv, sv = O.quant_rows(fmt, x_v)
    def dec(c):
        c = np.asarray(c).reshape(1)
        return float((O.e4m3fn_to_f32(c) if fmt == O.FMT_FP8_ROW else c.astype(np.float32))[0])

    def f16(h):
        return float(O.f16_bits_to_f32(np.asarray(h).reshape(1))[0])
    for b in range(2):
        for t in (0, 1, 53, 54, 69):
            pos = start[b] + t
            blk, slot = bt[b, pos // 64], pos % 64
            for h in range(H):
                for d in (0, 5, 63, 64, 127):
                    if fmt == O.FMT_INT8_G64:
                        want_k = dec(ck[b, t, h, d]) * f16(sk[b, t, h, d // 64])
                        want_v = dec(cv[b, t, h, d]) * f16(sv[b, t, h, d // 64])
                    else:
                        want_k = dec(ck[b, t, h, d]) * float(sk[b, t, h])
                        want_v = dec(cv[b, t, h, d]) * float(sv[b, t, h])
                    assert pool.dequant(0, blk, h, slot, d) == want_k
                    assert pool.dequant(1, blk, h, slot, d) == want_v
    # slots before the first appended row, and blocks never referenced, keep the poison bytes
    first = O.k_byte(9, 0, D)
    assert pool.k_codes[4 * H * 64 * D + first] == 0x7F
    # sequence 1 ends at position 169: slot 42 of its third block (2) was never written
    assert pool.v_codes[2 * H * 64 * D + O.v_byte(42, 7, D)] == 0x7F


def test_append_rejects_positions_outside_the_table():
    pool = O.Pool(O.FMT_INT8_G64, 2, 1, 128)
    x = np.zeros((1, 2, 1, 128), np.float32)
    with pytest.raises(ValueError):
        pool.append(x, x, O.SRC_F32, np.array([[0, 1]], np.int32), np.array([127], np.int32))
    with pytest.raises(ValueError):
        pool.append(x, x, O.SRC_F32, np.array([[0, 7]], np.int32), np.array([63], np.int32))

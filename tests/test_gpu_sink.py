"""Parity where the P.V operands span a wide dynamic range: attention sinks, and value
rows of widely different magnitudes, in every chunking mode.

A few keys lie 13-16 nats above thousands of near-uniform keys whose values have
a nonzero mean (kvq_synth.make_sink).  The near-uniform keys' weights are tiny
(e^-13 ~ 2e-6 of the sink's) but there are so many of them that together they
carry a visible share of the output, so a kernel that loses or biases small
weights in P.V misses the 2e-3 bar here even though it passes on N(0,1) data.
The sinks sit at chunk starts, so every context chunk of the split has one.

Modes: 64 chunks per KV head (128K T=4, 256K T=1), chunks of a common length set
from the lengths in the C=8-shaped cohort, one chunk per (sequence, KV head) in a 64-sequence
cohort, and prefill with one chunk over the whole context (the prefill kernel and
the split kernel's prefill instance).  Codes and scales are compared byte for
byte, attention element by element against the fp64 oracle on every query row t
of the sampled heads.
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
FMTS = {"int8": S.FMT_INT8_G64, "fp8": S.FMT_FP8_ROW, "rk8v4": S.FMT_RK8V4, "rk4v4": S.FMT_RK4V4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    import paged_attention_quantized_kv_amd as K
    return K


def rows_every_t(w, heads_per_seq, ts=None, seed=11):
    """Output rows (b, t, h) for a few heads of every sequence and every t (or the given t)."""
    s = w.shape
    g = np.random.default_rng(seed)
    rows = []
    for b in range(s.B):
        hs = g.choice(s.Hq, size=min(heads_per_seq, s.Hq), replace=False)
        for t in (range(s.T) if ts is None else ts):
            rows += [(b * s.T + t) * s.Hq + int(h) for h in hs]
    return np.array(sorted(set(rows)), np.int32)


def check(K, w, rows, chunk=65536, prefill=False, label=""):
    s = w.shape
    say(f"[sink] {label} B={s.B} T={s.T} Hq={s.Hq} Hkv={s.Hkv} D={s.D} lens={s.lens[:4]}... fmt={s.fmt} "
        f"prefill={prefill} rows={len(rows)}")
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV, chunk=chunk)
    out = H.run_attn(K, w, cache, bt, DEV, prefill=prefill)
    torch.cuda.synchronize()
    pool = H.oracle_pool(O, w)
    mism = H.pool_equal(cache, pool)
    assert mism == {"k_codes": 0, "v_codes": 0, "k_scales": 0, "v_scales": 0}, mism
    got = out.cpu().numpy().reshape(-1, s.D)[rows]
    ref = H.oracle_attn(pool, w, rows)
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - ref).max())
    say(f"[sink] {label}: max-abs err {err:.3e} over {got.size} outputs")
    assert err <= TOL, err


@pytest.mark.parametrize("fmt", list(FMTS))
def test_sink_128k_t4_64_chunks(K, fmt):
    shp = S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(131072,), src=S.SRC_BF16, fmt=FMTS[fmt])
    w = S.make_sink(shp, gap_nats=13.0, stride=2048, seed=1)
    assert K.num_splits(1, 4, 24, 4, 256, 131072)[1] == 2048
    check(K, w, rows_every_t(w, 2), label=f"128K T=4 {fmt}")


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_sink_256k_t1_64_chunks(K, fmt):
    shp = S.tiny_shape(B=1, T=1, Hq=24, Hkv=4, D=256, lens=(262144,), src=S.SRC_BF16, fmt=FMTS[fmt])
    w = S.make_sink(shp, gap_nats=13.0, stride=4096, seed=2)
    assert K.num_splits(1, 1, 24, 4, 256, 262144)[1] == 4096
    check(K, w, rows_every_t(w, 3), label=f"256K T=1 {fmt}")


def balanced_chunk_tokens(lens, Hkv, W=256):
    """Chunk length of a balanced call (2..64 sequences, fewer than 256 (sequence, KV head)
    pairs): the smallest even page count (at most 256) for
    which the call's chunks, sum of ceil(pages / length) over (sequence, KV head), fit in W."""
    pages = [(L + 63) // 64 for L in lens]
    count = lambda q: Hkv * sum(max(1, -(-p // q)) for p in pages)
    pp = next(q for q in range(2, max(pages) + 3, 2) if count(q) <= W)
    return min(pp, 256) * 64


@pytest.mark.parametrize("fmt,gap", [("int8", 13.0), ("fp8", 13.0), ("int8", 16.0), ("rk8v4", 13.0)])
def test_sink_cohort_8_chunks(K, fmt, gap):
    g = np.random.default_rng(3)
    lens = [int(x) for x in g.integers(4096, 65536 + 1, 8)]
    shp = S.tiny_shape(B=8, T=4, Hq=24, Hkv=4, D=256, lens=lens, src=S.SRC_BF16, fmt=FMTS[fmt])
    tps = balanced_chunk_tokens(lens, 4)
    w = S.make_sink(shp, gap_nats=gap, stride=tps, seed=3)
    check(K, w, rows_every_t(w, 1), label=f"C=8 {fmt} gap {gap} ({tps}-token chunks)")


@pytest.mark.parametrize("fmt,T", [("int8", 1), ("fp8", 1), ("int8", 4)])
def test_sink_cohort_one_chunk_per_sequence(K, fmt, T):
    g = np.random.default_rng(4)
    lens = [int(x) for x in g.integers(6000, 8192 + 1, 64)]
    shp = S.tiny_shape(B=64, T=T, Hq=24, Hkv=4, D=256, lens=lens, src=S.SRC_BF16, fmt=FMTS[fmt])
    n, tps = K.num_splits(64, T, 24, 4, 256, max(lens))
    assert n == 1
    w = S.make_sink(shp, gap_nats=13.0, stride=tps, seed=4)
    check(K, w, rows_every_t(w, 1), chunk=8192, label=f"64 sequences T={T} {fmt}")


@pytest.mark.parametrize("fmt,T,src", [("int8", 1536, S.SRC_BF16), ("fp8", 1536, S.SRC_BF16),
                                       ("rk8v4", 1024, S.SRC_BF16), ("int8", 1024, S.SRC_F32)])
def test_sink_prefill_one_chunk(K, fmt, T, src):
    # T rows x 6 query heads per KV head fill >= 256 row blocks of 4 KV heads, so each block
    # streams the whole 65,536-token context as one chunk and writes its rows directly
    shp = S.tiny_shape(B=1, T=T, Hq=24, Hkv=4, D=256, lens=(65536,), src=src, fmt=FMTS[fmt])
    w = S.make_sink(shp, gap_nats=13.0, stride=16384, seed=5)
    check(K, w, rows_every_t(w, 2, ts=(0, T // 2, T - 1)), prefill=True, label=f"prefill T={T} {fmt} src={src}")


# Value rows whose magnitudes span 2^-6 .. 2^6: the largest V scale of a page sits on any
# slot, so an exponent taken from part of the page's scales would overflow the products.
WIDE = {
    "int8_t4": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(20000,), src=S.SRC_BF16),
    "int8_t1_d128_f32": S.tiny_shape(B=2, T=1, Hq=8, Hkv=2, D=128, lens=(9000, 3000), src=S.SRC_F32),
    "fp8_t4": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(20000,), src=S.SRC_BF16, fmt=S.FMT_FP8_ROW),
    "rk8v4_t4": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(20000,), src=S.SRC_BF16, fmt=S.FMT_RK8V4),
    "rk4v4_t1": S.tiny_shape(B=1, T=1, Hq=24, Hkv=4, D=256, lens=(20000,), src=S.SRC_BF16, fmt=S.FMT_RK4V4),
    "bf16_t4": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(20000,), src=S.SRC_BF16, fmt=S.FMT_BF16),
}


@pytest.mark.parametrize("name", list(WIDE))
def test_wide_value_rows(K, name):
    w = S.make_wide(WIDE[name], span_log2=6.0, seed=list(WIDE).index(name))
    check(K, w, rows_every_t(w, 4), chunk=4096, label=f"wide V rows {name}")


@pytest.mark.parametrize("fmt,src", [("int8", S.SRC_BF16), ("fp8", S.SRC_BF16), ("int8", S.SRC_F32)])
def test_wide_value_rows_prefill(K, fmt, src):
    shp = S.tiny_shape(B=1, T=300, Hq=24, Hkv=4, D=256, lens=(6000,), src=src, fmt=FMTS[fmt])
    w = S.make_wide(shp, span_log2=6.0, seed=7)
    check(K, w, rows_every_t(w, 2, ts=(0, 150, 299)), chunk=4096, prefill=True, label=f"wide V rows prefill {fmt}")


@pytest.mark.parametrize("run", [0, 1, 2, 3])
@pytest.mark.parametrize("fmt", ["int8", "fp8", "rk8v4"])
def test_striped_value_rows(K, fmt, run):
    # every 16-slot run of a page holds the same four rows at 2^-6 and twelve at 2^6, so the
    # four 16-lane groups of a wave see different largest V scales: the exponent must come
    # from all of them, or the large rows' products overflow f16
    shp = S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(8192,), src=S.SRC_BF16, fmt=FMTS[fmt])
    w = S.make_wide(shp, span_log2=6.0, seed=20 + run, small_run=run)
    check(K, w, rows_every_t(w, 3), chunk=4096, label=f"striped V rows {fmt} small run {run}")

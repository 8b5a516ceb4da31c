"""Parity of the rk8v4 format (H64-rotated INT8 group-64 keys, signed 4-bit group-32
values) on the HIP path with the CPU oracle, through the C ABI.

Pools byte for byte (codes, nibbles and scales) after appends through both append
kernels (chunks of 64+ rows page by page, fewer rows row by row, pages shared by
several chunks and by the decode rows), then attention within 2e-3 of the oracle's fp64
result: decode (T = 1 and 4), the fused decode step, prefill, the 128K T=4 workload.
"""
import numpy as np
import pytest
import torch

import kvq_synth as S
from tests import gpu_harness as H
from tests.test_gpu_parity import DEV, K, TOL, _fused_check, _sample_rows, check, say  # noqa: F401

pytestmark = pytest.mark.gpu

RK = S.FMT_RK8V4
SMALL = {
    "rk_t1_d128_f32": S.tiny_shape(B=1, T=1, Hq=8, Hkv=1, D=128, lens=(2048,), src=S.SRC_F32, fmt=RK),
    "rk_t4_d256_bf16": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(777,), src=S.SRC_BF16, fmt=RK,
                                    outliers=True),
    "rk_ragged_b3": S.tiny_shape(B=3, T=4, Hq=12, Hkv=2, D=256, lens=(4, 65, 300), src=S.SRC_BF16, fmt=RK,
                                 outliers=True),
    "rk_rows32_d128": S.tiny_shape(B=2, T=8, Hq=8, Hkv=2, D=128, lens=(513, 70), src=S.SRC_BF16, fmt=RK,
                                   outliers=True),
    "rk_g8_t2_f32": S.tiny_shape(B=1, T=2, Hq=8, Hkv=1, D=256, lens=(2049,), src=S.SRC_F32, fmt=RK),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_rk8v4_small_shapes(K, name):
    w = S.make(SMALL[name], seed=S.seed_of("tiny") + 700 + list(SMALL).index(name))
    check(K, w, chunk=100)


@pytest.mark.parametrize("name", ["rk_t4_d256_bf16", "rk_ragged_b3", "rk_rows32_d128"])
def test_rk8v4_fused_step(K, name):
    _fused_check(K, S.make(SMALL[name], seed=S.seed_of("tiny") + 750 + list(SMALL).index(name)))


def test_rk8v4_prefill(K):
    w = S.make(S.tiny_shape(B=2, T=100, Hq=24, Hkv=4, D=256, lens=(300, 180), src=S.SRC_BF16, fmt=RK,
                            outliers=True), seed=S.seed_of("tiny") + 780)
    check(K, w, chunk=100, prefill=True)


def test_rk8v4_mtp128k_sampled(K):
    w = S.make("mtp128k_rk8v4")
    check(K, w, rows=_sample_rows(w, 2), chunk=65536)


def test_rk8v4_single_row_appends_share_nibble_words(K):
    """Rows appended one call at a time (each call's rows land in words that earlier
    calls filled) and T = 8 rows of several sequences in one call must leave the pool
    identical to the oracle's."""
    w = S.make(S.tiny_shape(B=2, T=8, Hq=8, Hkv=2, D=128, lens=(90, 37), src=S.SRC_BF16, fmt=RK), seed=791)
    s = w.shape
    cache = H.new_cache(K, w, DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    for b in range(s.B):
        L = int(w.seq_lens[b])
        for t in range(L - s.T):  # one row per call
            k = H.src_tensor(w.rows("k", b, t, t + 1), s.src, DEV)
            v = H.src_tensor(w.rows("v", b, t, t + 1), s.src, DEV)
            K.kv_append_quant(cache, k, v, bt[b:b + 1].contiguous(), torch.tensor([t], dtype=torch.int32, device=DEV))
    k = H.src_tensor(w.new_rows("k"), s.src, DEV)
    v = H.src_tensor(w.new_rows("v"), s.src, DEV)
    K.kv_append_quant(cache, k, v, bt, torch.from_numpy(w.seq_lens - s.T).to(DEV))
    torch.cuda.synchronize()
    import oracle as O
    pool = H.oracle_pool(O, w)
    mism = H.pool_equal(cache, pool)
    say(f"[rk8v4 rows] mismatches {mism}")
    assert mism == {"k_codes": 0, "v_codes": 0, "k_scales": 0, "v_scales": 0}, mism


@pytest.mark.parametrize("fmt", [RK, S.FMT_RK4V4, S.FMT_INT8_G64])
def test_step_skips_sequences_with_bad_lengths(K, fmt):
    """paged_decode_step with one sequence longer than max_seq_len: that sequence's new rows
    are not written and its output rows are NaN; the other sequences' rows land exactly
    where kv_append_quant puts them.  With 24 query rows per KV head the rotated formats
    append through a separate launch first, INT8 inside the split launch: same outcome."""
    w = S.make(S.tiny_shape(B=3, T=4, Hq=24, Hkv=4, D=256, lens=(300, 500, 200), src=S.SRC_BF16, fmt=fmt,
                            outliers=True), seed=S.seed_of("tiny") + 790 + fmt)
    s = w.shape
    bt = torch.from_numpy(w.block_table).to(DEV)
    caches = [H.new_cache(K, w, DEV), H.new_cache(K, w, DEV)]
    for cache in caches:  # every context row but the T new ones
        for b in range(s.B):
            L = int(w.seq_lens[b])
            k = H.src_tensor(w.rows("k", b, 0, L - s.T), s.src, DEV)
            v = H.src_tensor(w.rows("v", b, 0, L - s.T), s.src, DEV)
            K.kv_append_quant(cache, k, v, bt[b:b + 1].contiguous(), torch.tensor([0], dtype=torch.int32, device=DEV))
    kn = H.src_tensor(w.new_rows("k"), s.src, DEV)
    vn = H.src_tensor(w.new_rows("v"), s.src, DEV)
    # reference pool: the new rows of sequences 0 and 1 only, through kv_append_quant
    sp = torch.from_numpy(w.seq_lens[:2] - s.T).to(DEV)
    K.kv_append_quant(caches[1], kn[:2].contiguous(), vn[:2].contiguous(), bt[:2].contiguous(), sp)
    q = H.src_tensor(w.q, s.src, DEV)
    sl = torch.from_numpy(w.seq_lens).to(DEV)
    sl[2] = w.max_seq_len + 5  # beyond max_seq_len: the sequence is skipped
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    ws = K.alloc_workspace(caches[0], s.B, s.T, s.Hq, w.max_seq_len, device=DEV)
    K.paged_decode_step(caches[0], kn, vn, q, bt, sl, w.max_seq_len, w.softmax_scale, out, ws)
    torch.cuda.synchronize()
    say(f"[step bad length] fmt={fmt}")
    for a, b in zip(caches[0].tensors(), caches[1].tensors()):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    assert torch.isnan(out[2]).all()
    assert torch.isfinite(out[:2]).all()

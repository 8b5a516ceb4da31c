"""Queries outside f16's range: each query row enters the matrix cores scaled by a power of
two chosen from its largest element, and its scores take the power of two back.

Rows are scaled by 2^17 (bf16 values up to ~5e5, beyond f16's 65504) or 2^-20 (below
f16's normal range), exactly, since a power of two moves only the exponent.  The softmax
scale is divided by the largest factor, so those rows give the unscaled attention and the
others near-uniform softmaxes (logits stay moderate: at logits near 1e6 nats fp32 score
rounding alone reaches 0.1 nat, which is no property of the range handling).  Every case
is compared element by element with the fp64 oracle.
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


def scale_queries(w, head_log2):
    """Multiply query head h of every row by 2^head_log2[h % len(head_log2)] (exact)."""
    s = w.shape
    f = np.array([2.0 ** head_log2[h % len(head_log2)] for h in range(s.Hq)], np.float32)[None, None, :, None]
    if s.src == S.SRC_BF16:
        x = O.bf16_bits_to_f32(w.q) * f
        w.q = O.f32_to_bf16_bits(x)
        assert np.array_equal(O.bf16_bits_to_f32(w.q), x)
    else:
        w.q = (w.q * f).astype(np.float32)


def check(K, w, prefill=False, label=""):
    s = w.shape
    say(f"[qrange] {label}")
    cache = H.new_cache(K, w, DEV)
    bt = H.fill_gpu(K, w, cache, DEV, chunk=2048)
    out = H.run_attn(K, w, cache, bt, DEV, prefill=prefill)
    torch.cuda.synchronize()
    pool = H.oracle_pool(O, w)
    got = out.cpu().numpy().reshape(-1, s.D)
    ref = H.oracle_attn(pool, w)
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - ref).max())
    say(f"[qrange] {label}: max-abs err {err:.3e} over {got.size} outputs")
    assert err <= TOL, err


CASES = {
    "int8_bf16": (S.FMT_INT8_G64, S.SRC_BF16),
    "int8_f32": (S.FMT_INT8_G64, S.SRC_F32),
    "fp8_bf16": (S.FMT_FP8_ROW, S.SRC_BF16),
    "rk8v4_bf16": (S.FMT_RK8V4, S.SRC_BF16),
    "rk4v4_bf16": (S.FMT_RK4V4, S.SRC_BF16),
    "bf16_bf16": (S.FMT_BF16, S.SRC_BF16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_large_rows_compensated(K, name):
    fmt, src = CASES[name]
    w = S.make(S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(3000,), src=src, fmt=fmt, outliers=True), seed=31)
    scale_queries(w, [17])
    w.softmax_scale = float(np.float32(w.softmax_scale * 2.0 ** -17))
    check(K, w, label=f"rows x2^17, scale / 2^17, {name}")


@pytest.mark.parametrize("name", list(CASES))
def test_mixed_row_magnitudes(K, name):
    fmt, src = CASES[name]
    w = S.make(S.tiny_shape(B=2, T=2, Hq=12, Hkv=2, D=256, lens=(1500, 700), src=src, fmt=fmt, outliers=True), seed=32)
    scale_queries(w, [17, 0, -20, 3, -8, 12])
    w.softmax_scale = float(np.float32(w.softmax_scale * 2.0 ** -17))
    check(K, w, label=f"rows x2^(17, 0, -20, 3, -8, 12), scale / 2^17, {name}")


def test_bf16_rows_at_the_f16_limit(K):
    # largest elements 65504 (f16's largest finite) and 65536 = 2^16 (beyond it): both bf16 values
    w = S.make(S.tiny_shape(B=1, T=1, Hq=8, Hkv=2, D=128, lens=(900,), src=S.SRC_BF16), seed=33)
    x = O.bf16_bits_to_f32(w.q)
    x[0, 0, :4, 5] = 65280.0  # the largest bf16 below 65504
    x[0, 0, 4:, 5] = 65536.0
    w.q = O.f32_to_bf16_bits(x)
    assert np.array_equal(O.bf16_bits_to_f32(w.q), x)
    w.softmax_scale = float(np.float32(1.0 / 65536.0))
    check(K, w, label="bf16 rows with elements 65280 and 65536")


@pytest.mark.parametrize("fmt", [S.FMT_INT8_G64, S.FMT_FP8_ROW])
def test_prefill_large_rows(K, fmt):
    w = S.make(S.tiny_shape(B=1, T=200, Hq=24, Hkv=4, D=256, lens=(2500,), src=S.SRC_BF16, fmt=fmt, outliers=True),
               seed=34)
    scale_queries(w, [17, -20, 0])
    w.softmax_scale = float(np.float32(w.softmax_scale * 2.0 ** -17))
    check(K, w, prefill=True, label=f"prefill rows x2^(17, -20, 0), scale / 2^17, fmt {fmt}")

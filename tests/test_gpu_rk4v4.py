"""Parity of the rk4v4 format (4-bit Lloyd-Max key indices over the INT8 group scale of
the rotated key, rk8v4's 4-bit values) on the HIP path with the CPU oracle, through the
C ABI: pools byte for byte after appends through both append kernels, attention within
2e-3 of the oracle's fp64 result for decode, the fused step, prefill and the 128K T=4
workload.
"""
import pytest

import kvq_synth as S
from tests.test_gpu_parity import K, _fused_check, _sample_rows, check  # noqa: F401

pytestmark = pytest.mark.gpu

R4 = S.FMT_RK4V4
SMALL = {
    "r4_t1_d128_f32": S.tiny_shape(B=1, T=1, Hq=8, Hkv=1, D=128, lens=(2048,), src=S.SRC_F32, fmt=R4),
    "r4_t4_d256_bf16": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(777,), src=S.SRC_BF16, fmt=R4,
                                    outliers=True),
    "r4_ragged_b3": S.tiny_shape(B=3, T=4, Hq=12, Hkv=2, D=256, lens=(4, 65, 300), src=S.SRC_BF16, fmt=R4,
                                 outliers=True),
    "r4_rows32_d128": S.tiny_shape(B=2, T=8, Hq=8, Hkv=2, D=128, lens=(513, 70), src=S.SRC_BF16, fmt=R4,
                                   outliers=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_rk4v4_small_shapes(K, name):
    w = S.make(SMALL[name], seed=S.seed_of("tiny") + 800 + list(SMALL).index(name))
    check(K, w, chunk=100)


@pytest.mark.parametrize("name", ["r4_t4_d256_bf16", "r4_rows32_d128"])
def test_rk4v4_fused_step(K, name):
    _fused_check(K, S.make(SMALL[name], seed=S.seed_of("tiny") + 850 + list(SMALL).index(name)))


def test_rk4v4_prefill(K):
    w = S.make(S.tiny_shape(B=2, T=100, Hq=24, Hkv=4, D=256, lens=(300, 180), src=S.SRC_BF16, fmt=R4,
                            outliers=True), seed=S.seed_of("tiny") + 880)
    check(K, w, chunk=100, prefill=True)


def test_rk4v4_mtp128k_sampled(K):
    w = S.make("mtp128k_rk4v4")
    check(K, w, rows=_sample_rows(w, 2), chunk=65536)

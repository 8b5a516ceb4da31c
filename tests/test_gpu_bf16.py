"""Parity of the BF16 reference format (bfloat16 elements, no scales) on the HIP path
with the CPU oracle, through the C ABI: pools byte for byte after appends through both
append kernels, attention (bf16 matrix-core products straight from the pool) within
2e-3 of the oracle's fp64 result for decode, the fused step, prefill and the 128K T=4
workload.
"""
import pytest

import kvq_synth as S
from tests.test_gpu_parity import K, _fused_check, _sample_rows, check  # noqa: F401

pytestmark = pytest.mark.gpu

BF = S.FMT_BF16
SMALL = {
    "bf_t1_d128_f32": S.tiny_shape(B=1, T=1, Hq=8, Hkv=1, D=128, lens=(2048,), src=S.SRC_F32, fmt=BF),
    "bf_t4_d256_bf16": S.tiny_shape(B=1, T=4, Hq=24, Hkv=4, D=256, lens=(777,), src=S.SRC_BF16, fmt=BF,
                                    outliers=True),
    "bf_ragged_b3": S.tiny_shape(B=3, T=4, Hq=12, Hkv=2, D=256, lens=(4, 65, 300), src=S.SRC_BF16, fmt=BF,
                                 outliers=True),
    "bf_rows32_d128_f32": S.tiny_shape(B=2, T=8, Hq=8, Hkv=2, D=128, lens=(513, 70), src=S.SRC_F32, fmt=BF,
                                       outliers=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_bf16_small_shapes(K, name):
    w = S.make(SMALL[name], seed=S.seed_of("tiny") + 900 + list(SMALL).index(name))
    check(K, w, chunk=100)


@pytest.mark.parametrize("name", ["bf_t4_d256_bf16", "bf_rows32_d128_f32"])
def test_bf16_fused_step(K, name):
    _fused_check(K, S.make(SMALL[name], seed=S.seed_of("tiny") + 950 + list(SMALL).index(name)))


def test_bf16_prefill(K):
    w = S.make(S.tiny_shape(B=2, T=100, Hq=24, Hkv=4, D=256, lens=(300, 180), src=S.SRC_BF16, fmt=BF,
                            outliers=True), seed=S.seed_of("tiny") + 980)
    check(K, w, chunk=100, prefill=True)


def test_bf16_mtp128k_sampled(K):
    w = S.make("mtp128k_bf16")
    check(K, w, rows=_sample_rows(w, 2), chunk=65536)

"""paged_decode_attn_noalloc (the library's fixed scratch in place of a workspace) through the
C ABI: on two calls in a row, the second with a smaller input, its output equals
paged_decode_attn's with a caller workspace bit for bit (the same kernels), and both are
within the 2e-3 bar of the fp64 oracle."""
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


def test_noalloc_matches_workspace_call_twice(K):
    shapes = [S.tiny_shape(B=2, T=4, Hq=24, Hkv=4, D=256, lens=(20000, 7000), src=S.SRC_BF16, outliers=True),
              S.tiny_shape(B=1, T=1, Hq=8, Hkv=2, D=128, lens=(3000,), src=S.SRC_F32)]
    for i, shp in enumerate(shapes):
        w = S.make(shp, seed=500 + i)
        s = w.shape
        say(f"[noalloc] call {i}: B={s.B} T={s.T} Hq={s.Hq} Hkv={s.Hkv} D={s.D} lens={s.lens}")
        need = K.workspace_bytes(s.B, s.T, s.Hq, s.Hkv, s.D, w.max_seq_len)
        assert 0 < need <= K.noalloc_max_bytes()
        cache = H.new_cache(K, w, DEV)
        bt = H.fill_gpu(K, w, cache, DEV)
        ref = H.run_attn(K, w, cache, bt, DEV)
        q = H.src_tensor(w.q, s.src, DEV)
        sl = torch.from_numpy(w.seq_lens).to(DEV)
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV)
        K.paged_decode_attn_noalloc(cache, q, bt, sl, w.max_seq_len, w.softmax_scale, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        pool = H.oracle_pool(O, w)
        exp = H.oracle_attn(pool, w)
        err = float(np.abs(out.cpu().numpy().reshape(exp.shape) - exp).max())
        say(f"[noalloc] call {i}: equal to the workspace call; max-abs err vs oracle {err:.3e}")
        assert err <= TOL


def test_noalloc_refuses_oversize_shape(K):
    q = torch.zeros((8, 4, 32, 256), dtype=torch.bfloat16, device=DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    bt = torch.zeros((8, 1 << 15), dtype=torch.int32, device=DEV)
    sl = torch.full((8,), 1 << 21, dtype=torch.int32, device=DEV)
    big = K.Cache(S.FMT_INT8_G64, 4, 4, 256, device=DEV)
    with pytest.raises(K.KvqError) as e:
        K.paged_decode_attn_noalloc(big, q, bt, sl, 1 << 21, 0.0625, out)
    assert e.value.status == -3

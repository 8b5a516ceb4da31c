"""The C-ABI library without a GPU: it loads, exports every declared call, and
every invalid argument returns its documented status before anything runs."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def K():
    import paged_attention_quantized_kv_amd as K
    return K


def _declared():
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported(K):
    names = _declared()
    assert {"kv_append_quant", "paged_decode_attn", "paged_decode_attn_workspace_bytes",
            "kvq_status_string", "paged_decode_attn_noalloc", "kvq_hbm_read_probe"} <= set(names)
    raw = C.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(K):
    for s in (0, -1, -2, -3, -4, -5):
        assert K.status_string(s).startswith("KVQ_")
    assert K.status_string(-99) == "KVQ_ERR_UNKNOWN"


def _desc(K, fmt=0, D=256, H=4, nblk=16, block=64, k=0x1000):
    return K.CacheDesc(fmt, nblk, block, H, D, 0, k, 0x2000, 0x3000, 0x4000)


def _append(K, d, B=1, n=4, dtype=1, kn=0x5000, vn=0x6000, bt=0x7000, mb=4, sp=0x8000):
    return K.lib.kv_append_quant(C.byref(d), C.c_void_p(kn), C.c_void_p(vn), dtype, B, n, C.c_void_p(bt), mb,
                                 C.c_void_p(sp), None)


def _attn(K, d, q=0x5000, qdt=1, B=1, T=4, Hq=24, bt=0x7000, mb=4, sl=0x8000, L=256, scale=0.0625,
          out=0x9000, ws=0xA000, wsb=1 << 30, fn="paged_decode_attn"):
    return getattr(K.lib, fn)(C.byref(d), C.c_void_p(q), qdt, B, T, Hq, C.c_void_p(bt), mb, C.c_void_p(sl), L, scale,
                              C.c_void_p(out), C.c_void_p(ws), wsb, None)


def test_append_validation(K):
    E = dict(inv=-1, uns=-2, cap=-4, launch=-5)
    assert K.lib.kv_append_quant(None, None, None, 1, 1, 1, None, 1, None, None) == E["inv"]
    assert _append(K, _desc(K, fmt=5)) == E["inv"]
    assert _append(K, _desc(K, fmt=-1)) == E["inv"]
    assert _append(K, _desc(K, fmt=3)) == E["launch"]  # rk4v4
    assert _append(K, _desc(K, fmt=2)) == E["launch"]  # rk8v4: valid, reaches the runtime
    assert _append(K, _desc(K, D=192)) == E["uns"]
    assert _append(K, _desc(K, block=32)) == E["uns"]
    assert _append(K, _desc(K, H=0)) == E["inv"]
    assert _append(K, _desc(K, k=0x1004)) == E["inv"]  # misaligned pool
    assert _append(K, _desc(K), dtype=7) == E["inv"]
    assert _append(K, _desc(K), kn=0x5008) == E["inv"]
    assert _append(K, _desc(K), bt=0) == E["inv"]
    assert _append(K, _desc(K), sp=0x8002) == E["inv"]
    assert _append(K, _desc(K), B=0) == E["inv"]
    assert _append(K, _desc(K), n=-1) == E["inv"]
    assert _append(K, _desc(K), n=4 * 64 + 1, mb=4) == E["cap"]
    assert _append(K, _desc(K), n=0) == 0  # no-op, nothing launched
    assert _append(K, _desc(K), B=2000) == E["uns"]
    assert _append(K, _desc(K)) == E["launch"]  # valid: reaches the runtime, which has no device here


@pytest.mark.parametrize("fn", ["paged_decode_attn", "paged_decode_attn_split", "paged_decode_attn_merge"])
def test_attention_validation(K, fn):
    d = _desc(K)
    assert _attn(K, d, qdt=5, fn=fn) == -1
    assert _attn(K, d, q=0x5001, fn=fn) == -1
    assert _attn(K, d, out=0, fn=fn) == -1
    assert _attn(K, d, ws=0xA008, fn=fn) == -1
    assert _attn(K, d, sl=0x8001, fn=fn) == -1
    assert _attn(K, d, scale=float("nan"), fn=fn) == -1
    assert _attn(K, d, Hq=25, fn=fn) == -2  # not a multiple of Hkv
    assert _attn(K, d, T=9, fn=fn) == -2
    assert _attn(K, d, T=8, Hq=32, fn=fn) == -2  # 8 x 8 rows > 32
    assert _attn(K, d, B=0, fn=fn) == -1
    assert _attn(K, d, L=3, T=4, fn=fn) == -1  # fewer keys than query rows
    assert _attn(K, d, L=257, mb=4, fn=fn) == -4
    assert _attn(K, d, wsb=16, fn=fn) == -3
    assert _attn(K, _desc(K, D=64), fn=fn) == -2
    assert _attn(K, d, fn=fn) == -5


def test_workspace_and_chunking_are_pure_functions_of_the_shape(K):
    ws = K.workspace_bytes(1, 4, 24, 4, 256, 131072)
    assert ws == K.workspace_bytes(1, 4, 24, 4, 256, 131072) > 0
    n, tps = K.num_splits(1, 4, 24, 4, 256, 131072)
    assert tps % 64 == 0 and n * tps >= 131072 and (n - 1) * tps < 131072
    rows = 4 * 6
    parts = 1 * 4 * n * rows
    assert ws >= parts * 256 * 4 + parts * 2 * 4
    assert K.workspace_bytes(1, 9, 24, 4, 256, 1024) == 0
    assert K.num_splits(1, 9, 24, 4, 256, 1024) == (0, 0)
    # about one workgroup per compute unit at the headline shapes
    for L in (32768, 131072, 262144):
        n, _ = K.num_splits(1, 1, 24, 4, 256, L)
        assert n * 4 == 256


def test_decode_chunk_rule(K):
    # each (sequence, KV head) gets 256 / pairs chunks, at least one, its pages spread evenly
    assert K.num_splits(1, 4, 24, 4, 256, 131072) == (64, 32 * 64)
    assert K.num_splits(1, 1, 8, 1, 256, 262144) == (256, 16 * 64)
    assert K.num_splits(64, 1, 16, 2, 128, 8192) == (2, 64 * 64)   # 128 pairs: 256 workgroups
    assert K.num_splits(48, 1, 24, 4, 256, 4096) == (1, 64 * 64)   # 192 pairs: one chunk each
    # past the 256-page chunk cap: 294 pages as 148 + 146, not 256 + 38
    assert K.num_splits(64, 1, 32, 4, 128, 18768) == (2, 148 * 64)


def test_prefill_chunks_fill_whole_rounds(K):
    # 262,144 tokens, Hq=24 over Hkv=4, D=256: the 128-row prefill kernel's 24 * T / 512
    # row blocks x 4 KV heads take the chunk counts whose workgroups fill whole rounds of
    # 256 (512 rows: 96 units x 8 = 768), and the 4096-row chunk (768 units) one chunk
    for T, chunks in ((512, 8), (1024, 4), (2048, 2)):
        parts = 4 * chunks * T * 6
        ml = (parts * 2 * 4 + 255) // 256 * 256
        assert K.prefill_workspace_bytes(1, T, 24, 4, 256, 262144) == ml + parts * 256 * 4, T
    assert K.prefill_workspace_bytes(1, 4096, 24, 4, 256, 262144) == 256


def test_check_tables_validation(K):
    d = _desc(K)

    def chk(d=d, B=1, T=4, bt=0x7000, mb=4, sl=0x8000, L=256, res=0x9000):
        return K.lib.kvq_check_tables(C.byref(d), B, T, C.c_void_p(bt), mb, C.c_void_p(sl), L, C.c_void_p(res), None)

    assert chk(B=0) == -1
    assert chk(T=0) == -1
    assert chk(bt=0) == -1
    assert chk(sl=0x8002) == -1
    assert chk(res=0) == -1
    assert chk(L=257) == -4
    assert chk(d=_desc(K, D=192)) == -2
    assert chk() == -5  # valid: reaches the runtime, which has no device here


def test_prefill_validation(K):
    d = _desc(K)
    fn = "paged_prefill_attn"
    assert _attn(K, d, qdt=5, fn=fn) == -1
    assert _attn(K, d, q=0x5001, fn=fn) == -1
    assert _attn(K, d, out=0, fn=fn) == -1
    assert _attn(K, d, ws=0, fn=fn) == -1
    assert _attn(K, d, sl=0x8001, fn=fn) == -1
    assert _attn(K, d, scale=float("inf"), fn=fn) == -1
    assert _attn(K, d, Hq=25, fn=fn) == -2
    assert _attn(K, d, B=0, fn=fn) == -1
    assert _attn(K, d, T=0, fn=fn) == -1
    assert _attn(K, d, L=99, T=100, fn=fn) == -1  # fewer keys than query rows
    assert _attn(K, d, L=257, mb=4, fn=fn) == -4
    assert _attn(K, d, wsb=16, T=100, Hq=8, L=256, fn=fn) == -3
    assert _attn(K, _desc(K, D=64), fn=fn) == -2
    assert _attn(K, d, B=1025, fn=fn) == -2
    # row blocks (128 rows for INT8 with bf16 queries) x KV heads beyond the grid's y limit
    assert _attn(K, d, T=400000, Hq=24, L=400000, mb=6250, fn=fn) == -2
    assert _attn(K, d, T=200000, Hq=24, L=200000, mb=3125, qdt=0, fn=fn) == -2  # fp32 queries: 64-row blocks
    # any T, and T x group beyond the decode limit: valid, reaches the runtime (no device here)
    assert _attn(K, d, T=9, fn=fn) == -5
    assert _attn(K, d, T=4096, Hq=24, L=4096, mb=64, fn=fn) == -5
    assert _attn(K, d, T=8, Hq=32, fn=fn) == -5


def test_prefill_workspace(K):
    # 4096-row chunk at 262,144 tokens: 384 row blocks x 4 KV heads fill the chip with one
    # chunk each, written directly (the workspace is the minimum 256 bytes)
    assert K.prefill_workspace_bytes(1, 4096, 24, 4, 256, 262144) == 256
    # 100 rows x group 4 = 400 rows (7 blocks) x 2 KV heads: chunks of 2 pages over 5 pages
    parts = 1 * 2 * 3 * 400
    ml = (parts * 2 * 4 + 255) // 256 * 256
    assert K.prefill_workspace_bytes(1, 100, 8, 2, 128, 300) == ml + parts * 128 * 4
    assert K.prefill_workspace_bytes(1, 100, 8, 2, 128, 99) == 0  # fewer keys than rows
    assert K.prefill_workspace_bytes(1, 4, 24, 4, 192, 4096) == 0


@pytest.mark.parametrize("fmt", [2, 3, 4])
def test_rk_and_bf16_formats_are_accepted_by_every_attention_call(K, fmt):
    d = _desc(K, fmt=fmt)
    for fn in ("paged_decode_attn", "paged_decode_attn_split", "paged_decode_attn_merge", "paged_prefill_attn"):
        assert _attn(K, d, fn=fn) == -5  # valid: reaches the runtime, which has no device here
    assert _attn(K, _desc(K, fmt=fmt, D=64)) == -2


def test_bf16_pool_needs_no_scales(K):
    d = K.CacheDesc(4, 16, 64, 4, 256, 0, 0x1000, 0x2000, 0, 0)
    assert _attn(K, d) == -5  # valid: reaches the runtime, which has no device here
    d = K.CacheDesc(0, 16, 64, 4, 256, 0, 0x1000, 0x2000, 0, 0)
    assert _attn(K, d) == -1  # the INT8 pool does


def test_noalloc_validation(K):
    """The allocation-free call: its scratch size is fixed, shapes whose workspace exceeds it
    are refused with KVQ_ERR_WORKSPACE before the device is touched, a null cache is invalid,
    and a valid call with no GPU reaches the runtime (KVQ_ERR_LAUNCH)."""
    cap = K.noalloc_max_bytes()
    assert cap == 16 << 20
    f = K.lib.paged_decode_attn_noalloc

    def call(d, B=1, T=4, Hq=24, L=131072):
        return f(C.byref(d) if d is not None else None, C.c_void_p(0x5000), 1, B, T, Hq, C.c_void_p(0x7000),
                 (L + 63) // 64, C.c_void_p(0x8000), L, 0.0625, C.c_void_p(0x9000), None)
    d = _desc(K)
    assert K.workspace_bytes(1, 4, 24, 4, 256, 131072) <= cap  # the headline shape fits
    big = next(L for L in (1 << 20, 1 << 21, 1 << 22) if K.workspace_bytes(8, 4, 32, 4, 256, L) > cap)
    assert call(d, B=8, T=4, Hq=32, L=big) == -3
    assert call(None) == -1
    assert call(d) == -5  # valid shape, no device here


def test_page_bytes_match_the_format_table(K):
    """kvq_page_bytes against the pages' bytes-per-token table (NInfer-3090 README, "Choosing
    a KV format"; 16 layers x 4 KV heads at head_dim 256): a page is 64 tokens of one KV head
    of one layer.  FP8 follows this library's layout (fp32 row scales: 8 bytes per token per
    head where the table's total implies 4), and 0 marks an unsupported format or head_dim."""
    table = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "kv_format_table.txt")):
        f = line.split()
        if f and not line.startswith("#") and f[0] in ("bf16", "int8", "fp8", "rk8v4", "rk4v4"):
            table[f[0]] = int(f[1])
    per_head_layer = {k: v // (16 * 4) for k, v in table.items()}
    assert K.page_bytes(K.INT8_G64, 256) == 64 * per_head_layer["int8"]
    assert K.page_bytes(K.RK8V4, 256) == 64 * per_head_layer["rk8v4"]
    assert K.page_bytes(K.RK4V4, 256) == 64 * per_head_layer["rk4v4"]
    assert K.page_bytes(K.BF16_KV, 256) == 64 * per_head_layer["bf16"]
    assert K.page_bytes(K.FP8_E4M3_ROW, 256) == 64 * (2 * 256 + 2 * 4)
    assert K.page_bytes(K.INT8_G64, 128) == 64 * (2 * 128 + 2 * 2 * 2)
    assert K.page_bytes(K.INT8_G64, 64) == 0 and K.page_bytes(7, 256) == 0


def test_capacity_check_states_the_exact_deficit(K):
    """A pool of 100 blocks (4 KV heads, INT8, head_dim 256) and a 40-entry block table."""
    d = _desc(K, fmt=K.INT8_G64, D=256, H=4, nblk=100)
    page = K.page_bytes(K.INT8_G64, 256)
    assert K.capacity_check(d, [64 * 40, 64 * 60], 60) == 0            # 100 blocks exactly
    assert K.capacity_check(d, [64 * 40, 64 * 60 + 1], 61) == 4 * page  # one block more: 4 pages
    assert K.capacity_check(d, [64 * 40, 64 * 60], 40) == 20 * 2 * 4   # rows 20 entries short
    assert K.capacity_check(d, [0, 1, 63, 64], 1) == 0
    # a 41-page sequence: the pool fits (41 + 40 blocks) but every table row needs one more entry
    assert K.capacity_check(d, [64 * 41, 64 * 40], 40) == 2 * 4
    # both short: 3 blocks and 5 table entries per row for 3 sequences
    assert K.capacity_check(d, [64 * 45, 64 * 29, 64 * 29], 40) == 3 * 4 * page + 5 * 3 * 4
    out = C.c_int64(-1)
    lens = (C.c_int32 * 2)(64 * 40, 64 * 61)
    assert K.lib.kvq_capacity_check(C.byref(d), 2, lens, 61, C.byref(out)) == -4 and out.value == 4 * page
    assert K.lib.kvq_capacity_check(C.byref(d), 2, lens, 40, None) == -1
    assert K.lib.kvq_capacity_check(C.byref(d), 0, lens, 40, C.byref(out)) == -1 and out.value == 0
    bad = (C.c_int32 * 1)(-1)
    assert K.lib.kvq_capacity_check(C.byref(d), 1, bad, 40, C.byref(out)) == -1
    big = (C.c_int32 * 1)((1 << 30) + 1)
    assert K.lib.kvq_capacity_check(C.byref(d), 1, big, 40, C.byref(out)) == -2
    assert K.lib.kvq_capacity_check(C.byref(_desc(K, fmt=9)), 1, lens, 40, C.byref(out)) == -1

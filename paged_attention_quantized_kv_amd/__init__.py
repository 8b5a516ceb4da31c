"""Python binding of libkvq.so, the gfx950 C-ABI library (include/kvq.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and a negative status raises KvqError.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback, and importing this package fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY names another build of the same sources (e.g. for A/B timing of two builds)
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(_HERE, "libkvq.so")

INT8_G64 = 0
FP8_E4M3_ROW = 1
RK8V4 = 2
RK4V4 = 3
BF16_KV = 4
F32 = 0
BF16 = 1
PAGE = 64

_EXPORTS = ("kv_append_quant", "paged_decode_attn", "paged_decode_attn_split", "paged_decode_attn_merge",
            "paged_decode_step", "paged_decode_attn_workspace_bytes", "paged_decode_attn_num_splits",
            "paged_prefill_attn", "paged_prefill_attn_workspace_bytes", "kvq_check_tables", "kvq_status_string",
            "paged_decode_attn_noalloc", "paged_decode_attn_noalloc_max_bytes", "kvq_page_bytes",
            "kvq_capacity_check")


class KvqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class CacheDesc(C.Structure):
    _fields_ = [("format", C.c_int32), ("num_blocks", C.c_int32), ("block_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("reserved", C.c_int32),
                ("k_codes", C.c_void_p), ("v_codes", C.c_void_p), ("k_scales", C.c_void_p), ("v_scales", C.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with paged_attention_quantized_kv_amd/build.py "
                          "(or __graft_entry__.build()); there is no fallback path")
    L = C.CDLL(LIB_PATH)
    vp, i32 = C.c_void_p, C.c_int32
    P = C.POINTER(CacheDesc)
    L.kv_append_quant.argtypes = [P, vp, vp, i32, i32, i32, vp, i32, vp, vp]
    L.kv_append_quant.restype = C.c_int
    attn = [P, vp, i32, i32, i32, i32, vp, i32, vp, i32, C.c_float, vp, vp, C.c_size_t, vp]
    for name in ("paged_decode_attn", "paged_decode_attn_split", "paged_decode_attn_merge", "paged_prefill_attn"):
        getattr(L, name).argtypes = attn
        getattr(L, name).restype = C.c_int
    L.kvq_hbm_read_probe.argtypes = [vp, C.c_size_t, i32, vp, vp]
    L.kvq_hbm_read_probe.restype = C.c_int
    L.paged_decode_attn_noalloc.argtypes = attn[:12] + [vp]
    L.paged_decode_attn_noalloc.restype = C.c_int
    L.paged_decode_attn_noalloc_max_bytes.argtypes = []
    L.paged_decode_attn_noalloc_max_bytes.restype = C.c_size_t
    L.paged_decode_step.argtypes = [P, vp, vp, vp, i32, i32, i32, i32, vp, i32, vp, i32, C.c_float, vp, vp,
                                    C.c_size_t, vp]
    L.paged_decode_step.restype = C.c_int
    L.paged_decode_attn_workspace_bytes.argtypes = [i32] * 6
    L.paged_decode_attn_workspace_bytes.restype = C.c_size_t
    L.paged_prefill_attn_workspace_bytes.argtypes = [i32] * 6
    L.paged_prefill_attn_workspace_bytes.restype = C.c_size_t
    L.paged_decode_attn_num_splits.argtypes = [i32] * 6 + [C.POINTER(i32)]
    L.paged_decode_attn_num_splits.restype = i32
    L.kvq_check_tables.argtypes = [P, i32, i32, vp, i32, vp, i32, vp, vp]
    L.kvq_check_tables.restype = C.c_int
    L.kvq_status_string.argtypes = [C.c_int]
    L.kvq_status_string.restype = C.c_char_p
    L.kvq_page_bytes.argtypes = [i32, i32]
    L.kvq_page_bytes.restype = C.c_size_t
    L.kvq_capacity_check.argtypes = [P, i32, vp, i32, C.POINTER(C.c_int64)]
    L.kvq_capacity_check.restype = C.c_int
    return L


lib = _load()


def page_bytes(fmt: int, head_dim: int) -> int:
    """Pool bytes one page (64 slots of one KV head) takes in the format (kvq_page_bytes)."""
    return int(lib.kvq_page_bytes(fmt, head_dim))


def capacity_check(cache, context_lens, max_blocks_per_seq: int) -> int:
    """Host-side capacity plan (kvq_capacity_check): the bytes the pool and block table lack
    for sequences reaching context_lens (0 when they fit).  `cache` may be a Cache or a
    CacheDesc (only its shape fields are read)."""
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    deficit = C.c_int64(0)
    desc = cache.desc if isinstance(cache, Cache) else C.byref(cache)
    rc = lib.kvq_capacity_check(desc, int(lens.size), lens.ctypes.data_as(C.c_void_p), int(max_blocks_per_seq),
                                C.byref(deficit))
    if rc not in (0, -4):
        raise KvqError(rc, status_string(rc))
    return int(deficit.value)


def status_string(status: int) -> str:
    return lib.kvq_status_string(status).decode()


def _check(status: int) -> None:
    if status != 0:
        raise KvqError(status, status_string(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32")


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor) -> C.c_void_p:
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return C.c_void_p(t.data_ptr())


class Cache:
    """A page pool: four device tensors in the layout of kvq.h, plus its shape."""

    def __init__(self, fmt: int, num_blocks: int, num_kv_heads: int, head_dim: int, device="cuda",
                 k_codes=None, v_codes=None, k_scales=None, v_scales=None):
        self.format, self.num_blocks, self.num_kv_heads, self.head_dim = fmt, num_blocks, num_kv_heads, head_dim
        n = num_blocks * num_kv_heads * PAGE
        if k_codes is None and fmt == BF16_KV:  # bf16 elements, no scales (small placeholders)
            k_codes = torch.empty(n * head_dim, dtype=torch.bfloat16, device=device)
            v_codes = torch.empty(n * head_dim, dtype=torch.bfloat16, device=device)
            k_scales = torch.zeros(8, dtype=torch.float16, device=device)
            v_scales = torch.zeros(8, dtype=torch.float16, device=device)
        elif k_codes is None:
            k_codes = torch.empty(n * head_dim // (2 if fmt == RK4V4 else 1), dtype=torch.uint8, device=device)
            v_codes = torch.empty(n * head_dim // (2 if fmt in (RK8V4, RK4V4) else 1), dtype=torch.uint8, device=device)
            if fmt in (RK8V4, RK4V4):  # fp16 group-64 key scales; 4-bit values with one fp16 scale per 32 dims
                k_scales = torch.empty(n * (head_dim // 64), dtype=torch.float16, device=device)
                v_scales = torch.empty(n * (head_dim // 32), dtype=torch.float16, device=device)
            elif fmt == INT8_G64:
                k_scales = torch.empty(n * (head_dim // 64), dtype=torch.float16, device=device)
                v_scales = torch.empty(n * (head_dim // 64), dtype=torch.float16, device=device)
            else:
                k_scales = torch.empty(n, dtype=torch.float32, device=device)
                v_scales = torch.empty(n, dtype=torch.float32, device=device)
        self.k_codes, self.v_codes, self.k_scales, self.v_scales = k_codes, v_codes, k_scales, v_scales
        self._desc = CacheDesc(fmt, num_blocks, PAGE, num_kv_heads, head_dim, 0, k_codes.data_ptr(),
                               v_codes.data_ptr(), k_scales.data_ptr(), v_scales.data_ptr())

    @property
    def desc(self):
        return C.byref(self._desc)

    def tensors(self):
        return self.k_codes, self.v_codes, self.k_scales, self.v_scales

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.tensors())


def _check_table(t: torch.Tensor, B: int, name: str, ndim: int) -> None:
    if t.dtype != torch.int32 or t.dim() != ndim or t.shape[0] != B or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor with {B} rows")


def _check_rows(x: torch.Tensor, cache: Cache, name: str) -> None:
    if x.dim() != 4 or x.shape[2] != cache.num_kv_heads or x.shape[3] != cache.head_dim:
        raise ValueError(f"{name} must be [B, n, {cache.num_kv_heads}, {cache.head_dim}]")


def kv_append_quant(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, block_table: torch.Tensor,
                    start_pos: torch.Tensor, stream=None) -> None:
    """k_new, v_new: [B, n_new, Hkv, D] bf16|fp32; block_table [B, max_blocks] int32; start_pos [B] int32."""
    if k_new.dtype != v_new.dtype or k_new.shape != v_new.shape or k_new.dim() != 4:
        raise ValueError("k_new and v_new must both be [B, n_new, Hkv, D] of one dtype")
    _check_rows(k_new, cache, "k_new")
    B, n_new = k_new.shape[0], k_new.shape[1]
    _check_table(block_table, B, "block_table", 2)
    _check_table(start_pos, B, "start_pos", 1)
    _check(lib.kv_append_quant(cache.desc, _ptr(k_new), _ptr(v_new), _dtype_code(k_new), B, n_new,
                               _ptr(block_table), block_table.shape[1], _ptr(start_pos), _stream(stream)))


def workspace_bytes(num_seqs: int, T: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    max_seq_len: int) -> int:
    return int(lib.paged_decode_attn_workspace_bytes(num_seqs, T, num_q_heads, num_kv_heads, head_dim, max_seq_len))


def num_splits(num_seqs: int, T: int, num_q_heads: int, num_kv_heads: int, head_dim: int, max_seq_len: int):
    tps = C.c_int32(0)
    n = lib.paged_decode_attn_num_splits(num_seqs, T, num_q_heads, num_kv_heads, head_dim, max_seq_len, C.byref(tps))
    return int(n), int(tps.value)


def alloc_workspace(cache: Cache, num_seqs: int, T: int, num_q_heads: int, max_seq_len: int, device="cuda"):
    n = workspace_bytes(num_seqs, T, num_q_heads, cache.num_kv_heads, cache.head_dim, max_seq_len)
    if n == 0:
        raise KvqError(-2, "unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill_workspace_bytes(num_seqs: int, T: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                            max_seq_len: int) -> int:
    return int(lib.paged_prefill_attn_workspace_bytes(num_seqs, T, num_q_heads, num_kv_heads, head_dim, max_seq_len))


def alloc_prefill_workspace(cache: Cache, num_seqs: int, T: int, num_q_heads: int, max_seq_len: int, device="cuda"):
    n = prefill_workspace_bytes(num_seqs, T, num_q_heads, cache.num_kv_heads, cache.head_dim, max_seq_len)
    if n == 0:
        raise KvqError(-2, "unsupported shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _check_attn(cache, q, block_table, seq_lens, out, workspace):
    if q.dim() != 4 or q.shape[3] != cache.head_dim:
        raise ValueError(f"q must be [B, T, Hq, {cache.head_dim}]")
    B = q.shape[0]
    _check_table(block_table, B, "block_table", 2)
    _check_table(seq_lens, B, "seq_lens", 1)
    if out.dtype != torch.float32 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor with the shape of q")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _attn(fn, cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out, workspace, stream):
    _check_attn(cache, q, block_table, seq_lens, out, workspace)
    B, T, Hq = q.shape[0], q.shape[1], q.shape[2]
    _check(fn(cache.desc, _ptr(q), _dtype_code(q), B, T, Hq, _ptr(block_table), block_table.shape[1],
              _ptr(seq_lens), int(max_seq_len), float(softmax_scale), _ptr(out), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def paged_decode_attn(cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out, workspace, stream=None):
    """out[B, T, Hq, D] (fp32) = softmax(q k^T * softmax_scale) v over the paged cache."""
    return _attn(lib.paged_decode_attn, cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out, workspace,
                 stream)


def paged_decode_attn_noalloc(cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out, stream=None):
    """paged_decode_attn without a workspace: the library's fixed device array takes its place
    (nothing is allocated; calls that overlap on one GPU race)."""
    _check_attn(cache, q, block_table, seq_lens, out, out)
    B, T, Hq = q.shape[0], q.shape[1], q.shape[2]
    _check(lib.paged_decode_attn_noalloc(cache.desc, _ptr(q), _dtype_code(q), B, T, Hq, _ptr(block_table),
                                         block_table.shape[1], _ptr(seq_lens), int(max_seq_len), float(softmax_scale),
                                         _ptr(out), _stream(stream)))
    return out


def hbm_read_probe(buf, workgroups, sink, stream=None):
    """Read the whole of `buf` once with the library's streaming-read probe kernel."""
    rc = lib.kvq_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), int(workgroups), _ptr(sink),
                                _stream(stream))
    if rc != 0:
        raise KvqError(rc, "kvq_hbm_read_probe: invalid arguments or launch refused")


def noalloc_max_bytes() -> int:
    return int(lib.paged_decode_attn_noalloc_max_bytes())


def paged_decode_attn_split(cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out, workspace, stream=None):
    return _attn(lib.paged_decode_attn_split, cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out,
                 workspace, stream)


def paged_decode_attn_merge(cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out, workspace, stream=None):
    return _attn(lib.paged_decode_attn_merge, cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out,
                 workspace, stream)


def paged_prefill_attn(cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out, workspace, stream=None):
    """Attention of a prefill chunk: q [B, T, Hq, D] with any T, the chunk's rows already
    appended at seq_lens - T .. seq_lens - 1; row t sees keys 0 .. seq_lens - T + t."""
    return _attn(lib.paged_prefill_attn, cache, q, block_table, seq_lens, max_seq_len, softmax_scale, out, workspace,
                 stream)


def paged_decode_step(cache, k_new, v_new, q, block_table, seq_lens, max_seq_len, softmax_scale, out, workspace,
                      stream=None):
    """Append the T new rows of each sequence (at seq_lens - T) and attend, in one launch.
    k_new, v_new: [B, T, Hkv, D] with the dtype of q."""
    _check_attn(cache, q, block_table, seq_lens, out, workspace)
    if k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must have one shape")
    _check_rows(k_new, cache, "k_new")
    if k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise TypeError("the new rows and the queries must share one dtype")
    B, T, Hq = q.shape[0], q.shape[1], q.shape[2]
    if k_new.shape[0] != B or k_new.shape[1] != T:
        raise ValueError("k_new must hold T rows per sequence")
    _check(lib.paged_decode_step(cache.desc, _ptr(k_new), _ptr(v_new), _ptr(q), _dtype_code(q), B, T, Hq,
                                 _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(max_seq_len),
                                 float(softmax_scale), _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def check_tables(cache, T, block_table, seq_lens, max_seq_len, stream=None):
    """Debug check of the device tables: returns a device int32 tensor [bad lengths,
    bad block ids among the used pages] (read it after the stream is synchronized)."""
    B = seq_lens.shape[0]
    _check_table(block_table, B, "block_table", 2)
    _check_table(seq_lens, B, "seq_lens", 1)
    result = torch.empty(2, dtype=torch.int32, device=seq_lens.device)
    _check(lib.kvq_check_tables(cache.desc, B, int(T), _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
                                int(max_seq_len), _ptr(result), _stream(stream)))
    return result

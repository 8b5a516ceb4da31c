"""ctypes wrapper of the plain C oracle (kvq_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The HIP library never imports it and shares no
code with it.

Every function returns plain numpy arrays; inputs are numpy arrays (bf16 data
travels as its raw uint16 bit patterns so the oracle widens it itself).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq_oracle.so")
SRC_PATH = os.path.join(_HERE, "kvq_oracle.c")
# the pin suite's mutation check loads deliberately broken builds of the oracle through
# this variable (tests/test_oracle_mutations.py); unset, the oracle is the one above
_LIB_OVERRIDE = os.environ.get("KVQ_ORACLE_LIB")

FMT_INT8_G64 = 0
FMT_FP8_ROW = 1
FMT_RK8V4 = 2
FMT_RK4V4 = 3
FMT_BF16 = 4
SRC_F32 = 0
SRC_BF16 = 1


def build(force: bool = False) -> str:
    """Compile kvq_oracle.c with gcc into oracle/libkvq_oracle.so."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               "-fPIC", "-shared", "-o", LIB_PATH, SRC_PATH, "-lm"]
        subprocess.run(cmd, check=True)
    return LIB_PATH


class _Pool(C.Structure):
    _fields_ = [("format", C.c_int32), ("num_blocks", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("k_codes", C.c_void_p), ("v_codes", C.c_void_p),
                ("k_scales", C.c_void_p), ("v_scales", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = C.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = C.CDLL(LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int
        for name in ("orc_f32_to_f16_n", "orc_f16_to_f32_n", "orc_bf16_to_f32_n",
                     "orc_f32_to_e4m3fn_n", "orc_e4m3fn_to_f32_n", "orc_f32_to_bf16_n"):
            getattr(L, name).argtypes = [vp, vp, i64]
            getattr(L, name).restype = None
        L.orc_quant_rows.argtypes = [i32, vp, i64, i32, vp, vp]
        L.orc_quant_rows.restype = None
        L.orc_h64_rotate_n.argtypes = [vp, vp, i64]
        L.orc_h64_rotate_n.restype = None
        L.orc_quant_int4_rows.argtypes = [vp, i64, i32, vp, vp]
        L.orc_quant_int4_rows.restype = None
        L.orc_v4_bit.argtypes = [i32, i32, i32]
        L.orc_v4_bit.restype = i64
        L.orc_k4_bit.argtypes = [i32, i32, i32]
        L.orc_k4_bit.restype = i64
        L.orc_lloyd_max16.argtypes = [vp]
        L.orc_lloyd_max16.restype = None
        L.orc_rk4_codes.argtypes = [vp]
        L.orc_rk4_codes.restype = None
        L.orc_quant_rk4v4_rows.argtypes = [vp, i64, i32, vp, vp]
        L.orc_quant_rk4v4_rows.restype = None
        L.orc_k_byte.argtypes = [i32, i32, i32]
        L.orc_k_byte.restype = i64
        L.orc_v_byte.argtypes = [i32, i32, i32]
        L.orc_v_byte.restype = i64
        L.orc_scale_elem.argtypes = [i32, i32, i32, i32, i32]
        L.orc_scale_elem.restype = i64
        L.orc_append.argtypes = [C.POINTER(_Pool), vp, vp, i32, i32, i32, vp, i32, vp]
        L.orc_append.restype = i32
        L.orc_dequant.argtypes = [C.POINTER(_Pool), i32, i32, i32, i32, i32]
        L.orc_dequant.restype = C.c_double
        L.orc_dense_attn.argtypes = [vp, vp, vp, i32, i32, i32, C.c_double, vp, vp]
        L.orc_dense_attn.restype = i32
        L.orc_paged_attn.argtypes = [C.POINTER(_Pool), vp, i32, i32, i32, i32, vp, i32, vp,
                                     C.c_float, vp, i32, vp]
        L.orc_paged_attn.restype = i32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- conversions
def f32_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16_n(_ptr(x), _ptr(y), x.size)
    return y


def f16_bits_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    y = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32_n(_ptr(h), _ptr(y), h.size)
    return y


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    y = np.empty(b.shape, np.float32)
    lib().orc_bf16_to_f32_n(_ptr(b), _ptr(y), b.size)
    return y


def f32_to_bf16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_bf16_n(_ptr(x), _ptr(y), x.size)
    return y


def f32_to_e4m3fn(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint8)
    lib().orc_f32_to_e4m3fn_n(_ptr(x), _ptr(y), x.size)
    return y


def e4m3fn_to_f32(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    y = np.empty(c.shape, np.float32)
    lib().orc_e4m3fn_to_f32_n(_ptr(c), _ptr(y), c.size)
    return y


# ---------------------------------------------------------------- quantizers
def quant_rows(fmt: int, x) -> tuple[np.ndarray, np.ndarray]:
    """x: float32 [..., D] -> (codes [..., D] (int8 | uint8), scales [..., D/64] uint16 | [...] float32).
    FMT_RK8V4 gives the key encoding (rotated, then INT8 group-64)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    n = x.size // D
    if fmt in (FMT_INT8_G64, FMT_RK8V4):
        codes = np.empty(x.shape, np.int8)
        scales = np.empty(x.shape[:-1] + (D // 64,), np.uint16)
    else:
        codes = np.empty(x.shape, np.uint8)
        scales = np.empty(x.shape[:-1], np.float32)
    lib().orc_quant_rows(fmt, _ptr(x), n, D, _ptr(codes), _ptr(scales))
    return codes, scales


def h64_rotate(x) -> np.ndarray:
    """x: float32 [..., 64*k] -> each 64-element group rotated by the Sylvester Hadamard / 8."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape[-1] % 64 == 0
    y = np.empty(x.shape, np.float32)
    lib().orc_h64_rotate_n(_ptr(x), _ptr(y), x.size // 64)
    return y


def quant_int4_g32(x) -> tuple[np.ndarray, np.ndarray]:
    """rk8v4 values: x float32 [..., D] -> (codes [..., D] int8 in -7..7, scales [..., D/32] uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    n = x.size // D
    codes = np.empty(x.shape, np.int8)
    scales = np.empty(x.shape[:-1] + (D // 32,), np.uint16)
    lib().orc_quant_int4_rows(_ptr(x), n, D, _ptr(codes), _ptr(scales))
    return codes, scales


def lloyd_max16() -> np.ndarray:
    """The 16 Lloyd-Max levels for N(0,1), ascending (the oracle's iteration)."""
    out = np.empty(16, np.float64)
    lib().orc_lloyd_max16(_ptr(out))
    return out


def rk4_codes() -> np.ndarray:
    """The INT8 code of each rk4v4 level."""
    out = np.empty(16, np.int8)
    lib().orc_rk4_codes(_ptr(out))
    return out


def quant_rk4v4_keys(x) -> tuple[np.ndarray, np.ndarray]:
    """rk4v4 keys: x float32 [..., D] -> (level indices [..., D] uint8 0..15, scales [..., D/64] uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    D = x.shape[-1]
    n = x.size // D
    idx = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1] + (D // 64,), np.uint16)
    lib().orc_quant_rk4v4_rows(_ptr(x), n, D, _ptr(idx), _ptr(scales))
    return idx, scales


# ---------------------------------------------------------------- layout
def k_byte(s: int, d: int, D: int) -> int:
    return lib().orc_k_byte(s, d, D)


def v_byte(s: int, d: int, D: int) -> int:
    return lib().orc_v_byte(s, d, D)


def v4_bit(s: int, d: int, D: int) -> int:
    return lib().orc_v4_bit(s, d, D)


def k4_bit(s: int, d: int, D: int) -> int:
    return lib().orc_k4_bit(s, d, D)


def scale_elem(fmt: int, which: int, s: int, g: int, D: int) -> int:
    return lib().orc_scale_elem(fmt, which, s, g, D)


# ---------------------------------------------------------------- pool
class Pool:
    """Host copy of the paged pool in the documented byte layout."""

    def __init__(self, fmt: int, num_blocks: int, num_kv_heads: int, head_dim: int, fill: int = 0):
        self.fmt, self.num_blocks, self.num_kv_heads, self.head_dim = fmt, num_blocks, num_kv_heads, head_dim
        n = num_blocks * num_kv_heads * 64
        if fmt == FMT_BF16:  # two bytes per element, no scales (one-element placeholders)
            self.k_codes = np.full(n * head_dim * 2, fill, np.uint8)
            self.v_codes = np.full(n * head_dim * 2, fill, np.uint8)
            self.k_scales = np.zeros(1, np.uint16)
            self.v_scales = np.zeros(1, np.uint16)
            return
        self.k_codes = np.full(n * head_dim // (2 if fmt == FMT_RK4V4 else 1), fill, np.uint8)
        self.v_codes = np.full(n * head_dim // (2 if fmt in (FMT_RK8V4, FMT_RK4V4) else 1), fill, np.uint8)
        if fmt in (FMT_RK8V4, FMT_RK4V4):
            self.k_scales = np.zeros(n * (head_dim // 64), np.uint16)
            self.v_scales = np.zeros(n * (head_dim // 32), np.uint16)
        elif fmt == FMT_INT8_G64:
            self.k_scales = np.zeros(n * (head_dim // 64), np.uint16)
            self.v_scales = np.zeros(n * (head_dim // 64), np.uint16)
        else:
            self.k_scales = np.zeros(n, np.float32)
            self.v_scales = np.zeros(n, np.float32)

    def _c(self) -> _Pool:
        return _Pool(self.fmt, self.num_blocks, self.num_kv_heads, self.head_dim,
                     self.k_codes.ctypes.data, self.v_codes.ctypes.data,
                     self.k_scales.ctypes.data, self.v_scales.ctypes.data)

    def append(self, k_new, v_new, src_dtype: int, block_table, start_pos) -> None:
        k_new = np.ascontiguousarray(k_new)
        v_new = np.ascontiguousarray(v_new)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        sp = np.ascontiguousarray(start_pos, dtype=np.int32)
        B, n_new = k_new.shape[0], k_new.shape[1]
        pool = self._c()
        rc = lib().orc_append(C.byref(pool), _ptr(k_new), _ptr(v_new), src_dtype, B, n_new,
                              _ptr(bt), bt.shape[1], _ptr(sp))
        if rc != 0:
            raise ValueError("oracle append: position or block id out of range")

    def dequant(self, which: int, block: int, kvh: int, slot: int, d: int) -> float:
        pool = self._c()
        return lib().orc_dequant(C.byref(pool), which, block, kvh, slot, d)

    def paged_attn(self, q, q_dtype: int, T: int, Hq: int, block_table, seq_lens, softmax_scale: float,
                   rows=None) -> np.ndarray:
        q = np.ascontiguousarray(q)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B = bt.shape[0]
        D = self.head_dim
        if rows is None:
            n = B * T * Hq
            rows_p = None
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int32)
            n = rows.size
            rows_p = _ptr(rows)
        out = np.empty((n, D), np.float64)
        pool = self._c()
        rc = lib().orc_paged_attn(C.byref(pool), _ptr(q), q_dtype, B, T, Hq, _ptr(bt), bt.shape[1],
                                  _ptr(sl), C.c_float(softmax_scale), rows_p, n, _ptr(out))
        if rc != 0:
            raise ValueError("oracle paged_attn: bad shape or index")
        return out


def dense_attn(q, k, v, scale: float, last) -> np.ndarray:
    """q [nq, D], k/v [L, D] (float64); query r sees keys 0..last[r]."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    last = np.ascontiguousarray(last, dtype=np.int32)
    nq, D = q.shape
    L = k.shape[0]
    out = np.empty((nq, D), np.float64)
    rc = lib().orc_dense_attn(_ptr(q), _ptr(k), _ptr(v), nq, L, D, float(scale), _ptr(last), _ptr(out))
    if rc != 0:
        raise ValueError("oracle dense_attn: last index out of range")
    return out

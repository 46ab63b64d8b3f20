"""ctypes binding of the plain CPU oracle (``libkvq_oracle.so``).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the product path
(``bit_kv_cache_block_amd``) never does.  The oracle shares no code with the
GPU library (see ``kvq_oracle.h`` for the method, the readings taken where the
pages are silent, and the cache layout written out in words).

Every function takes host numpy arrays and returns numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.cpp")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

F16, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (fp32 steps kept exact: no contraction, no
    fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = C.CDLL(_LIB)
        _declare(_lib)
    return _lib


_p = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64


def _declare(L):
    L.kvq_oracle_f32_to_f16.argtypes = [C.c_float]
    L.kvq_oracle_f32_to_f16.restype = C.c_uint16
    L.kvq_oracle_f16_to_f32.argtypes = [C.c_uint16]
    L.kvq_oracle_f16_to_f32.restype = C.c_float
    L.kvq_oracle_f32_to_bf16.argtypes = [C.c_float]
    L.kvq_oracle_f32_to_bf16.restype = C.c_uint16
    L.kvq_oracle_bf16_to_f32.argtypes = [C.c_uint16]
    L.kvq_oracle_bf16_to_f32.restype = C.c_float
    L.kvq_oracle_block_scale.argtypes = [_i32]
    L.kvq_oracle_block_scale.restype = C.c_float
    L.kvq_oracle_rotate.argtypes = [_p, _p, _i32, _i32]
    L.kvq_oracle_rotate.restype = None
    L.kvq_oracle_quantize.argtypes = [_p, _i32, _p, _p, _p]
    L.kvq_oracle_quantize.restype = None
    L.kvq_oracle_quantize_int8.argtypes = [_p, _i32, _p, _p, _p]
    L.kvq_oracle_quantize_int8.restype = None
    L.kvq_oracle_grid_sse.argtypes = [_p, _i32, _p, C.c_uint16, C.c_uint16, _i32]
    L.kvq_oracle_grid_sse.restype = C.c_int64
    L.kvq_oracle_grid_exponent.argtypes = [C.c_float]
    L.kvq_oracle_grid_exponent.restype = _i32
    L.kvq_oracle_quantize_search.argtypes = [_p, _i32, _p, _p, _p]
    L.kvq_oracle_quantize_search.restype = _i32
    L.kvq_oracle_quantize_hybrid.argtypes = [_p, _i32, _p, _p, _p]
    L.kvq_oracle_quantize_hybrid.restype = _i32
    L.kvq_oracle_append_int4_search.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32, _i64,
                                                _p, _i32]
    L.kvq_oracle_append_int4_search.restype = _i32
    L.kvq_oracle_append_int4g_hybrid.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32,
                                                 _i64, _p, _i32]
    L.kvq_oracle_append_int4g_hybrid.restype = _i32
    L.kvq_oracle_int8_slab_bytes.argtypes = [_i32, _i32]
    L.kvq_oracle_int8_slab_bytes.restype = C.c_size_t
    L.kvq_oracle_append_int8.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32, _i64, _p, _i32]
    L.kvq_oracle_append_int8.restype = _i32
    L.kvq_oracle_int8_read.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p]
    L.kvq_oracle_int8_read.restype = C.c_double
    L.kvq_oracle_decode_int8.argtypes = [_p, _i32, _i32, _i32, _i32, _p, _i32, _i32, _p, _i32, _p,
                                         _i32, C.c_double, _p, _p]
    L.kvq_oracle_decode_int8.restype = _i32
    L.kvq_oracle_int4g_slab_bytes.argtypes = [_i32, _i32, _i32]
    L.kvq_oracle_int4g_slab_bytes.restype = C.c_size_t
    L.kvq_oracle_append_int4g.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32, _i64,
                                          _p, _i32]
    L.kvq_oracle_append_int4g.restype = _i32
    L.kvq_oracle_int4g_read.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _p, _p, _p]
    L.kvq_oracle_int4g_read.restype = C.c_double
    L.kvq_oracle_decode_int4g.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _p, _i32, _i32, _p, _i32,
                                          _p, _i32, C.c_double, _p, _p]
    L.kvq_oracle_decode_int4g.restype = _i32
    L.kvq_oracle_e2m1_encode.argtypes = [C.c_float]
    L.kvq_oracle_e2m1_encode.restype = C.c_uint8
    L.kvq_oracle_e2m1_decode.argtypes = [C.c_uint8]
    L.kvq_oracle_e2m1_decode.restype = C.c_double
    L.kvq_oracle_quantize_mx.argtypes = [_p, _i32, _p, _p]
    L.kvq_oracle_quantize_mx.restype = None
    L.kvq_oracle_mxfp4_slab_bytes.argtypes = [_i32, _i32]
    L.kvq_oracle_mxfp4_slab_bytes.restype = C.c_size_t
    L.kvq_oracle_append_mxfp4.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32, _i64, _p, _i32]
    L.kvq_oracle_append_mxfp4.restype = _i32
    L.kvq_oracle_mxfp4_read.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p]
    L.kvq_oracle_mxfp4_read.restype = C.c_double
    L.kvq_oracle_decode_mxfp4.argtypes = [_p, _i32, _i32, _i32, _i32, _p, _i32, _i32, _p, _i32, _p,
                                          _i32, C.c_double, _p, _p]
    L.kvq_oracle_decode_mxfp4.restype = _i32
    L.kvq_oracle_int4_slab_bytes.argtypes = [_i32, _i32]
    L.kvq_oracle_int4_slab_bytes.restype = C.c_size_t
    L.kvq_oracle_bf16_slab_bytes.argtypes = [_i32, _i32]
    L.kvq_oracle_bf16_slab_bytes.restype = C.c_size_t
    L.kvq_oracle_append_int4.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _p, _p, _i32, _i64, _p, _i32]
    L.kvq_oracle_append_int4.restype = _i32
    L.kvq_oracle_append_bf16.argtypes = [_p, _i32, _i32, _i32, _i32, _p, _p, _i32, _i64, _p, _i32]
    L.kvq_oracle_append_bf16.restype = _i32
    L.kvq_oracle_int4_read.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p]
    L.kvq_oracle_int4_read.restype = C.c_double
    L.kvq_oracle_bf16_read.argtypes = [_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]
    L.kvq_oracle_bf16_read.restype = C.c_double
    L.kvq_oracle_decode_int4.argtypes = [_p, _i32, _i32, _i32, _i32, _p, _i32, _i32, _p, _i32, _p,
                                         _i32, C.c_double, _p, _p]
    L.kvq_oracle_decode_int4.restype = _i32
    L.kvq_oracle_decode_bf16.argtypes = [_p, _i32, _i32, _i32, _p, _i32, _i32, _p, _i32, _p, _i32,
                                         C.c_double, _p, _p]
    L.kvq_oracle_decode_bf16.restype = _i32
    L.kvq_oracle_decode_int4_bruteforce.argtypes = [_p, _i32, _i32, _i32, _i32, _p, _i32, _i32, _p,
                                                    _i32, _p, _i32, C.c_double, _p]
    L.kvq_oracle_decode_int4_bruteforce.restype = _i32
    L.kvq_oracle_decode_windowed.argtypes = [_p, _p, _i32, _i32, _i32, _i32, _p, _i32, _i32, _p, _i32,
                                             _p, _i32, _p, _i32, _i32, _i32, C.c_double, _p, _p]
    L.kvq_oracle_decode_windowed.restype = _i32
    L.kvq_oracle_num_threads.argtypes = []
    L.kvq_oracle_num_threads.restype = _i32
    L.kvq_oracle_set_num_threads.argtypes = [_i32]
    L.kvq_oracle_set_num_threads.restype = None


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- scalar formats --------------------------------------------------------

def f32_to_f16(x: float) -> int:
    return int(lib().kvq_oracle_f32_to_f16(float(x)))


def f16_to_f32(h: int) -> float:
    return float(lib().kvq_oracle_f16_to_f32(int(h)))


def f32_to_bf16(x: float) -> int:
    return int(lib().kvq_oracle_f32_to_bf16(float(x)))


def bf16_to_f32(h: int) -> float:
    return float(lib().kvq_oracle_bf16_to_f32(int(h)))


def block_scale(b: int) -> np.float32:
    return np.float32(lib().kvq_oracle_block_scale(int(b)))


# ---- per-vector steps ------------------------------------------------------

def rotate(x: np.ndarray, block: int) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().kvq_oracle_rotate(_ptr(x), _ptr(y), x.shape[-1], int(block))
    return y


def quantize(y: np.ndarray, bits: int = 4):
    """Returns (codes uint8[D], scale fp16 bits, zero fp16 bits); bits 4 or 8."""
    y = _c(y, np.float32)
    codes = np.empty(y.shape[-1], np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    fn = {4: lib().kvq_oracle_quantize, 8: lib().kvq_oracle_quantize_int8}[bits]
    fn(_ptr(y), y.shape[-1], _ptr(codes), _ptr(s), _ptr(z))
    return codes, int(s[0]), int(z[0])


def grid_sse(y: np.ndarray, codes: np.ndarray, scale: int, zero: int, k: int) -> int:
    """Grid SSE of the scale search and the hybrid mode (integer)."""
    y = _c(y, np.float32)
    codes = _c(codes, np.uint8)
    return int(lib().kvq_oracle_grid_sse(_ptr(y), y.shape[-1], _ptr(codes), int(scale), int(zero), int(k)))


def grid_exponent(amax: float) -> int:
    return int(lib().kvq_oracle_grid_exponent(float(amax)))


def quantize_search(y: np.ndarray):
    """Scale-searched INT4 of one key vector: (codes, scale bits, zero bits, j)."""
    y = _c(y, np.float32)
    codes = np.empty(y.shape[-1], np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    j = lib().kvq_oracle_quantize_search(_ptr(y), y.shape[-1], _ptr(codes), _ptr(s), _ptr(z))
    return codes, int(s[0]), int(z[0]), int(j)


def quantize_hybrid(y: np.ndarray):
    """Hybrid INT4 of one group: (codes, scale bits, zero bits, symmetric?)."""
    y = _c(y, np.float32)
    codes = np.empty(y.shape[-1], np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    sym = lib().kvq_oracle_quantize_hybrid(_ptr(y), y.shape[-1], _ptr(codes), _ptr(s), _ptr(z))
    return codes, int(s[0]), int(z[0]), bool(sym)


def e2m1_encode(v: float) -> int:
    return int(lib().kvq_oracle_e2m1_encode(float(v)))


def e2m1_decode(code: int) -> float:
    return float(lib().kvq_oracle_e2m1_decode(int(code)))


def quantize_mx(y: np.ndarray):
    """One MXFP4 block: (codes uint8[n], E8M0 scale byte)."""
    y = _c(y, np.float32)
    codes = np.empty(y.shape[-1], np.uint8)
    e = np.zeros(1, np.uint8)
    lib().kvq_oracle_quantize_mx(_ptr(y), y.shape[-1], _ptr(codes), _ptr(e))
    return codes, int(e[0])


# ---- cache -----------------------------------------------------------------

def int4_slab_bytes(page_size: int, head_dim: int) -> int:
    return int(lib().kvq_oracle_int4_slab_bytes(page_size, head_dim))


def int8_slab_bytes(page_size: int, head_dim: int) -> int:
    return int(lib().kvq_oracle_int8_slab_bytes(page_size, head_dim))


def int4g_slab_bytes(page_size: int, head_dim: int, group: int) -> int:
    return int(lib().kvq_oracle_int4g_slab_bytes(page_size, head_dim, group))


def new_int4g_pool(num_pages, num_kv_heads, head_dim, group, page_size=16, fill=0):
    n = num_pages * num_kv_heads * int4g_slab_bytes(page_size, head_dim, group)
    return np.full(n, fill, np.uint8)


def mxfp4_slab_bytes(page_size: int, head_dim: int) -> int:
    return int(lib().kvq_oracle_mxfp4_slab_bytes(page_size, head_dim))


def new_mxfp4_pool(num_pages, num_kv_heads, head_dim, page_size=16, fill=0):
    n = num_pages * num_kv_heads * mxfp4_slab_bytes(page_size, head_dim)
    return np.full(n, fill, np.uint8)


def bf16_slab_bytes(page_size: int, head_dim: int) -> int:
    return int(lib().kvq_oracle_bf16_slab_bytes(page_size, head_dim))


def new_int4_pool(num_pages, num_kv_heads, head_dim, page_size=16, fill=0):
    n = num_pages * num_kv_heads * int4_slab_bytes(page_size, head_dim)
    return np.full(n, fill, np.uint8)


def new_int8_pool(num_pages, num_kv_heads, head_dim, page_size=16, fill=0):
    n = num_pages * num_kv_heads * int8_slab_bytes(page_size, head_dim)
    return np.full(n, fill, np.uint8)


def new_bf16_pool(num_pages, num_kv_heads, head_dim, page_size=16, fill=0):
    n = num_pages * num_kv_heads * bf16_slab_bytes(page_size, head_dim)
    return np.full(n, fill, np.uint8)


def append_int4(pool, num_pages, num_kv_heads, head_dim, block, k, v, dtype, slot_mapping,
                page_size=16, token_stride=None):
    """k, v: uint16 bit patterns [T][token_stride] (or [T][Hkv][D])."""
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int32)
    t = sm.shape[0]
    if token_stride is None:
        token_stride = num_kv_heads * head_dim
    rc = lib().kvq_oracle_append_int4(_ptr(pool), num_pages, page_size, num_kv_heads, head_dim,
                                      int(block), _ptr(k), _ptr(v), int(dtype), int(token_stride),
                                      _ptr(sm), t)
    if rc != 0:
        raise ValueError("oracle append_int4 rejected its arguments")
    return pool


def append_int4_search(pool, num_pages, num_kv_heads, head_dim, block, k, v, dtype, slot_mapping,
                       page_size=16, token_stride=None):
    """As append_int4, with the keys quantized by the scale search."""
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int32)
    if token_stride is None:
        token_stride = num_kv_heads * head_dim
    rc = lib().kvq_oracle_append_int4_search(_ptr(pool), num_pages, page_size, num_kv_heads, head_dim,
                                             int(block), _ptr(k), _ptr(v), int(dtype), int(token_stride),
                                             _ptr(sm), sm.shape[0])
    if rc != 0:
        raise ValueError("oracle append_int4_search rejected its arguments")
    return pool


def append_int8(pool, num_pages, num_kv_heads, head_dim, block, k, v, dtype, slot_mapping,
                page_size=16, token_stride=None):
    """As append_int4, into the INT8 pool."""
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int32)
    if token_stride is None:
        token_stride = num_kv_heads * head_dim
    rc = lib().kvq_oracle_append_int8(_ptr(pool), num_pages, page_size, num_kv_heads, head_dim,
                                      int(block), _ptr(k), _ptr(v), int(dtype), int(token_stride),
                                      _ptr(sm), sm.shape[0])
    if rc != 0:
        raise ValueError("oracle append_int8 rejected its arguments")
    return pool


def append_int4g(pool, num_pages, num_kv_heads, head_dim, block, group, k, v, dtype,
                 slot_mapping, page_size=16, token_stride=None):
    """Per-group INT4 into the grouped pool."""
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int32)
    if token_stride is None:
        token_stride = num_kv_heads * head_dim
    rc = lib().kvq_oracle_append_int4g(_ptr(pool), num_pages, page_size, num_kv_heads, head_dim,
                                       int(block), int(group), _ptr(k), _ptr(v),
                                       int(dtype), int(token_stride), _ptr(sm), sm.shape[0])
    if rc != 0:
        raise ValueError("oracle append_int4g rejected its arguments")
    return pool


def append_int4g_hybrid(pool, num_pages, num_kv_heads, head_dim, block, group, k, v, dtype,
                        slot_mapping, page_size=16, token_stride=None):
    """Hybrid per-group INT4 into the grouped pool."""
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int32)
    if token_stride is None:
        token_stride = num_kv_heads * head_dim
    rc = lib().kvq_oracle_append_int4g_hybrid(_ptr(pool), num_pages, page_size, num_kv_heads, head_dim,
                                              int(block), int(group), _ptr(k), _ptr(v),
                                              int(dtype), int(token_stride), _ptr(sm), sm.shape[0])
    if rc != 0:
        raise ValueError("oracle append_int4g_hybrid rejected its arguments")
    return pool


def append_mxfp4(pool, num_pages, num_kv_heads, head_dim, block, k, v, dtype, slot_mapping,
                 page_size=16, token_stride=None):
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int32)
    if token_stride is None:
        token_stride = num_kv_heads * head_dim
    rc = lib().kvq_oracle_append_mxfp4(_ptr(pool), num_pages, page_size, num_kv_heads, head_dim,
                                       int(block), _ptr(k), _ptr(v), int(dtype), int(token_stride),
                                       _ptr(sm), sm.shape[0])
    if rc != 0:
        raise ValueError("oracle append_mxfp4 rejected its arguments")
    return pool


def append_bf16(pool, num_pages, num_kv_heads, head_dim, k, v, dtype, slot_mapping,
                page_size=16, token_stride=None):
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    sm = _c(slot_mapping, np.int32)
    if token_stride is None:
        token_stride = num_kv_heads * head_dim
    rc = lib().kvq_oracle_append_bf16(_ptr(pool), num_pages, page_size, num_kv_heads, head_dim,
                                      _ptr(k), _ptr(v), int(dtype), int(token_stride), _ptr(sm),
                                      sm.shape[0])
    if rc != 0:
        raise ValueError("oracle append_bf16 rejected its arguments")
    return pool


def int4_read(pool, num_kv_heads, head_dim, page, head, off, kind, channel, page_size=16):
    code = np.zeros(1, np.int32)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    val = lib().kvq_oracle_int4_read(_ptr(pool), page_size, num_kv_heads, head_dim, page, head,
                                     off, kind, channel, _ptr(code), _ptr(s), _ptr(z))
    return float(val), int(code[0]), int(s[0]), int(z[0])


def int8_read(pool, num_kv_heads, head_dim, page, head, off, kind, channel, page_size=16):
    code = np.zeros(1, np.int32)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    val = lib().kvq_oracle_int8_read(_ptr(pool), page_size, num_kv_heads, head_dim, page, head,
                                     off, kind, channel, _ptr(code), _ptr(s), _ptr(z))
    return float(val), int(code[0]), int(s[0]), int(z[0])


def int4g_read(pool, num_kv_heads, head_dim, group, page, head, off, kind, channel, page_size=16):
    code = np.zeros(1, np.int32)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    val = lib().kvq_oracle_int4g_read(_ptr(pool), page_size, num_kv_heads, head_dim, group, page,
                                      head, off, kind, channel, _ptr(code), _ptr(s), _ptr(z))
    return float(val), int(code[0]), int(s[0]), int(z[0])


def mxfp4_read(pool, num_kv_heads, head_dim, page, head, off, kind, channel, page_size=16):
    code = np.zeros(1, np.int32)
    e = np.zeros(1, np.uint8)
    val = lib().kvq_oracle_mxfp4_read(_ptr(pool), page_size, num_kv_heads, head_dim, page, head,
                                      off, kind, channel, _ptr(code), _ptr(e))
    return float(val), int(code[0]), int(e[0])


def bf16_read(pool, num_kv_heads, head_dim, page, head, off, kind, channel, page_size=16):
    return float(lib().kvq_oracle_bf16_read(_ptr(pool), page_size, num_kv_heads, head_dim, page,
                                            head, off, kind, channel))


def _pages_in_pool(block_table, pool, num_kv_heads, slab_bytes):
    """The block table with every id outside [0, num_pages) (num_pages from
    the pool's size) set to -1, which the decode reads as a page that is not
    there."""
    num_pages = np.asarray(pool).size // (num_kv_heads * slab_bytes)
    bt = np.asarray(block_table, dtype=np.int32)
    return np.where((bt >= 0) & (bt < num_pages), bt, -1).astype(np.int32)


def decode_int4(pool, num_kv_heads, head_dim, block, q, dtype, block_table, seq_lens, sm_scale,
                page_size=16, mask=None):
    q = _c(q, np.uint16)
    bt = _c(_pages_in_pool(block_table, pool, num_kv_heads, int4_slab_bytes(page_size, head_dim)), np.int32)
    sl = _c(seq_lens, np.int32)
    batch, hq, d = q.shape
    out = np.zeros((batch, hq, d), np.float64)
    mk = None if mask is None else _c(mask, np.uint8)
    rc = lib().kvq_oracle_decode_int4(_ptr(pool), page_size, num_kv_heads, head_dim, int(block),
                                      _ptr(q), int(dtype), hq, _ptr(bt), bt.shape[1], _ptr(sl),
                                      batch, float(sm_scale), None if mk is None else _ptr(mk),
                                      _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode_int4 rejected its arguments")
    return out


def decode_int8(pool, num_kv_heads, head_dim, block, q, dtype, block_table, seq_lens, sm_scale,
                page_size=16, mask=None):
    q = _c(q, np.uint16)
    bt = _c(_pages_in_pool(block_table, pool, num_kv_heads, int8_slab_bytes(page_size, head_dim)), np.int32)
    sl = _c(seq_lens, np.int32)
    batch, hq, d = q.shape
    out = np.zeros((batch, hq, d), np.float64)
    mk = None if mask is None else _c(mask, np.uint8)
    rc = lib().kvq_oracle_decode_int8(_ptr(pool), page_size, num_kv_heads, head_dim, int(block),
                                      _ptr(q), int(dtype), hq, _ptr(bt), bt.shape[1], _ptr(sl),
                                      batch, float(sm_scale), None if mk is None else _ptr(mk),
                                      _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode_int8 rejected its arguments")
    return out


def decode_int4g(pool, num_kv_heads, head_dim, block, group, q, dtype, block_table, seq_lens,
                 sm_scale, page_size=16, mask=None):
    q = _c(q, np.uint16)
    bt = _c(_pages_in_pool(block_table, pool, num_kv_heads, int4g_slab_bytes(page_size, head_dim, group)), np.int32)
    sl = _c(seq_lens, np.int32)
    batch, hq, d = q.shape
    out = np.zeros((batch, hq, d), np.float64)
    mk = None if mask is None else _c(mask, np.uint8)
    rc = lib().kvq_oracle_decode_int4g(_ptr(pool), page_size, num_kv_heads, head_dim, int(block),
                                       int(group), _ptr(q), int(dtype), hq, _ptr(bt), bt.shape[1],
                                       _ptr(sl), batch, float(sm_scale),
                                       None if mk is None else _ptr(mk), _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode_int4g rejected its arguments")
    return out


def decode_mxfp4(pool, num_kv_heads, head_dim, block, q, dtype, block_table, seq_lens, sm_scale,
                 page_size=16, mask=None):
    q = _c(q, np.uint16)
    bt = _c(_pages_in_pool(block_table, pool, num_kv_heads, mxfp4_slab_bytes(page_size, head_dim)), np.int32)
    sl = _c(seq_lens, np.int32)
    batch, hq, d = q.shape
    out = np.zeros((batch, hq, d), np.float64)
    mk = None if mask is None else _c(mask, np.uint8)
    rc = lib().kvq_oracle_decode_mxfp4(_ptr(pool), page_size, num_kv_heads, head_dim, int(block),
                                       _ptr(q), int(dtype), hq, _ptr(bt), bt.shape[1], _ptr(sl),
                                       batch, float(sm_scale), None if mk is None else _ptr(mk),
                                       _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode_mxfp4 rejected its arguments")
    return out


def decode_bf16(pool, num_kv_heads, head_dim, q, dtype, block_table, seq_lens, sm_scale,
                page_size=16, mask=None):
    q = _c(q, np.uint16)
    bt = _c(_pages_in_pool(block_table, pool, num_kv_heads, bf16_slab_bytes(page_size, head_dim)), np.int32)
    sl = _c(seq_lens, np.int32)
    batch, hq, d = q.shape
    out = np.zeros((batch, hq, d), np.float64)
    mk = None if mask is None else _c(mask, np.uint8)
    rc = lib().kvq_oracle_decode_bf16(_ptr(pool), page_size, num_kv_heads, head_dim, _ptr(q),
                                      int(dtype), hq, _ptr(bt), bt.shape[1], _ptr(sl), batch,
                                      float(sm_scale), None if mk is None else _ptr(mk), _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode_bf16 rejected its arguments")
    return out


def decode_windowed(int4_pool, win_pool, num_kv_heads, head_dim, block, q, dtype, block_table,
                    win_block_table, seq_lens, w_sink, w_recent, sm_scale, page_size=16, mask=None):
    q = _c(q, np.uint16)
    bt = _c(_pages_in_pool(block_table, int4_pool, num_kv_heads, int4_slab_bytes(page_size, head_dim)), np.int32)
    wbt = _c(_pages_in_pool(win_block_table, win_pool, num_kv_heads, bf16_slab_bytes(page_size, head_dim)), np.int32)
    sl = _c(seq_lens, np.int32)
    batch, hq, d = q.shape
    out = np.zeros((batch, hq, d), np.float64)
    mk = None if mask is None else _c(mask, np.uint8)
    rc = lib().kvq_oracle_decode_windowed(_ptr(int4_pool), _ptr(win_pool), page_size, num_kv_heads,
                                          head_dim, int(block), _ptr(q), int(dtype), hq, _ptr(bt),
                                          bt.shape[1], _ptr(wbt), wbt.shape[1], _ptr(sl), batch,
                                          int(w_sink), int(w_recent), float(sm_scale),
                                          None if mk is None else _ptr(mk), _ptr(out))
    if rc != 0:
        raise ValueError("oracle decode_windowed rejected its arguments")
    return out


def decode_int4_bruteforce(pool, num_kv_heads, head_dim, block, q, dtype, block_table, seq_lens,
                           sm_scale, page_size=16):
    q = _c(q, np.uint16)
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    batch, hq, d = q.shape
    out = np.zeros((batch, hq, d), np.float64)
    rc = lib().kvq_oracle_decode_int4_bruteforce(_ptr(pool), page_size, num_kv_heads, head_dim,
                                                 int(block), _ptr(q), int(dtype), hq, _ptr(bt),
                                                 bt.shape[1], _ptr(sl), batch, float(sm_scale),
                                                 _ptr(out))
    if rc != 0:
        raise ValueError("oracle bruteforce rejected its arguments")
    return out


def num_threads() -> int:
    return int(lib().kvq_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the following calls (timing only: the results are the same)."""
    lib().kvq_oracle_set_num_threads(int(n))

"""Python binding of libkvq.so (include/kvq.h): Hadamard-rotated token-wise
INT4 paged KV cache for MI355X (gfx950).

Argument marshalling only: torch tensors are passed as device pointers and the
current torch stream; every step of the write and read paths runs in the HIP
kernels of libkvq.so.  There is no fallback: if the library is missing, every
call raises.

Entry points carry the C names: ``kvq_append_paged``, ``kvq_decode_attn``,
``kvq_append_paged_int4_search``, ``kvq_append_paged_int4g_hybrid``,
``kvq_decode_attn_windowed``, ``kvq_append_paged_int8``, ``kvq_decode_attn_int8``,
``kvq_append_paged_int4g``, ``kvq_decode_attn_int4g``, ``kvq_append_paged_mxfp4``,
``kvq_decode_attn_mxfp4``,
``kvq_append_paged_bf16``, ``kvq_decode_attn_bf16``, the workspace and page
size queries.
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_ERR_INVALID_ARGUMENT, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE_TOO_SMALL, KVQ_ERR_HIP = range(5)
KVQ_F16, KVQ_BF16 = 0, 1
PAGE_SIZE = 16

# every symbol include/kvq.h declares
EXPORTED = (
    "kvq_int4_page_bytes", "kvq_int8_page_bytes", "kvq_int4g_page_bytes", "kvq_bf16_page_bytes",
    "kvq_append_paged", "kvq_decode_attn", "kvq_append_paged_int8", "kvq_decode_attn_int8",
    "kvq_append_paged_int4_search", "kvq_append_paged_int4g_hybrid", "kvq_decode_attn_noalloc",
    "kvq_append_paged_int4g", "kvq_decode_attn_int4g", "kvq_mxfp4_page_bytes",
    "kvq_append_paged_mxfp4", "kvq_decode_attn_mxfp4",
    "kvq_decode_workspace_bytes", "kvq_append_paged_bf16", "kvq_decode_attn_bf16",
    "kvq_decode_attn_windowed", "kvq_decode_windowed_workspace_bytes",
    "kvq_status_string", "kvq_last_error", "kvq_abi_version",
)


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _QuantDesc(C.Structure):   # kvq_int4_cache, kvq_int8_cache and kvq_mxfp4_cache
    _fields_ = [("pool", C.c_void_p), ("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("hadamard_block", C.c_int32)]


class _GroupedDesc(C.Structure):   # kvq_int4g_cache
    _fields_ = [("pool", C.c_void_p), ("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("hadamard_block", C.c_int32), ("group_size", C.c_int32)]


class _Bf16Desc(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32)]


_lib_handle = None


def lib() -> C.CDLL:
    """The loaded libkvq.so (raises if it was not built)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libkvq.so not found at {LIB_PATH}: build it with "
                "`python -m bit_kv_cache_block_amd.build` (no CPU fallback exists)")
        L = C.CDLL(LIB_PATH)
        p, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.kvq_int4_page_bytes.argtypes = [i32, i32, i32]
        L.kvq_int4_page_bytes.restype = sz
        L.kvq_int8_page_bytes.argtypes = [i32, i32, i32]
        L.kvq_int8_page_bytes.restype = sz
        L.kvq_mxfp4_page_bytes.argtypes = [i32, i32, i32]
        L.kvq_mxfp4_page_bytes.restype = sz
        L.kvq_int4g_page_bytes.argtypes = [i32, i32, i32, i32]
        L.kvq_int4g_page_bytes.restype = sz
        L.kvq_bf16_page_bytes.argtypes = [i32, i32, i32]
        L.kvq_bf16_page_bytes.restype = sz
        L.kvq_append_paged.argtypes = [C.POINTER(_QuantDesc), p, p, i32, i64, p, i32, p]
        L.kvq_append_paged.restype = i32
        L.kvq_append_paged_int4_search.argtypes = [C.POINTER(_QuantDesc), p, p, i32, i64, p, i32, p]
        L.kvq_append_paged_int4_search.restype = i32
        L.kvq_append_paged_int4g_hybrid.argtypes = [C.POINTER(_GroupedDesc), p, p, i32, i64, p, i32, p]
        L.kvq_append_paged_int4g_hybrid.restype = i32
        L.kvq_append_paged_int8.argtypes = [C.POINTER(_QuantDesc), p, p, i32, i64, p, i32, p]
        L.kvq_append_paged_int8.restype = i32
        L.kvq_append_paged_mxfp4.argtypes = [C.POINTER(_QuantDesc), p, p, i32, i64, p, i32, p]
        L.kvq_append_paged_mxfp4.restype = i32
        L.kvq_append_paged_int4g.argtypes = [C.POINTER(_GroupedDesc), p, p, i32, i64, p, i32, p]
        L.kvq_append_paged_int4g.restype = i32
        L.kvq_append_paged_bf16.argtypes = [C.POINTER(_Bf16Desc), p, p, i32, i64, p, i32, p]
        L.kvq_append_paged_bf16.restype = i32
        dec = [p, i32, i32, p, i32, p, i32, i32, C.c_float, i32, p, p, sz, p]
        L.kvq_decode_attn.argtypes = [C.POINTER(_QuantDesc), *dec]
        L.kvq_decode_attn.restype = i32
        L.kvq_decode_attn_noalloc.argtypes = [C.POINTER(_QuantDesc), *dec[:11], p]
        L.kvq_decode_attn_noalloc.restype = i32
        L.kvq_decode_attn_int8.argtypes = [C.POINTER(_QuantDesc), *dec]
        L.kvq_decode_attn_int8.restype = i32
        L.kvq_decode_attn_mxfp4.argtypes = [C.POINTER(_QuantDesc), *dec]
        L.kvq_decode_attn_mxfp4.restype = i32
        L.kvq_decode_attn_int4g.argtypes = [C.POINTER(_GroupedDesc), *dec]
        L.kvq_decode_attn_int4g.restype = i32
        L.kvq_decode_attn_bf16.argtypes = [C.POINTER(_Bf16Desc), *dec]
        L.kvq_decode_attn_bf16.restype = i32
        L.kvq_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.kvq_decode_workspace_bytes.restype = sz
        L.kvq_decode_attn_windowed.argtypes = [C.POINTER(_QuantDesc), C.POINTER(_Bf16Desc), p, i32, i32,
                                               p, i32, p, i32, p, i32, i32, i32, i32, C.c_float, i32,
                                               p, p, sz, p]
        L.kvq_decode_attn_windowed.restype = i32
        L.kvq_decode_windowed_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
        L.kvq_decode_windowed_workspace_bytes.restype = sz
        L.kvq_status_string.argtypes = [i32]
        L.kvq_status_string.restype = C.c_char_p
        L.kvq_last_error.argtypes = []
        L.kvq_last_error.restype = C.c_char_p
        L.kvq_abi_version.argtypes = []
        L.kvq_abi_version.restype = i32
        _lib_handle = L
    return _lib_handle


def _check(status: int) -> None:
    if status != KVQ_OK:
        L = lib()
        name = L.kvq_status_string(status).decode()
        raise KvqError(status, f"{name}: {L.kvq_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return KVQ_F16
    if t.dtype == torch.bfloat16:
        return KVQ_BF16
    raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")


# torch's current stream as a raw handle without building a Stream object
# (the per-call host cost matters for decode steps of a few sequences)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device) -> C.c_void_p:
    if stream is not None:
        return C.c_void_p(stream.cuda_stream)
    if _raw_stream is not None and device.index is not None:
        return C.c_void_p(_raw_stream(device.index))
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None) -> C.c_void_p:
    return C.c_void_p(0 if t is None else t.data_ptr())


def _same_gpu(pool: torch.Tensor, **tensors) -> None:
    """Every tensor handed to the library must live on the GPU that holds the
    cache pool: a host pointer or another device's pointer would reach a
    kernel as an address it cannot use."""
    dev = pool.get_device()
    if dev < 0 or not pool.is_cuda:
        raise ValueError("the cache pool must be a GPU tensor")
    for name, t in tensors.items():
        if t is not None and t.get_device() != dev:
            raise ValueError(f"{name} must be on the cache's GPU (cuda:{dev})")


def kvq_int4_page_bytes(page_size: int, num_kv_heads: int, head_dim: int) -> int:
    return int(lib().kvq_int4_page_bytes(page_size, num_kv_heads, head_dim))


def kvq_int8_page_bytes(page_size: int, num_kv_heads: int, head_dim: int) -> int:
    return int(lib().kvq_int8_page_bytes(page_size, num_kv_heads, head_dim))


def kvq_mxfp4_page_bytes(page_size: int, num_kv_heads: int, head_dim: int) -> int:
    return int(lib().kvq_mxfp4_page_bytes(page_size, num_kv_heads, head_dim))


def kvq_int4g_page_bytes(page_size: int, num_kv_heads: int, head_dim: int, group_size: int) -> int:
    return int(lib().kvq_int4g_page_bytes(page_size, num_kv_heads, head_dim, group_size))


def kvq_bf16_page_bytes(page_size: int, num_kv_heads: int, head_dim: int) -> int:
    return int(lib().kvq_bf16_page_bytes(page_size, num_kv_heads, head_dim))


class _QuantCache:
    """Caller-owned quantized page pool (uint8 tensor [num_pages][page bytes])."""

    _page_bytes = None

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int, hadamard_block: int,
                 device="cuda", page_size: int = PAGE_SIZE, pool: torch.Tensor | None = None):
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, num_kv_heads, head_dim
        self.hadamard_block, self.page_size = hadamard_block, page_size
        nbytes = type(self)._page_bytes(page_size, num_kv_heads, head_dim)
        if pool is None:
            pool = torch.zeros((num_pages, nbytes), dtype=torch.uint8, device=device)
        if pool.numel() < num_pages * nbytes or pool.dtype != torch.uint8 or not pool.is_contiguous():
            raise ValueError("pool must be a contiguous uint8 tensor of num_pages * page bytes")
        self.pool = pool

    def desc(self) -> _QuantDesc:
        return _QuantDesc(self.pool.data_ptr(), self.num_pages, self.page_size, self.num_kv_heads,
                          self.head_dim, self.hadamard_block)


class Int4Cache(_QuantCache):
    """INT4 page pool (kvq_int4_cache)."""
    _page_bytes = staticmethod(kvq_int4_page_bytes)


class Int8Cache(_QuantCache):
    """INT8 page pool (kvq_int8_cache)."""
    _page_bytes = staticmethod(kvq_int8_page_bytes)


class MxFp4Cache(_QuantCache):
    """MXFP4 page pool (kvq_mxfp4_cache)."""
    _page_bytes = staticmethod(kvq_mxfp4_page_bytes)


class Int4GroupedCache:
    """Caller-owned grouped INT4 page pool (kvq_int4g_cache)."""

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int, hadamard_block: int,
                 group_size: int, device="cuda", page_size: int = PAGE_SIZE,
                 pool: torch.Tensor | None = None):
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, num_kv_heads, head_dim
        self.hadamard_block, self.group_size, self.page_size = hadamard_block, group_size, page_size
        nbytes = kvq_int4g_page_bytes(page_size, num_kv_heads, head_dim, group_size)
        if nbytes == 0:
            raise ValueError("group_size must divide head_dim")
        if pool is None:
            pool = torch.zeros((num_pages, nbytes), dtype=torch.uint8, device=device)
        if pool.numel() < num_pages * nbytes or pool.dtype != torch.uint8 or not pool.is_contiguous():
            raise ValueError("pool must be a contiguous uint8 tensor of num_pages * page bytes")
        self.pool = pool

    def desc(self) -> _GroupedDesc:
        return _GroupedDesc(self.pool.data_ptr(), self.num_pages, self.page_size, self.num_kv_heads,
                            self.head_dim, self.hadamard_block, self.group_size)


def _need(cache, cls):
    if not isinstance(cache, cls):
        raise TypeError(f"expected {cls.__name__}, got {type(cache).__name__}")
    return cache


class Bf16Cache:
    """Caller-owned bf16 page pool (uint8 tensor [num_pages][page bytes])."""

    def __init__(self, num_pages: int, num_kv_heads: int, head_dim: int, device="cuda",
                 page_size: int = PAGE_SIZE, pool: torch.Tensor | None = None):
        self.num_pages, self.num_kv_heads, self.head_dim = num_pages, num_kv_heads, head_dim
        self.page_size = page_size
        nbytes = kvq_bf16_page_bytes(page_size, num_kv_heads, head_dim)
        if pool is None:
            pool = torch.zeros((num_pages, nbytes), dtype=torch.uint8, device=device)
        if pool.numel() < num_pages * nbytes or pool.dtype != torch.uint8 or not pool.is_contiguous():
            raise ValueError("pool must be a contiguous uint8 tensor of num_pages * page bytes")
        self.pool = pool

    def desc(self) -> _Bf16Desc:
        return _Bf16Desc(self.pool.data_ptr(), self.num_pages, self.page_size, self.num_kv_heads,
                         self.head_dim)


def _token_stride(k: torch.Tensor, v: torch.Tensor, hkv: int, d: int) -> int:
    ks, kst = k.shape, k.stride()
    if (len(ks) == 3 and ks[1] == hkv and ks[2] == d and kst[1] == d and kst[2] == 1
            and v.shape == ks and v.stride() == kst and v.dtype == k.dtype):
        return int(kst[0])
    for t in (k, v):   # say what is wrong
        if t.dim() != 3 or t.shape[1] != hkv or t.shape[2] != d:
            raise ValueError(f"k/v must be [T][{hkv}][{d}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != d:
            raise ValueError("each token's [Hkv][D] block of k/v must be contiguous")
    raise ValueError("k and v must share shape, dtype and token stride")


def _append(fn, cache, k, v, slot_mapping, stream):
    stride = _token_stride(k, v, cache.num_kv_heads, cache.head_dim)
    if slot_mapping.dtype != torch.int32 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int32 tensor")
    if slot_mapping.numel() != k.shape[0]:
        raise ValueError(f"slot_mapping has {slot_mapping.numel()} entries for {k.shape[0]} tokens")
    _same_gpu(cache.pool, k=k, v=v, slot_mapping=slot_mapping)
    _check(fn(C.byref(cache.desc()), _ptr(k), _ptr(v), _dtype_code(k), stride, _ptr(slot_mapping),
              int(k.shape[0]), _stream(stream, k.device)))


def kvq_append_paged(cache: Int4Cache, k: torch.Tensor, v: torch.Tensor,
                     slot_mapping: torch.Tensor, stream=None) -> None:
    """Rotate + quantize + scatter new tokens (k, v: [T][Hkv][D] fp16/bf16)."""
    _append(lib().kvq_append_paged, _need(cache, Int4Cache), k, v, slot_mapping, stream)


def kvq_append_paged_int4_search(cache: Int4Cache, k: torch.Tensor, v: torch.Tensor,
                                 slot_mapping: torch.Tensor, stream=None) -> None:
    """kvq_append_paged with the scale search for the keys."""
    _append(lib().kvq_append_paged_int4_search, _need(cache, Int4Cache), k, v, slot_mapping, stream)


def kvq_append_paged_int4g_hybrid(cache: Int4GroupedCache, k: torch.Tensor, v: torch.Tensor,
                                  slot_mapping: torch.Tensor, stream=None) -> None:
    """Per-group hybrid (symmetric or asymmetric) quantize + scatter into the grouped pool."""
    _append(lib().kvq_append_paged_int4g_hybrid, _need(cache, Int4GroupedCache), k, v, slot_mapping,
            stream)


def kvq_append_paged_int8(cache: Int8Cache, k: torch.Tensor, v: torch.Tensor,
                          slot_mapping: torch.Tensor, stream=None) -> None:
    """Rotate + quantize to 8 bits + scatter new tokens into the INT8 pool."""
    _append(lib().kvq_append_paged_int8, _need(cache, Int8Cache), k, v, slot_mapping, stream)


def kvq_append_paged_int4g(cache: Int4GroupedCache, k: torch.Tensor, v: torch.Tensor,
                           slot_mapping: torch.Tensor, stream=None) -> None:
    """Rotate + per-group quantize + scatter new tokens into the grouped pool."""
    _append(lib().kvq_append_paged_int4g, _need(cache, Int4GroupedCache), k, v, slot_mapping, stream)


def kvq_append_paged_mxfp4(cache: MxFp4Cache, k: torch.Tensor, v: torch.Tensor,
                           slot_mapping: torch.Tensor, stream=None) -> None:
    """Rotate + MXFP4-quantize + scatter new tokens into the MXFP4 pool."""
    _append(lib().kvq_append_paged_mxfp4, _need(cache, MxFp4Cache), k, v, slot_mapping, stream)


def kvq_append_paged_bf16(cache: Bf16Cache, k: torch.Tensor, v: torch.Tensor,
                          slot_mapping: torch.Tensor, stream=None) -> None:
    _append(lib().kvq_append_paged_bf16, _need(cache, Bf16Cache), k, v, slot_mapping, stream)


def kvq_decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                               max_seq_len: int, num_splits: int = 0) -> int:
    return int(lib().kvq_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                max_seq_len, num_splits))


def _decode_args(cache, q, block_table, seq_lens, out, **more):
    """Shape, dtype and device checks shared by the decode calls, made before
    anything is handed to the library; returns (batch, num_q_heads)."""
    d = cache.head_dim
    if q.dim() != 3 or q.shape[2] != d or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][Hq][D] tensor")
    batch, hq = int(q.shape[0]), int(q.shape[1])
    tables = (("block_table", block_table), ("seq_lens", seq_lens), *more.items())
    for name, t in tables:
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 tensor")
    if block_table.dim() != 2 or block_table.shape[0] != batch:
        raise ValueError(f"block_table must be [{batch}][max_pages_per_seq]")
    if seq_lens.numel() != batch:
        raise ValueError(f"seq_lens must hold {batch} lengths")
    for name, t in more.items():
        if t.dim() != 2 or t.shape[0] != batch:
            raise ValueError(f"{name} must be [{batch}][pages]")
    if out is not None:
        if out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor")
        if tuple(out.shape) != (batch, hq, d):
            raise ValueError(f"out must be [{batch}][{hq}][{d}], got {tuple(out.shape)}")
    _same_gpu(cache.pool, q=q, block_table=block_table, seq_lens=seq_lens, out=out, **more)
    return batch, hq


def _decode(fn, cache, q, block_table, seq_lens, max_seq_len, sm_scale, out, workspace,
            num_splits, stream):
    hkv, d = cache.num_kv_heads, cache.head_dim
    batch, hq = _decode_args(cache, q, block_table, seq_lens, out)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:   # (a caller's workspace size is checked by the library)
        need = kvq_decode_workspace_bytes(batch, hq, hkv, d, max_seq_len, num_splits)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _same_gpu(cache.pool, workspace=workspace)
    _check(fn(C.byref(cache.desc()), _ptr(q), _dtype_code(q), hq, _ptr(block_table),
              int(block_table.shape[1]), _ptr(seq_lens), batch, int(max_seq_len),
              float(sm_scale), int(num_splits), _ptr(out), _ptr(workspace),
              workspace.numel() * workspace.element_size(), _stream(stream, q.device)))
    return out


def kvq_decode_attn(cache: Int4Cache, q: torch.Tensor, block_table: torch.Tensor,
                    seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float | None = None,
                    out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                    num_splits: int = 0, stream=None) -> torch.Tensor:
    """Paged decode attention over the INT4 cache; returns fp32 [B][Hq][D]."""
    return _decode(lib().kvq_decode_attn, _need(cache, Int4Cache), q, block_table, seq_lens, max_seq_len,
                   sm_scale, out, workspace, num_splits, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20   # KVQ_NOALLOC_SCRATCH_BYTES


def kvq_decode_attn_noalloc(cache: Int4Cache, q: torch.Tensor, block_table: torch.Tensor,
                            seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float | None = None,
                            out: torch.Tensor | None = None, num_splits: int = 0,
                            stream=None) -> torch.Tensor:
    """kvq_decode_attn with the split-K partials in the library's static
    device scratch (no workspace); pass ``out`` and nothing is allocated."""
    cache = _need(cache, Int4Cache)
    batch, hq = _decode_args(cache, q, block_table, seq_lens, out)
    d = cache.head_dim
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    _check(lib().kvq_decode_attn_noalloc(
        C.byref(cache.desc()), _ptr(q), _dtype_code(q), hq, _ptr(block_table), int(block_table.shape[1]),
        _ptr(seq_lens), batch, int(max_seq_len), float(sm_scale), int(num_splits), _ptr(out),
        _stream(stream, q.device)))
    return out


def kvq_decode_attn_int8(cache: Int8Cache, q: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float | None = None,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         num_splits: int = 0, stream=None) -> torch.Tensor:
    """Paged decode attention over the INT8 cache; returns fp32 [B][Hq][D]."""
    return _decode(lib().kvq_decode_attn_int8, _need(cache, Int8Cache), q, block_table, seq_lens, max_seq_len,
                   sm_scale, out, workspace, num_splits, stream)


def kvq_decode_attn_int4g(cache: Int4GroupedCache, q: torch.Tensor, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float | None = None,
                          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                          num_splits: int = 0, stream=None) -> torch.Tensor:
    """Paged decode attention over the grouped INT4 cache; returns fp32 [B][Hq][D]."""
    return _decode(lib().kvq_decode_attn_int4g, _need(cache, Int4GroupedCache), q, block_table,
                   seq_lens, max_seq_len, sm_scale, out, workspace, num_splits, stream)


def kvq_decode_attn_mxfp4(cache: MxFp4Cache, q: torch.Tensor, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float | None = None,
                          out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                          num_splits: int = 0, stream=None) -> torch.Tensor:
    """Paged decode attention over the MXFP4 cache; returns fp32 [B][Hq][D]."""
    return _decode(lib().kvq_decode_attn_mxfp4, _need(cache, MxFp4Cache), q, block_table, seq_lens, max_seq_len,
                   sm_scale, out, workspace, num_splits, stream)


def kvq_decode_attn_bf16(cache: Bf16Cache, q: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float | None = None,
                         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                         num_splits: int = 0, stream=None) -> torch.Tensor:
    return _decode(lib().kvq_decode_attn_bf16, _need(cache, Bf16Cache), q, block_table, seq_lens,
                   max_seq_len, sm_scale, out, workspace, num_splits, stream)


def kvq_decode_windowed_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int,
                                        head_dim: int, max_seq_len: int, num_splits: int = 0) -> int:
    return int(lib().kvq_decode_windowed_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                         max_seq_len, num_splits))


def kvq_decode_attn_windowed(cache: Int4Cache, window: Bf16Cache, q: torch.Tensor,
                             block_table: torch.Tensor, window_table: torch.Tensor,
                             seq_lens: torch.Tensor, max_seq_len: int, w_sink: int, w_recent: int,
                             sm_scale: float | None = None, out: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None, num_splits: int = 0,
                             stream=None) -> torch.Tensor:
    """Decode attention with bf16 windows for the first w_sink and the last
    w_recent tokens of each sequence; returns fp32 [B][Hq][D]."""
    d = _need(cache, Int4Cache).head_dim
    batch, hq = _decode_args(cache, q, block_table, seq_lens, out, window_table=window_table)
    _same_gpu(cache.pool, window_pool=_need(window, Bf16Cache).pool)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:   # (a caller's workspace size is checked by the library)
        need = kvq_decode_windowed_workspace_bytes(batch, hq, cache.num_kv_heads, d, max_seq_len,
                                                   num_splits)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    else:
        _same_gpu(cache.pool, workspace=workspace)
    _check(lib().kvq_decode_attn_windowed(
        C.byref(cache.desc()), C.byref(window.desc()), _ptr(q), _dtype_code(q), hq,
        _ptr(block_table),
        int(block_table.shape[1]), _ptr(window_table), int(window_table.shape[1]), _ptr(seq_lens),
        batch, int(max_seq_len), int(w_sink), int(w_recent), float(sm_scale), int(num_splits),
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, q.device)))
    return out


def abi_version() -> int:
    return int(lib().kvq_abi_version())

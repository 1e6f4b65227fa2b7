"""CPU oracle for the block-paged KV cache path (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It wraps ``liboracle_hpkv.so`` (plain
C++, built by ``oracle/build.py`` with the host compiler) with numpy-facing
helpers. Nothing here touches the GPU library, and the GPU library never
touches this.

Element storage types are passed as strings: "f32", "f16", "bf16". Arrays of
bf16 values are carried as numpy ``uint16`` bit patterns, f16 as ``float16``
(or uint16 bits) and f32 as ``float32``.

Every function is pinned by the CPU tests in ``tests/test_oracle_*.py`` to
values the pages print, closed forms, library routines or invariants.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
KV_CODE = {"i8": 3, "fp8": 4}  # quantized pool element types (1 byte each)
_ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# status codes of the oracle library
OK = 0
BAD_ARG = 1
SEQ_PTR_FIRST = 2
SEQ_PTR_ORDER = 3
SEQ_PTR_LAST = 4
PAGE_RANGE = 5
CTX_RANGE = 6
OUT_OF_RANGE = 7

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    _build.ensure_built()
    lib = ctypes.CDLL(_build.LIB)
    vp, u64, i64, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
    lib.orc_validate_index_buffers.argtypes = [i32, u64, u64, vp, vp, u64, vp, u64]
    lib.orc_validate_index_buffers.restype = i32
    lib.orc_element_offset.argtypes = [i32, u64, u64, u64, u64, u64, u64, u64, u64, vp, u64,
                                       vp, u64, vp]
    lib.orc_element_offset.restype = i32
    lib.orc_slot_mapping.argtypes = [i32, vp, u64, vp, u64, u64, u64, vp, vp, vp]
    lib.orc_slot_mapping.restype = i32
    lib.orc_store_kvcache.argtypes = [u64, vp, vp, vp, vp, vp, u64, u64, u64, u64, u64]
    lib.orc_store_kvcache.restype = i64
    lib.orc_paged_attention_decode.argtypes = [i32, i32, vp, vp, vp, vp, u64, vp, vp, u64, u64,
                                               u64, u64, u64, u64, ctypes.c_double, vp, vp, i32]
    lib.orc_paged_attention_decode.restype = i32
    lib.orc_dense_attention.argtypes = [i32, vp, vp, vp, u64, u64, u64, u64, ctypes.c_double, vp]
    lib.orc_dense_attention.restype = i32
    lib.orc_paged_attention_prefill.argtypes = [i32, i32, vp, vp, vp, vp, u64, vp, vp, vp, u64,
                                                u64, u64, u64, u64, u64, ctypes.c_double, vp, vp]
    lib.orc_paged_attention_prefill.restype = i32
    lib.orc_paged_attention_decode_quant.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                                     vp, u64, vp, vp, u64, u64, u64, u64, u64,
                                                     u64, ctypes.c_double, vp, vp, i32]
    lib.orc_paged_attention_decode_quant.restype = i32
    lib.orc_store_kvcache_quant.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64,
                                            u64, u64, u64, u64]
    lib.orc_store_kvcache_quant.restype = i64
    lib.orc_fp8_e4m3_decode.argtypes = [vp, u64, vp]
    lib.orc_fp8_e4m3_decode.restype = None
    lib.orc_quantize.argtypes = [i32, vp, u64, vp]
    lib.orc_quantize.restype = None
    lib.orc_round_to_dtype.argtypes = [i32, vp, u64, vp]
    lib.orc_round_to_dtype.restype = None
    lib.orc_widen_dtype.argtypes = [i32, vp, u64, vp]
    lib.orc_widen_dtype.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _index_bytes(arr):
    if arr.dtype == np.uint32:
        return 4
    if arr.dtype == np.uint64:
        return 8
    raise TypeError(f"index buffers must be uint32 or uint64, got {arr.dtype}")


def _storage(arr, dtype):
    """Contiguous array holding the raw storage of elements of `dtype`."""
    a = np.ascontiguousarray(arr)
    want = {"f32": 4, "f16": 2, "bf16": 2}[dtype]
    if a.dtype.itemsize != want:
        raise TypeError(f"{dtype} storage needs {want}-byte elements, got {a.dtype}")
    return a


def validate_index_buffers(seq_ptr, block_table, num_pages, context_lens=None, page_size=0):
    """Returns the oracle status code of the storage-invariant check."""
    seq_ptr = np.ascontiguousarray(seq_ptr)
    block_table = np.ascontiguousarray(block_table, dtype=seq_ptr.dtype)
    ib = _index_bytes(seq_ptr)
    ctx = None if context_lens is None else np.ascontiguousarray(context_lens, dtype=np.int32)
    return _load().orc_validate_index_buffers(ib, num_pages, len(seq_ptr) - 1, _ptr(seq_ptr),
                                              _ptr(block_table), len(block_table), _ptr(ctx),
                                              page_size)


def element_offset(s, t, h, d, page_size, num_pages, num_heads, head_dim, block_table, seq_ptr):
    """(status, flat offset) of one logical element."""
    seq_ptr = np.ascontiguousarray(seq_ptr)
    block_table = np.ascontiguousarray(block_table, dtype=seq_ptr.dtype)
    out = np.zeros(1, dtype=np.uint64)
    st = _load().orc_element_offset(_index_bytes(seq_ptr), s, t, h, d, page_size, num_pages,
                                    num_heads, head_dim, _ptr(block_table), len(block_table),
                                    _ptr(seq_ptr), len(seq_ptr) - 1, _ptr(out))
    return st, int(out[0])


def slot_mapping(block_table, seq_ptr, page_size, num_pages, start_pos, cu_new):
    """Per-token slots over a CSR table (int64, -1 where no page or a page id >= num_pages)."""
    seq_ptr = np.ascontiguousarray(seq_ptr)
    block_table = np.ascontiguousarray(block_table, dtype=seq_ptr.dtype)
    start_pos = np.ascontiguousarray(start_pos, dtype=np.int32)
    cu_new = np.ascontiguousarray(cu_new, dtype=np.int64)
    slots = np.zeros(max(int(cu_new[-1]), 1), dtype=np.int64)
    st = _load().orc_slot_mapping(_index_bytes(seq_ptr), _ptr(block_table), len(block_table),
                                  _ptr(seq_ptr), len(seq_ptr) - 1, page_size, num_pages,
                                  _ptr(start_pos),
                                  _ptr(cu_new), _ptr(slots))
    if st != OK:
        raise ValueError(f"slot_mapping: oracle status {st}")
    return slots[:int(cu_new[-1])]


def store_kvcache(key, value, k_cache, v_cache, slots):
    """In-place store into numpy caches [num_pages, bs, H, d]; returns #invalid slots."""
    if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous")
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    num_pages, bs, H, d = k_cache.shape
    return _load().orc_store_kvcache(k_cache.dtype.itemsize, _ptr(key), _ptr(value), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(slots), len(slots), bs, num_pages, H, d)


def paged_attention_decode(dtype, q, k_cache, v_cache, block_table, seq_ptr, context_lens, scale,
                           num_threads=1):
    """Returns (out in storage dtype, out as float64) for q [B, Hq, d]."""
    q = _storage(q, dtype)
    k_cache = _storage(k_cache, dtype)
    v_cache = _storage(v_cache, dtype)
    seq_ptr = np.ascontiguousarray(seq_ptr)
    block_table = np.ascontiguousarray(block_table, dtype=seq_ptr.dtype)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, Hq, d = q.shape
    num_pages, bs, Hkv, d2 = k_cache.shape
    assert d2 == d and v_cache.shape == k_cache.shape and len(ctx) == B == len(seq_ptr) - 1
    out = np.empty_like(q)
    out64 = np.empty((B, Hq, d), dtype=np.float64)
    st = _load().orc_paged_attention_decode(_DTYPE_CODE[dtype], _index_bytes(seq_ptr), _ptr(q),
                                            _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                            len(block_table), _ptr(seq_ptr), _ptr(ctx), B, Hq, Hkv,
                                            d, bs, num_pages, float(scale), _ptr(out), _ptr(out64),
                                            int(num_threads))
    if st != OK:
        raise ValueError(f"paged_attention_decode: oracle status {st}")
    return out, out64


def paged_attention_prefill(dtype, q, k_cache, v_cache, block_table, seq_ptr, q_start, cu_q,
                            scale):
    """Causal chunked-prefill attention: (out in storage dtype, out as float64), q [Nq, Hq, d]."""
    q = _storage(q, dtype)
    k_cache = _storage(k_cache, dtype)
    v_cache = _storage(v_cache, dtype)
    seq_ptr = np.ascontiguousarray(seq_ptr)
    block_table = np.ascontiguousarray(block_table, dtype=seq_ptr.dtype)
    q_start = np.ascontiguousarray(q_start, dtype=np.int32)
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int64)
    Nq, Hq, d = q.shape
    num_pages, bs, Hkv, _ = k_cache.shape
    assert int(cu_q[-1]) == Nq and len(cu_q) == len(seq_ptr)
    out = np.empty_like(q)
    out64 = np.empty((Nq, Hq, d), dtype=np.float64)
    st = _load().orc_paged_attention_prefill(_DTYPE_CODE[dtype], _index_bytes(seq_ptr), _ptr(q),
                                             _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                             len(block_table), _ptr(seq_ptr), _ptr(q_start),
                                             _ptr(cu_q), len(seq_ptr) - 1, Hq, Hkv, d, bs,
                                             num_pages, float(scale), _ptr(out), _ptr(out64))
    if st != OK:
        raise ValueError(f"paged_attention_prefill: oracle status {st}")
    return out, out64


def fp8_e4m3_decode(codes):
    """float64 values of OCP E4M3 ("e4m3fn") codes (uint8 array)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_fp8_e4m3_decode(_ptr(c), c.size, _ptr(out))
    return out


def quantize(kv_type, t):
    """Codes (uint8) of fp32 values t: nearest, ties to even, saturating."""
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.empty(t.shape, dtype=np.uint8)
    _load().orc_quantize(KV_CODE[kv_type], _ptr(t), t.size, _ptr(out))
    return out


def store_kvcache_quant(dtype, kv_type, key, value, k_cache, v_cache, k_scale, k_zero, v_scale,
                        v_zero, slots):
    """In-place quantized store into uint8 pools [num_pages, bs, Hkv, d]; returns #skipped."""
    if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous")
    assert k_cache.dtype == np.uint8 and v_cache.dtype == np.uint8
    key = _storage(key, dtype)
    value = _storage(value, dtype)
    sc = [np.ascontiguousarray(x, dtype=np.float32) for x in (k_scale, k_zero, v_scale, v_zero)]
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    num_pages, bs, H, d = k_cache.shape
    r = _load().orc_store_kvcache_quant(_DTYPE_CODE[dtype], KV_CODE[kv_type], _ptr(key),
                                        _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                        *[_ptr(x) for x in sc], _ptr(slots), len(slots), bs,
                                        num_pages, H, d)
    if r < 0:
        raise ValueError("store_kvcache_quant: bad arguments")
    return r


def paged_attention_decode_quant(dtype, kv_type, q, k_cache, v_cache, k_scale, k_zero, v_scale,
                                 v_zero, block_table, seq_ptr, context_lens, scale,
                                 num_threads=1):
    """Decode over quantized pools; returns (out in dtype, out as float64)."""
    q = _storage(q, dtype)
    k_cache = np.ascontiguousarray(k_cache, dtype=np.uint8)
    v_cache = np.ascontiguousarray(v_cache, dtype=np.uint8)
    sc = [np.ascontiguousarray(x, dtype=np.float32) for x in (k_scale, k_zero, v_scale, v_zero)]
    seq_ptr = np.ascontiguousarray(seq_ptr)
    block_table = np.ascontiguousarray(block_table, dtype=seq_ptr.dtype)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, Hq, d = q.shape
    num_pages, bs, Hkv, _ = k_cache.shape
    assert all(x.size == num_pages * Hkv for x in sc)
    out = np.empty_like(q)
    out64 = np.empty((B, Hq, d), dtype=np.float64)
    st = _load().orc_paged_attention_decode_quant(
        _DTYPE_CODE[dtype], KV_CODE[kv_type], _index_bytes(seq_ptr), _ptr(q), _ptr(k_cache),
        _ptr(v_cache), *[_ptr(x) for x in sc], _ptr(block_table), len(block_table),
        _ptr(seq_ptr), _ptr(ctx), B, Hq, Hkv, d, bs, num_pages, float(scale), _ptr(out),
        _ptr(out64), int(num_threads))
    if st != OK:
        raise ValueError(f"paged_attention_decode_quant: oracle status {st}")
    return out, out64


def dense_attention(dtype, q, K, V, scale):
    """Textbook attention of one query q [Hq, d] over contiguous K, V [L, Hkv, d]."""
    q = _storage(q, dtype)
    K = _storage(K, dtype)
    V = _storage(V, dtype)
    Hq, d = q.shape
    L, Hkv, _ = K.shape
    out = np.empty((Hq, d), dtype=np.float64)
    st = _load().orc_dense_attention(_DTYPE_CODE[dtype], _ptr(q), _ptr(K), _ptr(V), L, Hq, Hkv, d,
                                     float(scale), _ptr(out))
    if st != OK:
        raise ValueError(f"dense_attention: oracle status {st}")
    return out


def round_to_dtype(dtype, x):
    """Rounds float64 values to the storage type (nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype={"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}[dtype])
    _load().orc_round_to_dtype(_DTYPE_CODE[dtype], _ptr(x), x.size, _ptr(out))
    return out


def widen_dtype(dtype, bits):
    """Widens stored elements (given as raw bits or native arrays) to float64."""
    bits = _storage(bits, dtype)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().orc_widen_dtype(_DTYPE_CODE[dtype], _ptr(bits), bits.size, _ptr(out))
    return out

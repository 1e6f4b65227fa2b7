"""Python binding of libhpkv.so, the gfx950 block-paged KV cache library.

Argument marshalling only: every function below forwards to the C entry point
of the same name declared in include/hpkv.h, passing tensor data pointers,
sizes read from tensor shapes and the current HIP stream. All computation runs
in the library's HIP kernels; there is no CPU fallback. Importing works
without a GPU (the library loads; host-only helpers run). A libhpkv.so that is
missing, or older than its sources, is first built with hipcc by build.py (a
build, not a fallback); if that build fails, the import raises.

Device tensors are torch tensors on a ROCm device. Index tensors
(block_table, seq_ptr) may be 32- or 64-bit (signed or unsigned); their width
selects HPKV_INDEX_U32 / HPKV_INDEX_U64.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhpkv.so")

OK = 0
ERR_NULL = -1
ERR_INVALID_ARG = -2
ERR_INVALID_INDEX = -3
ERR_UNSUPPORTED = -4
ERR_HIP = -5
ERR_WORKSPACE = -6
ERR_SCRATCH_LIMIT = -7

F32, F16, BF16 = 0, 1, 2
KV_I8, KV_FP8_E4M3 = 3, 4
KV_TYPES = {"i8": KV_I8, "fp8": KV_FP8_E4M3}
INDEX_U32, INDEX_U64 = 0, 1

_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

EXPORTED = [
    "hpkv_status_string", "hpkv_validate_index_buffers", "hpkv_element_offset",
    "hpkv_validate_shape", "hpkv_slot_mapping", "hpkv_store_kvcache",
    "hpkv_paged_attention_decode_workspace_size", "hpkv_paged_attention_decode_partition_tokens",
    "hpkv_paged_attention_decode", "hpkv_paged_attention_decode_partitions",
    "hpkv_paged_attention_decode_reduce", "hpkv_paged_attention_decode_step",
    "hpkv_paged_attention_prefill", "hpkv_store_kvcache_quant",
    "hpkv_paged_attention_decode_quant", "hpkv_bm_create", "hpkv_bm_destroy", "hpkv_bm_admit",
    "hpkv_bm_append", "hpkv_bm_release", "hpkv_bm_stats", "hpkv_bm_export", "hpkv_bm_check",
    "hpkv_xxh64", "hpkv_read_ceiling", "hpkv_paged_attention_decode_noalloc",
    "hpkv_paged_attention_decode_shared",
    "hpkv_paged_attention_decode_noalloc_max_workspace",
    "hpkv_paged_attention_decode_quant_partition_tokens",
]


class HpkvError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


def _load():
    from . import build as _build  # the build script; it imports nothing from the package
    try:
        _build.ensure_built()
    except Exception as e:  # no library means no path at all: fail loudly
        raise ImportError(f"{LIB_PATH} could not be built ({e}); there is no fallback path") from e
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u32, u64, f32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64,
                              ctypes.c_float)
    sz = ctypes.c_size_t
    sig = {
        "hpkv_status_string": ([i32], ctypes.c_char_p),
        "hpkv_validate_index_buffers": ([i32, u64, u64, vp, vp, u64, vp, u32], i32),
        "hpkv_element_offset": ([i32, u64, u64, u32, u32, u32, u64, u32, u32, vp, u64, vp, u64,
                                 vp], i32),
        "hpkv_validate_shape": ([u32, vp], i32),
        "hpkv_slot_mapping": ([i32, vp, u64, vp, u32, u32, u64, vp, vp, u64, vp, vp], i32),
        "hpkv_store_kvcache": ([i32, vp, vp, vp, vp, vp, u64, u32, u64, u32, u32, vp], i32),
        "hpkv_paged_attention_decode_workspace_size": ([i32, u32, u32, u32, u32, u32], sz),
        "hpkv_paged_attention_decode_partition_tokens": ([i32, u32, u32, u32, u32, u32, u32],
                                                         u32),
        "hpkv_paged_attention_decode_quant_partition_tokens": (
            [i32, i32, u32, u32, u32, u32, u32, u32], u32),
        "hpkv_paged_attention_decode": ([i32, i32, vp, vp, vp, vp, u64, vp, vp, u32, u32, u32,
                                         u32, u32, u64, f32, u32, vp, sz, vp, vp], i32),
        "hpkv_paged_attention_decode_shared": ([i32, i32, vp, vp, vp, vp, u64, vp, vp, u32, u32,
                                                u32, u32, u32, u64, f32, u32, vp, sz, vp, vp],
                                               i32),
        "hpkv_paged_attention_decode_partitions": ([i32, i32, vp, vp, vp, vp, u64, vp, vp, u32,
                                                    u32, u32, u32, u32, u64, f32, u32, vp, sz,
                                                    vp, vp], i32),
        "hpkv_paged_attention_decode_reduce": ([i32, vp, u32, u32, u32, u32, u32, u32, vp, sz,
                                                vp, vp], i32),
        "hpkv_paged_attention_decode_step": ([i32, i32, vp, vp, vp, vp, vp, vp, u64, vp, vp, u32,
                                              u32, u32, u32, u32, u64, f32, u32, vp, vp, sz, vp,
                                              vp], i32),
        "hpkv_store_kvcache_quant": ([i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, u64, u32,
                                      u64, u32, u32, vp], i32),
        "hpkv_paged_attention_decode_quant": ([i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, u64,
                                               vp, vp, u32, u32, u32, u32, u32, u64, f32, u32,
                                               vp, sz, vp, vp], i32),
        "hpkv_bm_create": ([u64, u32], vp),
        "hpkv_bm_destroy": ([vp], None),
        "hpkv_bm_admit": ([vp, u64, vp, u64, vp], i32),
        "hpkv_bm_append": ([vp, u64, ctypes.c_int32, vp], i32),
        "hpkv_bm_release": ([vp, u64], i32),
        "hpkv_bm_stats": ([vp, vp, vp, vp, vp], i32),
        "hpkv_bm_export": ([vp, vp, u32, i32, vp, u64, vp, vp, vp], i32),
        "hpkv_bm_check": ([vp], i32),
        "hpkv_xxh64": ([vp, u64, u64], u64),
        "hpkv_read_ceiling": ([vp, u64, u32, u64, u32, vp, vp], i32),
        "hpkv_paged_attention_decode_noalloc": ([i32, i32, vp, vp, vp, vp, u64, vp, vp, u32, u32,
                                                 u32, u32, u32, u64, f32, u32, vp, vp], i32),
        "hpkv_paged_attention_decode_noalloc_max_workspace": ([], sz),
        "hpkv_paged_attention_prefill": ([i32, i32, vp, vp, vp, vp, u64, vp, vp, vp, u32, u64,
                                          u32, u32, u32, u32, u64, f32, u32, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.hpkv_status_string(int(status)).decode()


def _check(fn, status):
    if status != OK:
        raise HpkvError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, *tensors):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    dev = next((t.device for t in tensors if t is not None and t.is_cuda), None)
    if dev is None:
        raise ValueError("device entry points need tensors on a ROCm device")
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _index_type(t):
    if t.element_size() == 4:
        return INDEX_U32
    if t.element_size() == 8:
        return INDEX_U64
    raise TypeError(f"index tensors must be 32- or 64-bit, got {t.dtype}")


def _contig(*tensors):
    for t in tensors:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to libhpkv must be contiguous")


# ---------------------------------------------------------------- host helpers

def _np_ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def hpkv_validate_index_buffers(seq_ptr, block_table, num_pages, context_lens=None, page_size=0):
    """Host check of the storage invariants; returns the status code."""
    import numpy as np
    seq_ptr = np.ascontiguousarray(seq_ptr)
    block_table = np.ascontiguousarray(block_table, dtype=seq_ptr.dtype)
    it = INDEX_U64 if seq_ptr.dtype.itemsize == 8 else INDEX_U32
    ctx = None if context_lens is None else np.ascontiguousarray(context_lens, dtype=np.int32)
    return lib.hpkv_validate_index_buffers(it, num_pages, len(seq_ptr) - 1, _np_ptr(seq_ptr),
                                           _np_ptr(block_table), len(block_table), _np_ptr(ctx),
                                           page_size)


def hpkv_element_offset(s, t, h, d, page_size, num_pages, num_heads, head_dim, block_table,
                        seq_ptr):
    """Host lookup of one element's flat pool offset: (status, offset)."""
    import numpy as np
    seq_ptr = np.ascontiguousarray(seq_ptr)
    block_table = np.ascontiguousarray(block_table, dtype=seq_ptr.dtype)
    it = INDEX_U64 if seq_ptr.dtype.itemsize == 8 else INDEX_U32
    out = ctypes.c_uint64(0)
    st = lib.hpkv_element_offset(it, s, t, h, d, page_size, num_pages, num_heads, head_dim,
                                 _np_ptr(block_table), len(block_table), _np_ptr(seq_ptr),
                                 len(seq_ptr) - 1, ctypes.byref(out))
    return st, int(out.value)


def hpkv_validate_shape(dims):
    arr = (ctypes.c_uint64 * max(1, len(dims)))(*dims)
    return lib.hpkv_validate_shape(len(dims), arr)


def hpkv_paged_attention_decode_workspace_size(dtype, num_seqs, num_q_heads, head_dim, page_size,
                                               max_context_len):
    return int(lib.hpkv_paged_attention_decode_workspace_size(
        _DTYPE_CODE[dtype], num_seqs, num_q_heads, head_dim, page_size, max_context_len))


def hpkv_paged_attention_decode_partition_tokens(dtype, num_seqs, num_q_heads, num_kv_heads,
                                                 head_dim, page_size, max_context_len):
    return int(lib.hpkv_paged_attention_decode_partition_tokens(
        _DTYPE_CODE[dtype], num_seqs, num_q_heads, num_kv_heads, head_dim, page_size,
        max_context_len))


def hpkv_paged_attention_decode_quant_partition_tokens(dtype, kv_type, num_seqs, num_q_heads,
                                                       num_kv_heads, head_dim, page_size,
                                                       max_context_len):
    return int(lib.hpkv_paged_attention_decode_quant_partition_tokens(
        _DTYPE_CODE[dtype], KV_TYPES[kv_type], num_seqs, num_q_heads, num_kv_heads, head_dim,
        page_size, max_context_len))


# -------------------------------------------------------------- device entry points

def hpkv_slot_mapping(block_table, seq_ptr, page_size, num_pages, start_pos, cu_new, slots,
                      stream=None):
    """slots[i] for every new token (int64, -1 where the page is missing or outside the pool
    of num_pages pages)."""
    _contig(block_table, seq_ptr, start_pos, cu_new, slots)
    assert start_pos.dtype == torch.int32 and cu_new.dtype == torch.int64
    assert slots.dtype == torch.int64
    it = _index_type(seq_ptr)
    assert block_table.element_size() == seq_ptr.element_size()
    _check("hpkv_slot_mapping", lib.hpkv_slot_mapping(
        it, _ptr(block_table), block_table.numel(), _ptr(seq_ptr), seq_ptr.numel() - 1,
        page_size, int(num_pages), _ptr(start_pos), _ptr(cu_new), slots.numel(), _ptr(slots),
        _stream(stream, slots)))


def hpkv_store_kvcache(key, value, k_cache, v_cache, slots, stream=None):
    """Scatter key/value rows [N, Hkv, d] into the pools [num_pages, bs, Hkv, d]."""
    _contig(key, value, k_cache, v_cache, slots)
    assert key.dtype == value.dtype == k_cache.dtype == v_cache.dtype
    assert slots.dtype == torch.int64
    num_pages, bs, hkv, d = k_cache.shape
    _check("hpkv_store_kvcache", lib.hpkv_store_kvcache(
        _DTYPE_CODE[k_cache.dtype], _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
        _ptr(slots), slots.numel(), bs, num_pages, hkv, d, _stream(stream, k_cache)))


def _decode_args(q, k_cache, v_cache, block_table, seq_ptr, context_lens, scale, max_context_len,
                 workspace, out):
    _contig(q, k_cache, v_cache, block_table, seq_ptr, context_lens, workspace, out)
    assert q.dtype == k_cache.dtype == v_cache.dtype == out.dtype
    assert context_lens.dtype == torch.int32
    assert block_table.element_size() == seq_ptr.element_size()
    B, hq, d = q.shape
    num_pages, bs, hkv, d2 = k_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_DTYPE_CODE[q.dtype], _index_type(seq_ptr), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_table), block_table.numel(), _ptr(seq_ptr), _ptr(context_lens), B, hq, hkv,
            d, bs, num_pages, float(scale), int(max_context_len), _ptr(workspace), ws_bytes,
            _ptr(out))


def hpkv_paged_attention_decode(q, k_cache, v_cache, block_table, seq_ptr, context_lens, scale,
                                max_context_len, workspace, out, stream=None):
    """out[s, h] = softmax(scale * q[s, h] . K_s^T) V_s over each sequence's pages."""
    args = _decode_args(q, k_cache, v_cache, block_table, seq_ptr, context_lens, scale,
                        max_context_len, workspace, out)
    _check("hpkv_paged_attention_decode",
           lib.hpkv_paged_attention_decode(*args, _stream(stream, q)))


def hpkv_paged_attention_decode_shared(q, k_cache, v_cache, block_table, seq_ptr, context_lens,
                                       scale, max_context_len, workspace, out, stream=None):
    """hpkv_paged_attention_decode for batches that alias pages: full partitions that
    consecutive sequences share are read once for all of them (same results)."""
    args = _decode_args(q, k_cache, v_cache, block_table, seq_ptr, context_lens, scale,
                        max_context_len, workspace, out)
    _check("hpkv_paged_attention_decode_shared",
           lib.hpkv_paged_attention_decode_shared(*args, _stream(stream, q)))


def hpkv_paged_attention_decode_noalloc(q, k_cache, v_cache, block_table, seq_ptr, context_lens,
                                        scale, max_context_len, out, stream=None):
    """hpkv_paged_attention_decode with the library's own fixed device scratch as workspace:
    allocates nothing (batches needing more than the scratch raise ERR_SCRATCH_LIMIT)."""
    args = _decode_args(q, k_cache, v_cache, block_table, seq_ptr, context_lens, scale,
                        max_context_len, None, out)
    (dt, it, qp, kp, vp_, btp, bt_len, spp, ctxp, B, hq, hkv, d, bs, num_pages, sc, mcl, _, _,
     outp) = args
    _check("hpkv_paged_attention_decode_noalloc", lib.hpkv_paged_attention_decode_noalloc(
        dt, it, qp, kp, vp_, btp, bt_len, spp, ctxp, B, hq, hkv, d, bs, num_pages, sc, mcl, outp,
        _stream(stream, q)))


def hpkv_paged_attention_decode_partitions(q, k_cache, v_cache, block_table, seq_ptr,
                                           context_lens, scale, max_context_len, workspace, out,
                                           stream=None):
    args = _decode_args(q, k_cache, v_cache, block_table, seq_ptr, context_lens, scale,
                        max_context_len, workspace, out)
    _check("hpkv_paged_attention_decode_partitions",
           lib.hpkv_paged_attention_decode_partitions(*args, _stream(stream, q)))


def hpkv_paged_attention_decode_reduce(context_lens, num_kv_heads, page_size, max_context_len,
                                       workspace, out, stream=None):
    _contig(context_lens, workspace, out)
    B, hq, d = out.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hpkv_paged_attention_decode_reduce", lib.hpkv_paged_attention_decode_reduce(
        _DTYPE_CODE[out.dtype], _ptr(context_lens), B, hq, num_kv_heads, d, page_size,
        int(max_context_len), _ptr(workspace), ws_bytes, _ptr(out), _stream(stream, out)))


def hpkv_paged_attention_decode_step(q, new_key, new_value, k_cache, v_cache, block_table,
                                     seq_ptr, context_lens, scale, max_context_len, workspace,
                                     out, slots_out=None, stream=None):
    """Fused decode step: store each sequence's newest K/V row (position ctx-1), then decode."""
    _contig(new_key, new_value, slots_out)
    assert new_key.dtype == new_value.dtype == q.dtype
    assert slots_out is None or slots_out.dtype == torch.int64
    (dt, it, qp, kp, vp_, btp, bt_len, spp, ctxp, B, hq, hkv, d, bs, num_pages, sc, mcl, wsp,
     ws_bytes, outp) = _decode_args(q, k_cache, v_cache, block_table, seq_ptr, context_lens,
                                    scale, max_context_len, workspace, out)
    assert tuple(new_key.shape) == (B, hkv, d) and new_value.shape == new_key.shape
    _check("hpkv_paged_attention_decode_step", lib.hpkv_paged_attention_decode_step(
        dt, it, qp, _ptr(new_key), _ptr(new_value), kp, vp_, btp, bt_len, spp, ctxp, B, hq, hkv,
        d, bs, num_pages, sc, mcl, _ptr(slots_out), wsp, ws_bytes, outp, _stream(stream, q)))


def hpkv_paged_attention_prefill(q, k_cache, v_cache, block_table, seq_ptr, q_start, cu_q, scale,
                                 max_q_len, out, stream=None):
    """Causal chunked-prefill attention: q/out [num_q_tokens, Hq, d]; sequence s owns rows
    cu_q[s] .. cu_q[s+1]-1 at positions q_start[s] + (i - cu_q[s])."""
    _contig(q, k_cache, v_cache, block_table, seq_ptr, q_start, cu_q, out)
    assert q.dtype == k_cache.dtype == v_cache.dtype == out.dtype
    assert q_start.dtype == torch.int32 and cu_q.dtype == torch.int64
    assert block_table.element_size() == seq_ptr.element_size()
    assert out.shape == q.shape
    nq, hq, d = q.shape
    num_pages, bs, hkv, d2 = k_cache.shape
    B = q_start.numel()
    assert cu_q.numel() == B + 1 and seq_ptr.numel() == B + 1
    _check("hpkv_paged_attention_prefill", lib.hpkv_paged_attention_prefill(
        _DTYPE_CODE[q.dtype], _index_type(seq_ptr), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), block_table.numel(), _ptr(seq_ptr), _ptr(q_start), _ptr(cu_q), B, nq,
        hq, hkv, d, bs, num_pages, float(scale), int(max_q_len), _ptr(out), _stream(stream, q)))


def hpkv_store_kvcache_quant(kv_type, key, value, k_cache, v_cache, k_scale, k_zero, v_scale,
                             v_zero, slots, stream=None):
    """Quantizing store into uint8 pools [num_pages, bs, Hkv, d]; scales fp32 [num_pages, Hkv]."""
    _contig(key, value, k_cache, v_cache, k_scale, k_zero, v_scale, v_zero, slots)
    assert k_cache.dtype == v_cache.dtype == torch.uint8 and slots.dtype == torch.int64
    assert all(x.dtype == torch.float32 for x in (k_scale, k_zero, v_scale, v_zero))
    num_pages, bs, hkv, d = k_cache.shape
    _check("hpkv_store_kvcache_quant", lib.hpkv_store_kvcache_quant(
        _DTYPE_CODE[key.dtype], KV_TYPES[kv_type], _ptr(key), _ptr(value), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(k_zero), _ptr(v_scale), _ptr(v_zero), _ptr(slots),
        slots.numel(), bs, num_pages, hkv, d, _stream(stream, k_cache)))


def hpkv_paged_attention_decode_quant(kv_type, q, k_cache, v_cache, k_scale, k_zero, v_scale,
                                      v_zero, block_table, seq_ptr, context_lens, scale,
                                      max_context_len, workspace, out, stream=None):
    """Decode over quantized uint8 pools; q/out keep their float type."""
    _contig(q, k_cache, v_cache, k_scale, k_zero, v_scale, v_zero, block_table, seq_ptr,
            context_lens, workspace, out)
    assert k_cache.dtype == v_cache.dtype == torch.uint8 and q.dtype == out.dtype
    assert context_lens.dtype == torch.int32
    assert all(x.dtype == torch.float32 for x in (k_scale, k_zero, v_scale, v_zero))
    B, hq, d = q.shape
    num_pages, bs, hkv, d2 = k_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hpkv_paged_attention_decode_quant", lib.hpkv_paged_attention_decode_quant(
        _DTYPE_CODE[q.dtype], KV_TYPES[kv_type], _index_type(seq_ptr), _ptr(q), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(k_zero), _ptr(v_scale), _ptr(v_zero),
        _ptr(block_table), block_table.numel(), _ptr(seq_ptr), _ptr(context_lens), B, hq, hkv,
        d, bs, num_pages, float(scale), int(max_context_len), _ptr(workspace), ws_bytes,
        _ptr(out), _stream(stream, q)))


# ------------------------------------------------------------ host block manager

class BlockManager:
    """Host page allocator with reference counts and chained-hash prefix reuse
    (hpkv_bm_* in include/hpkv.h). Every method forwards to the library."""

    def __init__(self, num_pages, page_size):
        self._destroy = lib.hpkv_bm_destroy  # kept: module globals may be gone at exit
        self._h = lib.hpkv_bm_create(int(num_pages), int(page_size))
        if not self._h:
            raise HpkvError("hpkv_bm_create", ERR_INVALID_ARG)
        self.num_pages, self.page_size = int(num_pages), int(page_size)

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def admit(self, seq_id, token_ids):
        """Admits a sequence with its prompt; returns the prompt tokens served from cache."""
        import numpy as np
        t = np.ascontiguousarray(token_ids, dtype=np.int32)
        cached = ctypes.c_uint64(0)
        _check("hpkv_bm_admit", lib.hpkv_bm_admit(self._h, int(seq_id), _np_ptr(t), t.size,
                                                  ctypes.byref(cached)))
        return cached.value

    def append(self, seq_id, token_id):
        """Appends one token; returns its pool slot."""
        slot = ctypes.c_int64(0)
        _check("hpkv_bm_append", lib.hpkv_bm_append(self._h, int(seq_id), int(token_id),
                                                    ctypes.byref(slot)))
        return slot.value

    def release(self, seq_id):
        _check("hpkv_bm_release", lib.hpkv_bm_release(self._h, int(seq_id)))

    def stats(self):
        v = [ctypes.c_uint64(0) for _ in range(4)]
        _check("hpkv_bm_stats", lib.hpkv_bm_stats(self._h, *[ctypes.byref(x) for x in v]))
        return dict(zip(("free", "allocated", "sequences", "cached"), (x.value for x in v)))

    def export(self, seq_ids, index="u32"):
        """(block_table, seq_ptr, context_lens) numpy arrays for the listed sequences."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.uint64)
        it = INDEX_U32 if index == "u32" else INDEX_U64
        dt = np.uint32 if index == "u32" else np.uint64
        sp = np.zeros(len(ids) + 1, dtype=dt)
        ctx = np.zeros(len(ids), dtype=np.int32)
        need = ctypes.c_uint64(0)
        st = lib.hpkv_bm_export(self._h, _np_ptr(ids), len(ids), it, None, 0, _np_ptr(sp),
                                _np_ptr(ctx), ctypes.byref(need))
        if st not in (OK, ERR_WORKSPACE):
            raise HpkvError("hpkv_bm_export", st)
        bt = np.zeros(max(need.value, 1), dtype=dt)
        _check("hpkv_bm_export", lib.hpkv_bm_export(self._h, _np_ptr(ids), len(ids), it,
                                                    _np_ptr(bt), bt.size, _np_ptr(sp),
                                                    _np_ptr(ctx), ctypes.byref(need)))
        return bt[:need.value], sp, ctx

    def check(self):
        """Status of the accounting-invariant check (OK or ERR_INVALID_INDEX)."""
        return lib.hpkv_bm_check(self._h)


def xxh64(data: bytes, seed: int = 0) -> int:
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    return int(lib.hpkv_xxh64(buf, len(data), int(seed)))


def alloc_workspace(q, k_cache, max_context_len):
    """Device workspace (uint8) sized for a decode call, or None if none is needed."""
    B, hq, d = q.shape
    n = hpkv_paged_attention_decode_workspace_size(q.dtype, B, hq, d, k_cache.shape[1],
                                                   max_context_len)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n else None


def hpkv_read_ceiling(buf, row_bytes, stride_bytes, rows_per_workgroup, sink, stream=None):
    """Reads the device buffer `buf` in rows of row_bytes at stride_bytes (one column per
    workgroup), the HBM read-ceiling measurement; `sink` is a 4-byte device tensor."""
    _contig(buf, sink)
    assert buf.is_cuda and sink.is_cuda and sink.numel() * sink.element_size() >= 4
    nbytes = buf.numel() * buf.element_size()
    _check("hpkv_read_ceiling", lib.hpkv_read_ceiling(
        _ptr(buf), nbytes, int(row_bytes), int(stride_bytes), int(rows_per_workgroup), _ptr(sink),
        _stream(stream, buf)))

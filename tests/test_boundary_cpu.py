"""The C ABI of libhpkv.so, checked without a GPU.

* the library loads and exports every function include/hpkv.h declares;
* the host helpers (index validation, element offset, rank check) reproduce
  the worked examples of "Block-Paged KV Cache" (Hurray docs) and agree with
  the oracle on random tables;
* malformed calls of the device entry points are refused with the documented
  status before any HIP call (so no GPU is needed to see it).
"""
import ctypes
import re
import subprocess

import numpy as np
import pytest

import oracle
import paged_kv_cache_hpkv_amd as hpkv
from conftest import ROOT, ints, read_golden

HEADER = f"{ROOT}/include/hpkv.h"
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hpkv_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert len(declared) == 29
    out = subprocess.run(["nm", "-D", "--defined-only", hpkv.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(hpkv_\w+)", out))
    assert set(declared) <= exported
    assert sorted(hpkv.EXPORTED) == declared
    for name in declared:
        assert getattr(hpkv.lib, name) is not None


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert hpkv.status_string(st) and hpkv.status_string(st) != "unknown status"
    assert hpkv.status_string(42) == "unknown status"


def test_printed_examples_through_the_library():
    lines = read_golden("element_offset.txt")
    geo = {k: int(v) for k, v in (kv.split("=") for kv in lines[0].split())}
    sp = np.array(ints(lines[1].split("=")[1]), dtype=np.uint32)
    bt = np.array(ints(lines[2].split("=")[1]), dtype=np.uint32)
    args = (geo["page_size"], geo["num_pages"], geo["num_heads"], geo["head_dim"], bt, sp)
    assert hpkv.hpkv_element_offset(0, 4, 0, 0, *args) == (hpkv.OK, 64)
    a = hpkv.hpkv_element_offset(0, 0, 0, 0, *args)
    b = hpkv.hpkv_element_offset(1, 0, 0, 0, *args)
    assert a == b and a[0] == hpkv.OK
    for line in read_golden("validate.txt"):
        verdict, num_pages, s, t = line.split()
        for dt in (np.uint32, np.uint64):
            st = hpkv.hpkv_validate_index_buffers(np.array(ints(s), dt), np.array(ints(t), dt),
                                                  int(num_pages))
            assert (st == hpkv.OK) == (verdict == "ok")
    # the logical tensor is rank 3 only
    assert hpkv.hpkv_validate_shape([9, 2, 8]) == hpkv.OK
    assert hpkv.hpkv_validate_shape([9, 2]) == hpkv.ERR_INVALID_ARG


def test_host_helpers_agree_with_oracle():
    rng = np.random.default_rng(3)
    for trial in range(200):
        dt = np.uint32 if trial % 2 else np.uint64
        num_pages = int(rng.integers(1, 10))
        B = int(rng.integers(0, 4))
        lens = rng.integers(0, 4, size=B)
        sp = np.zeros(B + 1, dtype=np.int64)
        sp[1:] = np.cumsum(lens)
        bt = rng.integers(0, num_pages + 1, size=int(sp[-1]))  # sometimes one past the pool
        if trial % 7 == 0 and B > 0:
            sp[-1] += 1  # break the last-offset invariant
        ctx = rng.integers(-1, 10, size=B).astype(np.int32)
        ps = int(rng.integers(1, 5))
        got = hpkv.hpkv_validate_index_buffers(sp.astype(dt), bt.astype(dt), num_pages, ctx, ps)
        want = oracle.validate_index_buffers(sp.astype(dt), bt.astype(dt), num_pages, ctx, ps)
        assert (got == hpkv.OK) == (want == oracle.OK)
        if want != oracle.OK or B == 0:
            continue
        for _ in range(5):
            s = int(rng.integers(0, B + 1))
            t, h, d = (int(x) for x in rng.integers(0, 9, size=3))
            g_st, g_off = hpkv.hpkv_element_offset(s, t, h % 3, d % 5, ps, num_pages, 2, 4,
                                                   bt.astype(dt), sp.astype(dt))
            o_st, o_off = oracle.element_offset(s, t, h % 3, d % 5, ps, num_pages, 2, 4,
                                                bt.astype(dt), sp.astype(dt))
            assert (g_st == hpkv.OK) == (o_st == oracle.OK)
            if g_st == hpkv.OK:
                assert g_off == o_off


def _decode_call(fn=hpkv.lib.hpkv_paged_attention_decode, **over):
    args = dict(dtype=hpkv.BF16, index=hpkv.INDEX_U32, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, bt_len=4,
                sp=FAKE, ctx=FAKE, B=2, hq=4, hkv=2, d=128, bs=16, num_pages=8, scale=0.1,
                max_ctx=4096, ws=FAKE, ws_bytes=0, out=FAKE, stream=None)
    args.update(over)
    return fn(*args.values())


def test_decode_argument_errors():
    assert _decode_call(dtype=7) == hpkv.ERR_INVALID_ARG
    assert _decode_call(index=3) == hpkv.ERR_INVALID_ARG
    assert _decode_call(q=None) == hpkv.ERR_NULL
    assert _decode_call(ctx=None) == hpkv.ERR_NULL
    assert _decode_call(out=None) == hpkv.ERR_NULL
    assert _decode_call(hq=6, hkv=4) == hpkv.ERR_INVALID_ARG      # Hq % Hkv != 0
    assert _decode_call(hkv=0) == hpkv.ERR_INVALID_ARG
    assert _decode_call(bs=0) == hpkv.ERR_INVALID_ARG
    assert _decode_call(num_pages=0) == hpkv.ERR_INVALID_ARG
    assert _decode_call(scale=float("nan")) == hpkv.ERR_INVALID_ARG
    assert _decode_call(q=ctypes.c_void_p(0x1008)) == hpkv.ERR_INVALID_ARG  # not 16-B aligned
    assert _decode_call(d=96) == hpkv.ERR_UNSUPPORTED
    assert _decode_call(d=512) == hpkv.ERR_UNSUPPORTED
    for dt in (hpkv.F32, hpkv.BF16):
        assert _decode_call(dtype=dt, d=4) == hpkv.ERR_UNSUPPORTED
    assert _decode_call(dtype=hpkv.F32, d=512) == hpkv.ERR_UNSUPPORTED
    # the two-head matrix-core shape keeps 32-bit pool slots: at most 2^32 slots
    assert _decode_call(B=1024, hq=8, hkv=2, num_pages=(1 << 28) + 1, ws_bytes=1 << 34) == \
        hpkv.ERR_UNSUPPORTED
    assert _decode_call(ws=None) == hpkv.ERR_WORKSPACE            # max_ctx 4096 needs partials
    need = hpkv.lib.hpkv_paged_attention_decode_workspace_size(hpkv.BF16, 2, 4, 128, 16, 4096)
    assert need > 0
    assert _decode_call(ws_bytes=need - 1) == hpkv.ERR_WORKSPACE
    assert _decode_call(fn=hpkv.lib.hpkv_paged_attention_decode_partitions, ws=None) \
        == hpkv.ERR_WORKSPACE
    # an empty batch is a no-op that succeeds without touching any pointer
    assert _decode_call(B=0, q=None, k=None, v=None, out=None, ctx=None) == hpkv.OK
    # the fused step needs the new rows, 16-byte aligned
    step = hpkv.lib.hpkv_paged_attention_decode_step
    args = [hpkv.BF16, hpkv.INDEX_U32, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 2, 4, 2,
            128, 16, 8, 0.1, 4096, None, FAKE, 1 << 30, FAKE, None]
    assert step(*args) == hpkv.ERR_NULL
    args[3] = ctypes.c_void_p(0x1008)
    assert step(*args) == hpkv.ERR_INVALID_ARG
    args[1] = 7
    assert step(*args) == hpkv.ERR_INVALID_ARG


def _prefill_call(**over):
    args = dict(dtype=hpkv.BF16, index=hpkv.INDEX_U32, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, bt_len=4,
                sp=FAKE, q_start=FAKE, cu_q=FAKE, B=2, nq=10, hq=8, hkv=2, d=128, bs=16,
                num_pages=8, scale=0.1, max_q=6, out=FAKE, stream=None)
    args.update(over)
    return hpkv.lib.hpkv_paged_attention_prefill(*args.values())


def test_prefill_argument_errors():
    assert _prefill_call(dtype=7) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(index=3) == hpkv.ERR_INVALID_ARG
    for name in ("q", "k", "v", "sp", "q_start", "cu_q", "out"):
        assert _prefill_call(**{name: None}) == hpkv.ERR_NULL, name
    assert _prefill_call(bt=None) == hpkv.ERR_NULL
    assert _prefill_call(hq=6, hkv=4) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(hkv=0) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(bs=0) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(num_pages=0) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(max_q=0) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(scale=float("nan")) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(out=ctypes.c_void_p(0x1008)) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(k=ctypes.c_void_p(0x1004)) == hpkv.ERR_INVALID_ARG
    assert _prefill_call(d=96) == hpkv.ERR_UNSUPPORTED
    assert _prefill_call(d=16) == hpkv.ERR_UNSUPPORTED
    assert _prefill_call(dtype=hpkv.F32) == hpkv.ERR_UNSUPPORTED
    # a group wider than the 128 rows of a workgroup, at every head size
    assert _prefill_call(hq=512, hkv=1) == hpkv.ERR_UNSUPPORTED
    assert _prefill_call(hq=258, hkv=2) == hpkv.ERR_UNSUPPORTED
    for d in (32, 64, 128, 256):
        assert _prefill_call(hq=256, hkv=1, d=d) == hpkv.ERR_UNSUPPORTED, d
    # pool rows (page * page_size + offset) are kept in 32 bits
    assert _prefill_call(num_pages=(1 << 28) + 1, bs=16) == hpkv.ERR_UNSUPPORTED
    # nothing to do: no sequences or no query rows
    assert _prefill_call(B=0, q=None, k=None, v=None, out=None) == hpkv.OK
    assert _prefill_call(nq=0, q=None, k=None, v=None, out=None, max_q=0) == hpkv.OK


def test_quant_argument_errors():
    st = hpkv.lib.hpkv_store_kvcache_quant
    good = [hpkv.BF16, hpkv.KV_FP8_E4M3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4,
            16, 8, 2, 128, None]

    def call(i, v, fn=st, base=good):
        a = list(base)
        a[i] = v
        return fn(*a)
    assert call(0, 9) == hpkv.ERR_INVALID_ARG
    assert call(1, hpkv.BF16) == hpkv.ERR_INVALID_ARG           # not a quantized type
    for i in range(2, 11):
        assert call(i, None) == hpkv.ERR_NULL, i
    assert call(12, 0) == hpkv.ERR_INVALID_ARG                  # page_size
    assert call(15, 12) == hpkv.ERR_UNSUPPORTED                 # head_dim not a multiple of 8
    assert call(2, ctypes.c_void_p(0x1008)) == hpkv.ERR_INVALID_ARG
    assert call(11, 0) == hpkv.OK                               # nothing to store
    dq = hpkv.lib.hpkv_paged_attention_decode_quant
    base = [hpkv.BF16, hpkv.KV_I8, hpkv.INDEX_U32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, 4, FAKE, FAKE, 2, 4, 2, 128, 16, 8, 0.1, 256, None, 0, FAKE, None]
    assert call(1, 2, dq, base) == hpkv.ERR_INVALID_ARG
    assert call(1, 7, dq, base) == hpkv.ERR_INVALID_ARG
    for i in (6, 7, 8, 9):
        assert call(i, None, dq, base) == hpkv.ERR_NULL, i
    assert call(17, 8, dq, base) == hpkv.ERR_UNSUPPORTED         # head_dim 8: half a lane chunk
    assert call(17, 96, dq, base) == hpkv.ERR_UNSUPPORTED
    assert call(21, 4096, dq, base) == hpkv.ERR_WORKSPACE        # several partitions need partials
    assert call(19, 1 << 31, dq, base) == hpkv.ERR_UNSUPPORTED   # pages * heads >= 2^32
    assert call(14, 0, dq, base) == hpkv.OK                      # empty batch


def test_partition_tokens_per_shape():
    """2048-token partitions where the batch still gives >= 1024 workgroups with them,
    else 1024-token ones where it gives >= 256 (KV heads / heads per workgroup x
    sequences x partitions), else 512."""
    pt = hpkv.lib.hpkv_paged_attention_decode_partition_tokens
    # GQA 32/8 on the matrix cores, two KV heads per workgroup: 4 head tiles
    assert pt(hpkv.BF16, 256, 32, 8, 128, 16, 8192) == 2048    # 4 * 256 * 4
    assert pt(hpkv.BF16, 64, 32, 8, 128, 16, 8192) == 2048     # 4 * 64 * 4 = 1024
    assert pt(hpkv.BF16, 63, 32, 8, 128, 16, 8192) == 1024     # 1008 < 1024
    assert pt(hpkv.BF16, 8, 32, 8, 128, 16, 8192) == 1024      # 4 * 8 * 8 = 256
    assert pt(hpkv.BF16, 7, 32, 8, 128, 16, 8192) == 512       # 224 < 256
    assert pt(hpkv.BF16, 1, 32, 8, 128, 16, 4096) == 512
    # MHA 32/32 on the VALU kernel: 16 two-head tiles, or 32 one-head tiles
    assert pt(hpkv.BF16, 64, 32, 32, 128, 16, 4096) == 2048    # 16 * 64 * 2
    assert pt(hpkv.BF16, 16, 32, 32, 128, 16, 4096) == 1024    # 16 * 16 * 4
    assert pt(hpkv.BF16, 2, 32, 32, 128, 16, 4096) == 1024     # 32 * 2 * 4 = 256
    assert pt(hpkv.BF16, 1, 32, 32, 128, 16, 4096) == 512      # 128 < 256
    assert pt(hpkv.F32, 128, 32, 8, 128, 16, 8192) == 2048     # VALU, 8 heads per tile
    assert pt(hpkv.BF16, 512, 24, 3, 128, 16, 8192) == 512     # odd Hkv on the matrix cores
    assert pt(hpkv.BF16, 8, 32, 0, 128, 16, 4096) == 0
    assert pt(hpkv.BF16, 8, 30, 8, 128, 16, 4096) == 0
    assert pt(9, 8, 32, 8, 128, 16, 4096) == 0


def test_quant_partition_tokens_per_shape():
    """Quantized pools: the same thresholds, among partitions whose pages fit the
    kernels' 520-entry page table (2048 tokens needs pages of >= 4 tokens, 1024 of >= 2);
    2048-token partitions on the matrix cores only."""
    pt = hpkv.lib.hpkv_paged_attention_decode_quant_partition_tokens
    fp8, i8 = hpkv.KV_FP8_E4M3, hpkv.KV_I8
    # GQA 32/8 on the matrix cores, two KV heads per workgroup: 4 head tiles (one KV
    # head, 8 tiles, when the batch is too small even for 512-token partitions)
    assert pt(hpkv.BF16, fp8, 256, 32, 8, 128, 16, 8192) == 2048   # 4 * 256 * 4
    assert pt(hpkv.BF16, i8, 64, 32, 8, 128, 16, 8192) == 2048     # 4 * 64 * 4 = 1024
    assert pt(hpkv.BF16, i8, 63, 32, 8, 128, 16, 8192) == 1024     # 1008 < 1024
    assert pt(hpkv.BF16, fp8, 8, 32, 8, 128, 16, 8192) == 1024     # 4 * 8 * 8 = 256
    assert pt(hpkv.BF16, fp8, 4, 32, 8, 128, 16, 8192) == 512      # 4 * 4 * 16 = 256
    assert pt(hpkv.BF16, fp8, 3, 32, 8, 128, 16, 8192) == 512      # one KV head, 512
    # page sizes bound the partition: 1-token pages 512, 2- and 3-token pages 1024
    assert pt(hpkv.BF16, fp8, 256, 32, 8, 128, 1, 8192) == 512
    assert pt(hpkv.BF16, fp8, 256, 32, 8, 128, 2, 8192) == 1024
    assert pt(hpkv.BF16, fp8, 256, 32, 8, 128, 3, 8192) == 1024
    assert pt(hpkv.BF16, fp8, 256, 32, 8, 128, 4, 8192) == 2048
    # VALU kernel, MHA 32/32 (two KV heads per workgroup: 16 head tiles): at most 1024
    assert pt(hpkv.F16, i8, 64, 32, 32, 128, 16, 4096) == 1024     # 16 * 64 * 4
    assert pt(hpkv.F32, fp8, 256, 32, 8, 128, 16, 8192) == 1024    # f32 q: VALU
    assert pt(hpkv.BF16, fp8, 2, 32, 32, 128, 16, 4096) == 512     # 32 * 2 * 8 = 512 at 512
    assert pt(hpkv.BF16, 5, 8, 32, 8, 128, 16, 4096) == 0          # not a quantized type
    assert pt(hpkv.BF16, fp8, 8, 32, 8, 128, 0, 4096) == 0         # page size 0


def test_reduce_argument_errors():
    red = hpkv.lib.hpkv_paged_attention_decode_reduce
    assert red(hpkv.BF16, FAKE, 4, 32, 0, 128, 16, 4096, FAKE, 1 << 20, FAKE, None) == \
        hpkv.ERR_INVALID_ARG
    assert red(hpkv.BF16, FAKE, 4, 30, 8, 128, 16, 4096, FAKE, 1 << 20, FAKE, None) == \
        hpkv.ERR_INVALID_ARG
    assert red(hpkv.BF16, FAKE, 4, 32, 8, 128, 16, 4096, None, 0, FAKE, None) == \
        hpkv.ERR_WORKSPACE
    assert red(hpkv.BF16, FAKE, 4, 32, 8, 128, 16, 512, None, 0, FAKE, None) == hpkv.OK  # one part
    assert red(hpkv.BF16, FAKE, 0, 32, 8, 128, 16, 4096, None, 0, FAKE, None) == hpkv.OK


def test_workspace_size_accounting():
    """The workspace is counted with the smaller, 512-token partition, so it covers
    every shape's plan: the (max, sum) pairs and the partial vectors, each padded
    to 256 bytes, then one u32 per (sequence, partition) for the dispatch order
    (padded), then one byte per pair for the shared-run flags."""
    P = hpkv.lib.hpkv_paged_attention_decode_partition_tokens(hpkv.BF16, 1, 32, 32, 128, 16,
                                                              4096)
    assert P == 512
    ws = hpkv.lib.hpkv_paged_attention_decode_workspace_size
    assert ws(hpkv.BF16, 64, 32, 128, 16, P) == 0           # one partition: no partials
    parts = -(-4096 // P)
    rows = 64 * 32 * parts
    pad = lambda b: -(-b // 256) * 256
    assert ws(hpkv.BF16, 64, 32, 128, 16, 4096) == \
        pad(rows * 8) + pad(rows * 128 * 4) + pad(64 * parts * 4) + 64 * parts
    rows = 3 * 5 * 2  # ragged: 3 sequences, 5 query heads, d = 8, two partitions
    assert ws(hpkv.F32, 3, 5, 8, 4, 513) == \
        pad(rows * 8) + pad(rows * 8 * 4) + pad(3 * 2 * 4) + 3 * 2
    assert ws(9, 64, 32, 128, 16, 4096) == 0


def test_store_and_slot_mapping_argument_errors():
    st = hpkv.lib.hpkv_store_kvcache
    assert st(9, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 16, 8, 2, 128, None) == hpkv.ERR_INVALID_ARG
    assert st(hpkv.BF16, None, FAKE, FAKE, FAKE, FAKE, 4, 16, 8, 2, 128, None) == hpkv.ERR_NULL
    assert st(hpkv.BF16, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 0, 8, 2, 128, None) == \
        hpkv.ERR_INVALID_ARG
    assert st(hpkv.BF16, None, None, None, None, None, 0, 16, 8, 2, 128, None) == hpkv.OK
    sm = hpkv.lib.hpkv_slot_mapping
    assert sm(5, FAKE, 4, FAKE, 2, 16, 8, FAKE, FAKE, 4, FAKE, None) == hpkv.ERR_INVALID_ARG
    assert sm(hpkv.INDEX_U32, FAKE, 4, FAKE, 2, 0, 8, FAKE, FAKE, 4, FAKE, None) == \
        hpkv.ERR_INVALID_ARG
    assert sm(hpkv.INDEX_U32, FAKE, 4, None, 2, 16, 8, FAKE, FAKE, 4, FAKE, None) == hpkv.ERR_NULL
    assert sm(hpkv.INDEX_U32, None, 0, None, 0, 16, 8, None, None, 0, None, None) == hpkv.OK


def test_read_ceiling_argument_errors():
    rc = hpkv.lib.hpkv_read_ceiling
    assert rc(None, 1 << 20, 256, 8192, 512, FAKE, None) == hpkv.ERR_NULL
    assert rc(FAKE, 1 << 20, 256, 8192, 512, None, None) == hpkv.ERR_NULL
    for row, stride, rows in ((8, 8192, 512), (192, 8192, 512), (8192, 8192, 64),
                              (256, 8000, 512), (256, 128, 512), (256, 8192, 0)):
        assert rc(FAKE, 1 << 20, row, stride, rows, FAKE, None) == hpkv.ERR_INVALID_ARG
    assert rc(ctypes.c_void_p(0x1008), 1 << 20, 256, 8192, 512, FAKE, None) == \
        hpkv.ERR_INVALID_ARG


def test_noalloc_decode_rejects_batches_beyond_its_scratch():
    """The no-allocation decode refuses, before any GPU work, a batch whose workspace would
    exceed its fixed scratch; argument errors are those of the workspace decode."""
    cap = hpkv.lib.hpkv_paged_attention_decode_noalloc_max_workspace()
    assert cap == 128 << 20
    na = hpkv.lib.hpkv_paged_attention_decode_noalloc
    ws = hpkv.lib.hpkv_paged_attention_decode_workspace_size
    # 4096 sequences x 32 heads x 128-token contexts of 64k tokens: far more than 128 MiB
    assert ws(hpkv.BF16, 4096, 32, 128, 16, 65536) > cap
    assert na(hpkv.BF16, hpkv.INDEX_U32, FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 4096, 32, 8,
              128, 16, 1 << 20, 0.1, 65536, FAKE, None) == hpkv.ERR_SCRATCH_LIMIT
    assert ws(hpkv.BF16, 64, 32, 128, 16, 4096) <= cap
    assert na(hpkv.BF16, hpkv.INDEX_U32, None, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 64, 32, 8, 128,
              16, 1 << 20, 0.1, 4096, FAKE, None) == hpkv.ERR_NULL
    assert na(hpkv.BF16, hpkv.INDEX_U32, FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 64, 32, 5, 128,
              16, 1 << 20, 0.1, 4096, FAKE, None) == hpkv.ERR_INVALID_ARG
    assert hpkv.status_string(hpkv.ERR_SCRATCH_LIMIT).startswith("batch needs more")

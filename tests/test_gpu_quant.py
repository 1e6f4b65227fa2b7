"""GPU parity of quantized pools (int8 / OCP fp8 E4M3 with per page-slot and
KV-head scales: "Block-Paged KV Cache", section "Quantization compatibility")
against the oracle, through the C ABI.

Each case: slot mapping of the step's new tokens, the quantizing store
(pools must match the oracle byte for byte), then decode over the quantized
pools (2e-2 absolute for bf16/f16 outputs, 1e-5 relative for f32). Pool rows
outside every context hold the fp8 NaN code, and the scales of pages no
sequence references are NaN, so a stray read shows up as NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_hpkv_amd as hpkv
import workloads
from paths import decode_errors, host_bits, host_threads, used_slots

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _poison(w, qt, kv):
    used = torch.zeros(w.num_pages * w.page_size, dtype=torch.bool)
    used[torch.from_numpy(used_slots(w))] = True
    if kv == "fp8":
        for pool in (qt.k_codes, qt.v_codes):
            pool.view(w.num_pages * w.page_size, -1)[~used.to(pool.device)] = 0x7F
    pages = used.view(w.num_pages, w.page_size).any(1).to(qt.k_scale.device)
    for sc in (qt.k_scale, qt.v_scale):
        sc[~pages] = float("nan")


def _step(w, kv, max_context_len=None, fp8_full_range=False):
    print(f"[quant parity] {w.name} {w.dtype} {kv} {w.index} B={w.num_seqs} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} d={w.head_dim} bs={w.page_size} full={fp8_full_range}",
          flush=True)
    t = workloads.make_tensors(w, DEV)
    qt = workloads.make_quant_tensors(w, kv, DEV, fp8_full_range=fp8_full_range)
    _poison(w, qt, kv)
    h = {name: getattr(qt, name).cpu().numpy().copy() for name in
         ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero")}
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    ctx = torch.from_numpy(w.context_lens).to(DEV)
    for c, (start, cu) in enumerate(w.chunks):
        slots = torch.empty(int(cu[-1]), dtype=torch.int64, device=DEV)
        hpkv.hpkv_slot_mapping(bt, sp, w.page_size, w.num_pages,
                               torch.from_numpy(start).to(DEV), torch.from_numpy(cu).to(DEV),
                               slots)
        if w.drop_mask is not None and c == 0:
            slots[torch.from_numpy(w.drop_mask).to(DEV)] = -1
        hpkv.hpkv_store_kvcache_quant(kv, t.new_keys[c], t.new_values[c], qt.k_codes,
                                      qt.v_codes, qt.k_scale, qt.k_zero, qt.v_scale, qt.v_zero,
                                      slots)
        o_slots = oracle.slot_mapping(w.block_table, w.seq_ptr, w.page_size, w.num_pages,
                                      start, cu)
        if w.drop_mask is not None and c == 0:
            o_slots[w.drop_mask] = -1
        oracle.store_kvcache_quant(w.dtype, kv, host_bits(t.new_keys[c]),
                                   host_bits(t.new_values[c]), h["k_codes"], h["v_codes"],
                                   h["k_scale"], h["k_zero"], h["v_scale"], h["v_zero"], o_slots)
    mcl = w.max_context_len if max_context_len is None else max_context_len
    out = torch.empty_like(t.q)
    ws = hpkv.alloc_workspace(t.q, qt.k_codes, mcl)
    hpkv.hpkv_paged_attention_decode_quant(kv, t.q, qt.k_codes, qt.v_codes, qt.k_scale,
                                           qt.k_zero, qt.v_scale, qt.v_zero, bt, sp, ctx,
                                           w.scale, mcl, ws, out)
    torch.cuda.synchronize()
    for name in ("k_codes", "v_codes"):
        assert getattr(qt, name).cpu().numpy().tobytes() == h[name].tobytes(), \
            f"{name} differs after the quantizing store"
    _, ref = oracle.paged_attention_decode_quant(
        w.dtype, kv, host_bits(t.q), h["k_codes"], h["v_codes"], h["k_scale"], h["k_zero"],
        h["v_scale"], h["v_zero"], w.block_table, w.seq_ptr, w.context_lens, w.scale,
        host_threads())
    max_err, ratio, finite = decode_errors(w.dtype, host_bits(out), ref)
    assert finite, "non-finite decode output"
    assert ratio <= 1.0, f"decode error {max_err} above tolerance"
    return out, qt


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("case", ["tiny_f32", "tiny16_bf16", "tiny256_f16"])
def test_quant_tiny(case, kv):
    name, dtype = case.split("_")
    bs = {"tiny": 4, "tiny16": 16, "tiny256": 256}[name]
    w = workloads.tiny(bs=bs, dtype=dtype)
    # head_dim 16 is the smallest quantized row (16 one-byte codes per lane chunk)
    w = workloads.Workload(**{**w.__dict__, "head_dim": 16, "scale": 16 ** -0.5})
    _step(w, kv)


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("wl", ["llama7b", "gqa", "qwen3"])
def test_quant_full_workloads(wl, kv):
    _step(workloads.WORKLOADS[wl](), kv)


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_quant_other_shapes(kv):
    base = workloads.gqa(batch=24)
    # groups of 1, 2, 3 (VALU path), 8 at d=256 (VALU), 8 and 16 at d=64/32 (matrix cores)
    for hq, hkv, d in [(8, 8, 64), (16, 8, 32), (32, 4, 256), (12, 4, 128), (32, 4, 64),
                       (32, 2, 32)]:
        w = workloads.Workload(**{**base.__dict__, "num_q_heads": hq, "num_kv_heads": hkv,
                                  "head_dim": d, "scale": d ** -0.5})
        _step(w, kv)


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_quant_gqa_f16(kv):
    _step(workloads.gqa(batch=48).with_dtype("f16"), kv)


def test_quant_u64_and_single_partition():
    w = workloads.llama7b(batch=8).with_index("u64")
    _step(w, "fp8")
    w = workloads.llama7b(batch=8)
    w.context_lens = np.minimum(w.context_lens, 400).astype(np.int32)
    w.chunks = workloads._decode_step_chunks(w.context_lens)
    _step(w, "i8", max_context_len=512)


@pytest.mark.parametrize("case", ["tiny16_bf16", "llama7b_bf16", "gqa_bf16", "gqa_f16",
                                  "qwen3_bf16", "tiny_f32"])
def test_fp8_full_code_range(case):
    """Every non-NaN E4M3 code (exponent fields 0-15, up to +-448) through the decode's
    conversions, and a quantizing store that saturates at +-448 and meets rounding ties,
    against the oracle byte for byte ("Block-Paged KV Cache", Quantization compatibility).
    The tiny cases store every context row themselves, so they cover the store's
    saturation and ties; the decode-step cases keep random history codes."""
    name, dtype = case.split("_")
    if name.startswith("tiny"):
        w = workloads.tiny(bs=16 if name == "tiny16" else 4, dtype=dtype)
        w = workloads.Workload(**{**w.__dict__, "head_dim": 16, "scale": 16 ** -0.5})
    else:
        w = workloads.WORKLOADS[name](batch=12).with_dtype(dtype)
    out, qt = _step(w, "fp8", fp8_full_range=True)
    # the stored rows saturated somewhere (+-448 is code 0x7e / 0xfe)
    slots = oracle.slot_mapping(w.block_table, w.seq_ptr, w.page_size, w.num_pages,
                                *w.chunks[0])
    stored = qt.k_codes.view(w.num_pages * w.page_size, -1)[torch.from_numpy(slots).to(DEV)]
    assert ((stored == 0x7E) | (stored == 0xFE)).any()
    if not name.startswith("tiny"):  # tiny rows are all written by the store itself
        used = torch.from_numpy(used_slots(w)).to(DEV)
        codes = qt.k_codes.view(w.num_pages * w.page_size, -1)[used].cpu().numpy()
        assert len(np.unique(codes)) >= 250  # the decode read the whole code range


def _shape(name, ctx, hq, hkv, d, bs, dtype="bf16", seed=41):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    num_pages, seq_ptr, bt = workloads._random_pool_tables(rng, ctx, bs, "u32")
    return workloads.Workload(name, dtype, "u32", hq, hkv, d, bs, num_pages, ctx, seq_ptr, bt,
                              d ** -0.5, chunks=workloads._decode_step_chunks(ctx), seed=seed)


@pytest.mark.parametrize("bs,part", [(1, 512), (2, 1024), (3, 1024), (4, 2048), (16, 2048)])
def test_quant_page_table_sizes(bs, part):
    """The quantized kernels keep one row-table entry per page: 1-token pages fill
    the 512 entries of a 512-token partition, 2-token pages 513 of 1024, 4-token
    pages 513 of 2048; 3-token pages start partitions inside a page. Matrix cores
    (GQA 32/8) and, where pages allow 1024-token partitions, the two-head VALU
    kernel (MHA 16/16)."""
    rng = np.random.default_rng(bs)
    ctx = rng.integers(1, 4097, 128)
    ctx[::7] = 4096
    w = _shape(f"pages-bs{bs}", ctx, 32, 8, 128, bs)
    got = hpkv.hpkv_paged_attention_decode_quant_partition_tokens(
        w.torch_dtype, "fp8", w.num_seqs, 32, 8, 128, bs, w.max_context_len)
    assert got == part
    _step(w, "fp8" if bs % 2 else "i8")
    if part > 512:
        w = _shape(f"pages-valu-bs{bs}", ctx, 16, 16, 128, bs, dtype="f16")
        assert hpkv.hpkv_paged_attention_decode_quant_partition_tokens(
            w.torch_dtype, "i8", w.num_seqs, 16, 16, 128, bs, w.max_context_len) == 1024
        _step(w, "i8")
        _step(w, "fp8")


def test_quant_malformed_page_in_a_long_partition():
    """A page id past the pool in the second 2048-token partition of one sequence gives
    that sequence NaN rows; every other sequence keeps finite results."""
    ctx = np.full(128, 3000, dtype=np.int32)
    w = _shape("pages-bad", ctx, 32, 8, 128, 16)
    assert hpkv.hpkv_paged_attention_decode_quant_partition_tokens(
        w.torch_dtype, "fp8", 128, 32, 8, 128, 16, w.max_context_len) == 2048
    t = workloads.make_tensors(w, DEV)
    qt = workloads.make_quant_tensors(w, "fp8", DEV)
    bt = w.block_table.copy()
    bad = 5
    bt[int(w.seq_ptr[bad]) + 2048 // 16 + 3] = w.num_pages + 7  # partition 1 of sequence 5
    out = torch.empty_like(t.q)
    ws = hpkv.alloc_workspace(t.q, qt.k_codes, w.max_context_len)
    hpkv.hpkv_paged_attention_decode_quant(
        "fp8", t.q, qt.k_codes, qt.v_codes, qt.k_scale, qt.k_zero, qt.v_scale, qt.v_zero,
        torch.from_numpy(bt).to(DEV), torch.from_numpy(w.seq_ptr).to(DEV),
        torch.from_numpy(w.context_lens).to(DEV), w.scale, w.max_context_len, ws, out)
    torch.cuda.synchronize()
    o = out.float().cpu()
    assert torch.isnan(o[bad]).all()
    good = torch.ones(128, dtype=torch.bool)
    good[bad] = False
    assert torch.isfinite(o[good]).all()

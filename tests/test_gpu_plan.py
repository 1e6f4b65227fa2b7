"""GPU parity across the decode launch plan's shapes.

The decode picks a launch shape per call: 2048-token partitions when their
grid still has 1024 workgroups, else the coarsest shape (two KV heads per
workgroup and/or 1024-token partitions) whose grid still has 256 workgroups,
else finer ones. Batch sizes here straddle those thresholds so that every
shape runs: for each case the partition size the library reports is checked
against the planned one, then the full step (slot mapping, store, decode) is
compared with the oracle, and the split partition/reduce entry points must
reproduce the decode bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_hpkv_amd as hpkv
import workloads
from paths import check_step, decode_errors, host_bits, host_threads, used_slots

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _shape(name, ctx, hq, hkv, d=128, dtype="bf16", bs=16, seed=11):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    num_pages, seq_ptr, bt = workloads._random_pool_tables(rng, ctx, bs, "u32")
    return workloads.Workload(name, dtype, "u32", hq, hkv, d, bs, num_pages, ctx, seq_ptr, bt,
                              d ** -0.5, chunks=workloads._decode_step_chunks(ctx), seed=seed)


# (name, context lengths, Hq, Hkv, planned partition tokens, head_dim)
CASES = [
    # matrix cores, GQA 32/8: two KV heads & 2048 (4*64*4 = 1024 workgroups; slot
    # row table, partial last partitions) ...
    ("mfma-2h-2048", [8192] * 40 + [5000] * 20 + [3000] * 4, 32, 8, 2048, 128),
    # ... two KV heads & 1024 (4*8*8 = 256 workgroups) ...
    ("mfma-2h-1024", [8192] * 8, 32, 8, 1024, 128),
    # ... two KV heads & 512 (4*7*8 = 224 < 256; 4*7*16 = 448) ...
    ("mfma-2h-512", [8192] * 6 + [1000], 32, 8, 512, 128),
    # ... one KV head & 512 (4*1*4 = 16 and 4*1*8 = 32 are below 256)
    ("mfma-1h-512", [4096], 32, 8, 512, 128),
    # VALU kernel (MHA 32/32): two KV heads & 2048 (16*32*2 = 1024; a ragged last
    # partition), then 1024 (32*2*4 = 256), then 512 (32*1*4 = 128)
    ("valu-2h-2048", [4096] * 31 + [3001], 32, 32, 2048, 128),
    ("valu-1024", [4096, 2500], 32, 32, 1024, 128),
    ("valu-512", [4096], 32, 32, 512, 128),
    # VALU kernel at d=64 (128-byte head rows): four KV heads & 1024 (4*16*4 = 256)
    ("valu-4h-1024-d64", [4096] * 16, 16, 16, 1024, 64),
]


@pytest.mark.parametrize("name,ctx,hq,hkv,part,d", CASES, ids=[c[0] for c in CASES])
def test_decode_plan_shapes(name, ctx, hq, hkv, part, d):
    w = _shape(name, ctx, hq, hkv, d=d)
    got = hpkv.hpkv_paged_attention_decode_partition_tokens(
        w.torch_dtype, w.num_seqs, hq, hkv, w.head_dim, w.page_size, w.max_context_len)
    assert got == part
    r = check_step(w)
    print(f"[plan] {name} part={part} max err {r['max_err']:.3e}", flush=True)
    # the split entry points plan the same partitions as the one-call decode
    t = r["tensors"]
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    ctx_t = torch.from_numpy(w.context_lens).to(DEV)
    ws = hpkv.alloc_workspace(t.q, t.k_cache, w.max_context_len)
    out = torch.full_like(t.q, float("nan"))
    hpkv.hpkv_paged_attention_decode_partitions(t.q, t.k_cache, t.v_cache, bt, sp, ctx_t, w.scale,
                                                w.max_context_len, ws, out)
    hpkv.hpkv_paged_attention_decode_reduce(ctx_t, hkv, w.page_size, w.max_context_len, ws, out)
    torch.cuda.synchronize()
    assert host_bits(out).tobytes() == host_bits(r["out"]).tobytes()


# quantized pools, VALU kernel (MHA 32/32): two KV heads per workgroup when
# 16 head pairs x sequences x partitions >= 256, else one
QCASES = [("q-2h", [4096] * 4, 32, 32), ("q-1h", [4096], 32, 32), ("q-2h-g2", [3000] * 16, 16, 8)]


@pytest.mark.parametrize("kv", ["fp8", "i8"])
@pytest.mark.parametrize("name,ctx,hq,hkv", QCASES, ids=[c[0] for c in QCASES])
def test_quant_decode_plan_shapes(name, ctx, hq, hkv, kv):
    w = _shape(name, ctx, hq, hkv, seed=13)
    print(f"[plan quant] {name} {kv}", flush=True)
    t = workloads.make_tensors(w, DEV)
    qt = workloads.make_quant_tensors(w, kv, DEV)
    used = torch.zeros(w.num_pages * w.page_size, dtype=torch.bool)
    used[torch.from_numpy(used_slots(w))] = True
    pages = used.view(w.num_pages, w.page_size).any(1).to(DEV)
    for sc in (qt.k_scale, qt.v_scale):  # pages no sequence references: NaN scales
        sc[~pages] = float("nan")
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    ctx_t = torch.from_numpy(w.context_lens).to(DEV)
    out = torch.empty_like(t.q)
    ws = hpkv.alloc_workspace(t.q, qt.k_codes, w.max_context_len)
    hpkv.hpkv_paged_attention_decode_quant(kv, t.q, qt.k_codes, qt.v_codes, qt.k_scale,
                                           qt.k_zero, qt.v_scale, qt.v_zero, bt, sp, ctx_t,
                                           w.scale, w.max_context_len, ws, out)
    torch.cuda.synchronize()
    hs = {n: getattr(qt, n).cpu().numpy() for n in
          ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero")}
    _, ref = oracle.paged_attention_decode_quant(
        w.dtype, kv, host_bits(t.q), hs["k_codes"], hs["v_codes"], hs["k_scale"], hs["k_zero"],
        hs["v_scale"], hs["v_zero"], w.block_table, w.seq_ptr, w.context_lens, w.scale,
        host_threads())
    max_err, ratio, finite = decode_errors(w.dtype, host_bits(out), ref)
    assert finite and ratio <= 1.0, max_err


def _expected_order(ctx, num_seqs, max_parts, part, max_ctx):
    """The dispatch order the ordering pass must write: pairs j = s + B * p stably
    sorted by length class (full partitions, 16 bands of partial ones from long to
    short, then empty or malformed pairs), with the pairs that have nothing to do
    (empty or malformed, partition 1 or later) written as 0xFFFFFFFF."""
    j = np.arange(num_seqs * max_parts, dtype=np.int64)
    n = np.asarray(ctx, dtype=np.int64)[j % num_seqs]
    p0 = (j // num_seqs) * part
    ln = np.clip(n - p0, 0, part)
    cls = np.where((n <= 0) | (n > max_ctx) | (n <= p0), 16, (part - ln) * 16 // part)
    order = np.argsort(cls, kind="stable")
    # pairs with nothing to do (empty class, not a first partition) are marked 0xFFFFFFFF
    no_work = (cls[order] == 16) & (order >= num_seqs)
    return np.where(no_work, 0xFFFFFFFF, order).astype(np.uint32)


def _pad256(b):
    return -(-b // 256) * 256


@pytest.mark.parametrize("name,ctx,hq,hkv,bad", [
    ("gqa-mixed", np.random.default_rng(5).integers(1, 5001, 300), 32, 8, True),
    ("mha-mixed", np.random.default_rng(6).integers(1, 3001, 40), 32, 32, False),
    ("small-grid", [2000] * 8, 8, 8, False),
])
def test_decode_dispatch_order(name, ctx, hq, hkv, bad):
    """The ordering pass writes, at the end of the workspace, the longest-first
    permutation of the (sequence, partition) pairs; grids that the chip holds at
    once (512 workgroups or fewer) skip it. Malformed lengths sort last and still
    give NaN rows."""
    w = _shape(name, ctx, hq, hkv, seed=17)
    t = workloads.make_tensors(w, DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    lens = w.context_lens.copy()
    if bad:
        lens[3], lens[10] = -3, w.max_context_len + 7
    ctx_t = torch.from_numpy(lens).to(DEV)
    part = hpkv.hpkv_paged_attention_decode_partition_tokens(
        w.torch_dtype, w.num_seqs, hq, hkv, w.head_dim, w.page_size, w.max_context_len)
    mp = -(-int(w.max_context_len) // part)
    rows = w.num_seqs * hq * mp
    off = _pad256(rows * 8) + _pad256(rows * w.head_dim * 4)
    ws = hpkv.alloc_workspace(t.q, t.k_cache, w.max_context_len)
    assert ws is not None and ws.numel() >= off + 4 * w.num_seqs * mp
    ws.fill_(0xFF)
    out = torch.empty_like(t.q)
    hpkv.hpkv_paged_attention_decode_partitions(t.q, t.k_cache, t.v_cache, bt, sp, ctx_t, w.scale,
                                                w.max_context_len, ws, out)
    torch.cuda.synchronize()
    got = ws[off:off + 4 * w.num_seqs * mp].cpu().numpy().view(np.uint32)
    print(f"[order] {name} part={part} pairs={w.num_seqs * mp}", flush=True)
    if name == "small-grid":
        assert np.all(got == 0xFFFFFFFF)
        return
    exp = _expected_order(lens, w.num_seqs, mp, part, w.max_context_len)
    assert np.array_equal(got, exp)
    if bad:
        hpkv.hpkv_paged_attention_decode_reduce(ctx_t, hkv, w.page_size, w.max_context_len, ws,
                                                out)
        torch.cuda.synchronize()
        o = out.float().cpu()
        assert torch.isnan(o[3]).all() and torch.isnan(o[10]).all()
        good = torch.ones(w.num_seqs, dtype=torch.bool)
        good[[3, 10]] = False
        assert torch.isfinite(o[good]).all()


def test_decode_dispatch_order_many_seqs():
    """Batches above 8192 sequences read the lengths from global memory instead
    of LDS in the ordering pass; the order must be the same permutation."""
    rng = np.random.default_rng(21)
    B, bs, d = 8300, 16, 64
    ctx = rng.integers(0, 4097, B).astype(np.int32)
    ctx[::97] = 4096  # the longest context sets max_context_len (two 2048-token partitions)
    pages = -(-ctx // bs)
    seq_ptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.uint32)
    num_pages = int(seq_ptr[-1])
    bt = torch.arange(num_pages, dtype=torch.int32, device=DEV)
    sp = torch.from_numpy(seq_ptr.view(np.int32)).to(DEV)
    ctx_t = torch.from_numpy(ctx).to(DEV)
    kc = torch.zeros(num_pages, bs, 1, d, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    q = torch.ones(B, 1, d, dtype=torch.bfloat16, device=DEV)
    max_ctx = int(ctx.max())
    part = hpkv.hpkv_paged_attention_decode_partition_tokens(torch.bfloat16, B, 1, 1, d, bs,
                                                             max_ctx)
    mp = -(-max_ctx // part)
    print(f"[order] many-seqs B={B} part={part} pairs={B * mp}", flush=True)
    rows = B * mp
    off = _pad256(rows * 8) + _pad256(rows * d * 4)
    ws = hpkv.alloc_workspace(q, kc, max_ctx)
    ws.fill_(0xFF)
    out = torch.empty_like(q)
    hpkv.hpkv_paged_attention_decode_partitions(q, kc, vc, bt, sp, ctx_t, d ** -0.5, max_ctx, ws,
                                                out)
    hpkv.hpkv_paged_attention_decode_reduce(ctx_t, 1, bs, max_ctx, ws, out)
    torch.cuda.synchronize()
    got = ws[off:off + 4 * B * mp].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, _expected_order(ctx, B, mp, part, max_ctx))
    assert torch.equal(out.float().cpu(), torch.zeros(B, 1, d))  # V rows are zeros


@pytest.mark.parametrize("hq,hkv", [(32, 8), (32, 32)])
def test_malformed_page_in_a_middle_partition(hq, hkv):
    """A partition that finds a page id past the pool writes NaN partials; the
    reduce turns them into NaN rows for that sequence alone, and every other
    sequence gets the bits of a clean run."""
    ctx = [5000, 3000, 4096, 700, 2049, 5000, 1]
    w = _shape("merge-bad", ctx, hq, hkv, seed=23)
    t = workloads.make_tensors(w, DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    ctx_t = torch.from_numpy(w.context_lens).to(DEV)
    ws = hpkv.alloc_workspace(t.q, t.k_cache, w.max_context_len)

    def run(bt_host):
        out = torch.full_like(t.q, float("nan"))
        hpkv.hpkv_paged_attention_decode(t.q, t.k_cache, t.v_cache,
                                         torch.from_numpy(bt_host).to(DEV), sp, ctx_t, w.scale,
                                         w.max_context_len, ws, out)
        torch.cuda.synchronize()
        return host_bits(out)

    good = run(w.block_table).copy()
    bt = w.block_table.copy()
    bt[int(w.seq_ptr[0]) + 1500 // w.page_size] = w.num_pages + 3  # token 1500 of sequence 0
    out = run(bt)
    outf = oracle.widen_dtype(w.dtype, out)
    print(f"[merge-bad] {hq}/{hkv}", flush=True)
    assert np.isnan(outf[0]).all()
    for s in range(1, len(ctx)):
        assert out[s].tobytes() == good[s].tobytes(), s
    r = check_step(w)  # and the clean run matches the oracle
    assert r["max_err"] < 2e-2

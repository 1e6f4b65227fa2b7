"""Shared partitions: hpkv_paged_attention_decode_shared.

Sequences that alias the same pages ("Block-Paged KV Cache", "Element lookup
through the block table"; the shared prefix pages of "Paged KV Cache · AI infra
interview lesson", Step 5) are served by one workgroup on the matrix cores when
they sit in one aligned block of 32/G consecutive sequences and a whole
partition covers the same page ids. Each sequence must get exactly the result
it gets when it owns private copies of those pages: the shared entry point on
the aliased batch, the plain decode on the aliased batch and the plain decode
on the same batch with every page duplicated per sequence must agree byte for
byte, and the result is checked against the oracle (2e-2 absolute for
bf16/f16).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_hpkv_amd as hpkv
import workloads
from paths import decode_errors, host_bits, host_threads, poison_unused
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode(w, q, kc, vc, block_table, seq_ptr, ctx, shared=False, keep_ws=False):
    out = torch.empty_like(q)
    mcl = w.max_context_len
    ws = hpkv.alloc_workspace(q, kc, mcl)
    if ws is not None:
        ws.fill_(0xFF)  # an order list the call does not write reads as no runs
    fn = hpkv.hpkv_paged_attention_decode_shared if shared else hpkv.hpkv_paged_attention_decode
    fn(q, kc, vc, torch.from_numpy(block_table).to(DEV), torch.from_numpy(seq_ptr).to(DEV),
       torch.from_numpy(ctx).to(DEV), w.scale, mcl, ws, out)
    torch.cuda.synchronize()
    return (out, ws) if keep_ws else out


def _private_copies(w, kc, vc):
    """Tables and pools in which every table entry is its own page (copied content)."""
    bt = w.block_table.astype(np.int64)
    idx = torch.from_numpy(bt).to(DEV)
    kc2 = kc[idx].contiguous() if len(bt) else kc[:1].clone()
    vc2 = vc[idx].contiguous() if len(bt) else vc[:1].clone()
    return np.arange(len(bt)).astype(w.block_table.dtype), kc2, vc2


def _runs(w, ws):
    """Entries of the dispatch order that serve a run of several sequences."""
    P = hpkv.hpkv_paged_attention_decode_partition_tokens(
        w.torch_dtype, w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
        w.max_context_len)
    mp = -(-w.max_context_len // P)
    rows = w.num_seqs * w.num_q_heads * mp
    pad = lambda b: -(-b // 256) * 256
    off = pad(rows * 8) + pad(rows * w.head_dim * 4)
    order = ws[off:off + 4 * w.num_seqs * mp].cpu().numpy().view(np.uint32)
    return int(((order != 0xFFFFFFFF) & (order >> 29 > 0)).sum())


def _check(w, ctx=None, expect_nan=(), expect_runs=None):
    print(f"[shared] {w.dtype} {w.index} B={w.num_seqs} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} d={w.head_dim} bs={w.page_size}", flush=True)
    ctx = w.context_lens if ctx is None else ctx
    t = workloads.make_tensors(w, DEV)
    poison_unused(w, t)
    out, ws = _decode(w, t.q, t.k_cache, t.v_cache, w.block_table, w.seq_ptr, ctx, shared=True,
                      keep_ws=True)
    plain = _decode(w, t.q, t.k_cache, t.v_cache, w.block_table, w.seq_ptr, ctx)
    bt2, kc2, vc2 = _private_copies(w, t.k_cache, t.v_cache)
    private = _decode(w, t.q, kc2, vc2, bt2, w.seq_ptr, ctx)
    assert host_bits(out).tobytes() == host_bits(private).tobytes()
    assert host_bits(plain).tobytes() == host_bits(private).tobytes()
    if expect_runs is not None:
        runs = _runs(w, ws)
        print(f"runs {runs}", flush=True)
        assert (runs > 0) == expect_runs
    got = host_bits(out)
    ok = np.ones(w.num_seqs, dtype=bool)
    ok[list(expect_nan)] = False
    for s in expect_nan:
        assert np.isnan(oracle.widen_dtype(w.dtype, got[s])).all()
    _, ref = oracle.paged_attention_decode(w.dtype, host_bits(t.q)[ok], host_bits(t.k_cache),
                                           host_bits(t.v_cache), *_subset(w, ok), ctx[ok],
                                           w.scale, host_threads())
    err, ratio, finite = decode_errors(w.dtype, got[ok], ref)
    assert finite and ratio <= 1.0, err
    return err


def _subset(w, keep):
    """Block table and seq_ptr of the kept sequences."""
    sp = w.seq_ptr.astype(np.int64)
    tables = [w.block_table[sp[s]:sp[s + 1]] for s in range(w.num_seqs) if keep[s]]
    seq_ptr = np.zeros(len(tables) + 1, dtype=np.int64)
    seq_ptr[1:] = np.cumsum([len(x) for x in tables])
    flat = np.concatenate(tables) if tables else np.zeros(0, dtype=w.block_table.dtype)
    return flat.astype(w.block_table.dtype), seq_ptr.astype(w.seq_ptr.dtype)


@pytest.mark.parametrize("group_size", [16, 6, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_aliased_prefix_equals_private_pages(group_size, dtype):
    """Aligned groups (runs of eight sequences fill two blocks of tile columns), groups that
    cross the blocks of eight, and groups smaller than a block."""
    w = workloads.chunked_prefill(dtype=dtype, groups=5, group_size=group_size,
                                  prefix_tokens=2048, tail_lo=4, tail_hi=900)
    _check(w, expect_runs=True)


@pytest.mark.parametrize("shape", [(64, 8, 128, 16), (32, 8, 64, 16), (32, 4, 32, 4),
                                   (128, 8, 128, 16), (32, 8, 128, 1)])
def test_shared_runs_other_shapes(shape):
    """Groups of 8 (runs of four), 16 (no runs), head sizes 64 and 32, 4-token pages
    (256 pages per partition, the most compared) and 1-token pages (too many pages to
    compare: no runs)."""
    hq, hkv, d, bs = shape
    w = workloads.chunked_prefill(groups=4, group_size=8,
                                  prefix_tokens=2048 if bs > 1 else 1024, num_q_heads=hq,
                                  num_kv_heads=hkv, head_dim=d, bs=bs, tail_lo=4, tail_hi=600)
    _check(w, expect_runs=hq // hkv <= 8 and bs > 1)


def test_prefix_not_a_whole_partition_and_u32():
    """A prefix of 1536 tokens: partition 0 is shared, partition 1 mixes shared and private
    pages and must not be; u32 tables."""
    w = workloads.chunked_prefill(index="u32", groups=4, group_size=8, prefix_tokens=1536,
                                  tail_lo=4, tail_hi=1200)
    _check(w)


def test_malformed_member_is_not_shared():
    """A sequence of a run whose length runs past its slice gets NaN; its neighbours keep
    their results, as with private pages."""
    w = workloads.chunked_prefill(groups=2, group_size=8, prefix_tokens=2048, tail_lo=16,
                                  tail_hi=300)
    ctx = w.context_lens.copy()
    sp = w.seq_ptr.astype(np.int64)
    bad = 5
    ctx[bad] = int(sp[bad + 1] - sp[bad]) * w.page_size + 1  # one token past the slice
    w2 = workloads.Workload(**{**w.__dict__, "context_lens": ctx})
    _check(w2, ctx=ctx, expect_nan=(bad,))


def test_no_aliasing_no_runs():
    """A batch without aliased pages (the GQA shape) forms no runs and gives the plain
    decode's bits."""
    _check(workloads.gqa(batch=48), expect_runs=False)

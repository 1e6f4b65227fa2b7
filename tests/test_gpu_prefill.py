"""GPU parity of causal chunked-prefill attention (hpkv_paged_attention_prefill)
against the oracle, through the C ABI.

Each case runs, per chunk: slot mapping + store of the chunk's K/V rows, then
prefill attention of the chunk's queries, on the library and on the oracle
from the same seeded inputs. Pool rows outside every sequence's final context
hold NaN, so a read past a chunk's visible keys or into an unreferenced page
shows up as NaN. Tolerance: 2e-2 absolute for bf16/f16 (fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_hpkv_amd as hpkv
import workloads
from paths import (decode_errors, gpu_prefill, host_bits, host_inputs, max_chunk_len,
                   oracle_prefill, poison_unused)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(name, dtype="bf16", index="u32", seed=11, **kw):
    return workloads.chunked_prefill(name, dtype, index, seed, **kw)


# (groups, group_size, prefix_tokens, n_chunks, Hq, Hkv, d, bs, tail_lo, tail_hi)
SHAPES = {
    # GQA 4:1 at the Llama head size; chunks span several workgroups and tiles
    "g4_d128_bs16": dict(groups=2, group_size=3, prefix_tokens=64, n_chunks=3, num_q_heads=8,
                         num_kv_heads=2, head_dim=128, bs=16, tail_lo=40, tail_hi=400),
    # MHA, 4-token pages (every tile crosses pages), chunks longer than a workgroup block
    "g1_d64_bs4": dict(groups=3, group_size=1, prefix_tokens=8, n_chunks=2, num_q_heads=4,
                       num_kv_heads=4, head_dim=64, bs=4, tail_lo=100, tail_hi=700),
    # wide group, 12-token pages (not a power of two), small heads
    "g8_d32_bs12": dict(groups=2, group_size=2, prefix_tokens=24, n_chunks=3, num_q_heads=16,
                        num_kv_heads=2, head_dim=32, bs=12, tail_lo=30, tail_hi=200),
    # 256-token pages, largest head size
    "g2_d256_bs256": dict(groups=2, group_size=2, prefix_tokens=256, n_chunks=2, num_q_heads=4,
                          num_kv_heads=2, head_dim=256, bs=256, tail_lo=50, tail_hi=300),
    # a group that does not divide the workgroup's rows (3 heads per KV head)
    "g3_d128_bs16": dict(groups=1, group_size=4, prefix_tokens=32, n_chunks=2, num_q_heads=6,
                         num_kv_heads=2, head_dim=128, bs=16, tail_lo=20, tail_hi=300),
    # 16 heads per KV head: 16 positions per workgroup
    "g16_d64_bs16": dict(groups=1, group_size=3, prefix_tokens=16, n_chunks=2, num_q_heads=32,
                         num_kv_heads=2, head_dim=64, bs=16, tail_lo=10, tail_hi=80),
    # one-token pages (every key its own page) and three-token pages
    "g2_d64_bs1": dict(groups=2, group_size=2, prefix_tokens=5, n_chunks=2, num_q_heads=4,
                       num_kv_heads=2, head_dim=64, bs=1, tail_lo=20, tail_hi=150),
    "g4_d128_bs3": dict(groups=1, group_size=3, prefix_tokens=9, n_chunks=3, num_q_heads=8,
                        num_kv_heads=2, head_dim=128, bs=3, tail_lo=30, tail_hi=200),
    # the widest group a workgroup holds (128 query heads per KV head: one position per
    # workgroup at every head size)
    "g128_d64_bs16": dict(groups=1, group_size=2, prefix_tokens=16, n_chunks=2, num_q_heads=128,
                          num_kv_heads=1, head_dim=64, bs=16, tail_lo=5, tail_hi=40),
    # whole prompts from position 0, one chunk each, no prefix
    "from0_g4_d128": dict(groups=4, group_size=1, prefix_tokens=0, n_chunks=1, num_q_heads=8,
                          num_kv_heads=2, head_dim=128, bs=16, tail_lo=1, tail_hi=300),
}


def _run(w, max_q_len=None, sample_rows=None):
    print(f"[prefill parity] {w.name} {w.dtype} {w.index} B={w.num_seqs} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} d={w.head_dim} bs={w.page_size} "
          f"rows={[int(cu[-1]) for _, cu in w.chunks]}", flush=True)
    t = workloads.make_tensors(w, DEV)
    poison_unused(w, t)
    qs = workloads.make_prefill_queries(w, DEV)
    h = host_inputs(t)
    q_bits = [host_bits(q) for q in qs]
    g_out = gpu_prefill(w, t, qs, max_q_len)
    o_out = oracle_prefill(w, h, q_bits, sample_rows)
    for name in ("k_cache", "v_cache"):
        assert host_bits(getattr(t, name)).tobytes() == h[name].tobytes(), name
    worst = 0.0
    for c in range(len(w.chunks)):
        got = host_bits(g_out[c])
        if sample_rows is not None:
            got = got[sample_rows[c]]
        max_err, ratio, finite = decode_errors(w.dtype, got, o_out[c])
        assert finite, f"chunk {c}: non-finite output"
        assert ratio <= 1.0, f"chunk {c}: error {max_err} above tolerance"
        worst = max(worst, max_err)
    return worst, g_out


@pytest.mark.parametrize("shape", sorted(SHAPES))
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_matches_oracle(shape, dtype):
    _run(_case(shape, dtype=dtype, **SHAPES[shape]))


@pytest.mark.parametrize("index", ["u32", "u64"])
def test_prefill_index_widths(index):
    _run(_case("g4_d128_bs16", index=index, seed=12, **SHAPES["g4_d128_bs16"]))


def test_prefill_prefix_workload_sampled():
    """The 512-sequence prefix-sharing batch at full size (32 groups alias a
    2048-token prefix; three chunks per tail), checked on sampled rows: every
    chunk's first and last row of a spread of sequences plus random rows."""
    w = workloads.prefix()
    rng = np.random.default_rng(0)
    rows = []
    for start, cu in w.chunks:
        seqs = rng.choice(w.num_seqs, 24, replace=False)
        pick = set(int(cu[s]) for s in seqs) | set(int(cu[s + 1]) - 1 for s in seqs)
        pick |= set(rng.choice(int(cu[-1]), 24, replace=False).tolist())
        rows.append(np.array(sorted(pick), dtype=np.int64))
    _run(w, sample_rows=rows)


def _small(seed=21, dtype="bf16"):
    return _case("edge", dtype=dtype, seed=seed, groups=2, group_size=2, prefix_tokens=16,
                 n_chunks=2, num_q_heads=8, num_kv_heads=2, head_dim=64, bs=16, tail_lo=20,
                 tail_hi=150)


def test_prefill_max_q_len_above_need_and_determinism():
    w = _small()
    _, a = _run(w)
    _, b = _run(w, max_q_len=10_000)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_prefill_empty_chunks_and_single_tokens():
    """Sequences with no rows in a chunk, and one-token chunks (the decode case)."""
    w = _small(seed=22)
    B = w.num_seqs
    start = w.context_lens.astype(np.int32) - 1
    counts = np.array([0, 1, 0, 1], dtype=np.int64)[:B]
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(counts)
    # chunk 0 writes each private tail up to the last token (the aliased prefix pages are
    # left as they are: writing them from every sequence of a group would race)
    first = np.full(B, 16, dtype=np.int32)
    cu0 = np.concatenate([[0], np.cumsum(w.context_lens.astype(np.int64) - 1 - 16)])
    w.chunks = [(first, cu0.astype(np.int64)), (start, cu)]
    _run(w)


def _setup_one_chunk(w):
    t = workloads.make_tensors(w, DEV)
    poison_unused(w, t)
    qs = workloads.make_prefill_queries(w, DEV)
    gpu_prefill(w, t, qs)
    return t, qs


def test_prefill_malformed_sequences_get_nan():
    w = _small(seed=23)
    w.chunks = w.chunks[:1]
    t, qs = _setup_one_chunk(w)
    start, cu = w.chunks[0]
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    q = qs[0]
    good = torch.empty_like(q)
    hpkv.hpkv_paged_attention_prefill(q, t.k_cache, t.v_cache, bt, sp,
                                      torch.from_numpy(start).to(DEV),
                                      torch.from_numpy(cu).to(DEV), w.scale, max_chunk_len(cu),
                                      good)
    lens = np.diff(cu)

    def run(start_h, max_q, bt_h=None):
        out = torch.zeros_like(q)
        hpkv.hpkv_paged_attention_prefill(q, t.k_cache, t.v_cache,
                                          bt if bt_h is None else torch.from_numpy(bt_h).to(DEV),
                                          sp, torch.from_numpy(start_h).to(DEV),
                                          torch.from_numpy(cu).to(DEV), w.scale, max_q, out)
        torch.cuda.synchronize()
        return out

    def rows_of(s):
        return slice(int(cu[s]), int(cu[s + 1]))

    def check(out, bad):
        for s in range(w.num_seqs):
            if s in bad:
                assert torch.isnan(out[rows_of(s)].float()).all(), s
            else:
                assert torch.equal(out[rows_of(s)].view(torch.int16),
                                   good[rows_of(s)].view(torch.int16)), s

    # a chunk longer than max_q_len: that sequence is NaN, the others are untouched
    longest = int(np.argmax(lens))
    check(run(start, int(lens[longest]) - 1), {s for s in range(w.num_seqs)
                                              if lens[s] > lens[longest] - 1})
    # a negative start position
    st = start.copy()
    st[1] = -1
    check(run(st, max_chunk_len(cu)), {1})
    # a chunk running past its slice
    st = start.copy()
    st[2] += 10_000
    check(run(st, max_chunk_len(cu)), {2})
    # a page id past the pool in the first page of sequence 3 (shared with its group)
    bth = w.block_table.copy()
    sp_h = w.seq_ptr.astype(np.int64)
    bth[sp_h[3]] = w.num_pages + 7
    out = run(start, max_chunk_len(cu), bth)
    assert torch.isnan(out[rows_of(3)].float()).all()
    for s in range(3):
        assert torch.equal(out[rows_of(s)].view(torch.int16), good[rows_of(s)].view(torch.int16))


def test_prefill_last_row_equals_decode():
    """A chunk's row at position p is the decode of a context of p+1 tokens."""
    w = _small(seed=24)
    w.chunks = w.chunks[:1]
    t, qs = _setup_one_chunk(w)
    start, cu = w.chunks[0]
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    out = torch.empty_like(qs[0])
    hpkv.hpkv_paged_attention_prefill(qs[0], t.k_cache, t.v_cache, bt, sp,
                                      torch.from_numpy(start).to(DEV),
                                      torch.from_numpy(cu).to(DEV), w.scale, max_chunk_len(cu),
                                      out)
    last = torch.from_numpy(cu[1:] - 1).to(DEV)
    ctx = torch.from_numpy((start + np.diff(cu)).astype(np.int32)).to(DEV)
    q_dec = qs[0][last].contiguous()
    dec = torch.empty_like(q_dec)
    mcl = int(ctx.max())
    ws = hpkv.alloc_workspace(q_dec, t.k_cache, mcl)
    hpkv.hpkv_paged_attention_decode(q_dec, t.k_cache, t.v_cache, bt, sp, ctx, w.scale, mcl, ws,
                                     dec)
    torch.cuda.synchronize()
    diff = (out[last].float() - dec.float()).abs().max().item()
    assert diff <= 2e-2, diff

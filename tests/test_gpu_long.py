"""Long contexts on the GPU path against the oracle.

Decode over ~70k-token contexts runs more split-context partitions per
sequence than the reduce kernel's wave has lanes (137 of 512 tokens; 69 of
1024 where a workgroup serves two KV heads on the matrix cores). Prefill chunks
at positions past 4096 and 8192 make a workgroup resolve its keys' pool rows
in several segments. Both are checked against the oracle (prefill on sampled
rows), with unused pool rows poisoned by NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_hpkv_amd as hpkv
import workloads
from paths import (decode_errors, gpu_prefill, host_bits, host_inputs, host_threads,
                   oracle_prefill, poison_unused)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _long_decode_workload(hq, hkv, d=128, bs=16, seed=31):
    rng = np.random.default_rng(seed)
    ctx = np.array([70001, 65536, 33000, 7, 512], dtype=np.int32)
    num_pages, seq_ptr, bt = workloads._random_pool_tables(rng, ctx, bs, "u32")
    return workloads.Workload("long", "bf16", "u32", hq, hkv, d, bs, num_pages, ctx, seq_ptr,
                              bt, d ** -0.5, chunks=workloads._decode_step_chunks(ctx),
                              seed=seed)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2)])  # the VALU and the matrix-core kernels
def test_long_context_decode(hq, hkv):
    w = _long_decode_workload(hq, hkv)
    print(f"[long decode] Hq={hq} Hkv={hkv} ctx={w.context_lens.tolist()}", flush=True)
    t = workloads.make_tensors(w, DEV)
    poison_unused(w, t)
    h = host_inputs(t)
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    ctx = torch.from_numpy(w.context_lens).to(DEV)
    out = torch.empty_like(t.q)
    mcl = w.max_context_len
    ws = hpkv.alloc_workspace(t.q, t.k_cache, mcl)
    assert ws is not None  # split context: partials and the reduce
    hpkv.hpkv_paged_attention_decode(t.q, t.k_cache, t.v_cache, bt, sp, ctx, w.scale, mcl, ws,
                                     out)
    torch.cuda.synchronize()
    _, ref = oracle.paged_attention_decode("bf16", h["q"], h["k_cache"], h["v_cache"],
                                           w.block_table, w.seq_ptr, w.context_lens, w.scale,
                                           host_threads())
    max_err, ratio, finite = decode_errors("bf16", host_bits(out), ref)
    assert finite and ratio <= 1.0, max_err


def test_long_context_decode_fp8_pools():
    w = _long_decode_workload(8, 2)
    print(f"[long decode fp8] ctx={w.context_lens.tolist()}", flush=True)
    t = workloads.make_tensors(w, DEV)
    qt = workloads.make_quant_tensors(w, "fp8", DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    ctx = torch.from_numpy(w.context_lens).to(DEV)
    out = torch.empty_like(t.q)
    mcl = w.max_context_len
    ws = hpkv.alloc_workspace(t.q, qt.k_codes, mcl)
    hpkv.hpkv_paged_attention_decode_quant("fp8", t.q, qt.k_codes, qt.v_codes, qt.k_scale,
                                           qt.k_zero, qt.v_scale, qt.v_zero, bt, sp, ctx,
                                           w.scale, mcl, ws, out)
    torch.cuda.synchronize()
    hs = {n: getattr(qt, n).cpu().numpy() for n in
          ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero")}
    _, ref = oracle.paged_attention_decode_quant(
        "bf16", "fp8", host_bits(t.q), hs["k_codes"], hs["v_codes"], hs["k_scale"],
        hs["k_zero"], hs["v_scale"], hs["v_zero"], w.block_table, w.seq_ptr, w.context_lens,
        w.scale, host_threads())
    max_err, ratio, finite = decode_errors("bf16", host_bits(out), ref)
    assert finite and ratio <= 1.0, max_err


def test_prefill_across_key_segments():
    """Prefixes of 9000 tokens (keys cross 4096 and 8192), chunks of their tails; and
    one whole 5000-token prompt in a single chunk from position 0."""
    w = workloads.chunked_prefill("longpre", "bf16", "u32", 41, groups=2, group_size=2,
                                  prefix_tokens=9008, n_chunks=2, num_q_heads=8,
                                  num_kv_heads=2, head_dim=128, bs=16, tail_lo=100,
                                  tail_hi=300)
    w2 = workloads.chunked_prefill("longpre0", "bf16", "u32", 42, groups=1, group_size=2,
                                   prefix_tokens=0, n_chunks=1, num_q_heads=8, num_kv_heads=2,
                                   head_dim=64, bs=16, tail_lo=4990, tail_hi=5010)
    rng = np.random.default_rng(1)
    for wl in (w, w2):
        print(f"[long prefill] {wl.name} rows={[int(cu[-1]) for _, cu in wl.chunks]}",
              flush=True)
        t = workloads.make_tensors(wl, DEV)
        poison_unused(wl, t)
        qs = workloads.make_prefill_queries(wl, DEV)
        h = host_inputs(t)
        q_bits = [host_bits(q) for q in qs]
        g_out = gpu_prefill(wl, t, qs)
        rows = []
        for start, cu in wl.chunks:
            pick = {int(cu[s]) for s in range(wl.num_seqs)} | \
                   {int(cu[s + 1]) - 1 for s in range(wl.num_seqs)}
            pick |= set(rng.choice(int(cu[-1]), 12, replace=False).tolist())
            rows.append(np.array(sorted(pick), dtype=np.int64))
        o_out = oracle_prefill(wl, h, q_bits, rows)
        for c in range(len(wl.chunks)):
            max_err, ratio, finite = decode_errors(wl.dtype, host_bits(g_out[c])[rows[c]],
                                                   o_out[c])
            assert finite and ratio <= 1.0, (wl.name, c, max_err)

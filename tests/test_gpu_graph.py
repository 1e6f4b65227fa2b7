"""HIP graph capture of the decode step.

A serving loop captures its decode step once and replays it. Every argument of
the fused step, hpkv_paged_attention_decode_step ("Paged KV Cache · AI infra
interview lesson", Step 1 store at p = ctx-1, then Step 2), is a device address
or a host scalar fixed at capture, and the library enqueues no memory fills or
host reads, so the captured step must give the eager step's bits on every
replay. The no-allocation decode (its scratch is a fixed device array) is
captured the same way. Between replays the test changes q on the eager side,
runs the eager step and synchronizes, so each replay is checked against fresh
eager results.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_hpkv_amd as hpkv
import workloads
from paths import host_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match(fn, q, out, replays=4, seed=7):
    g = _capture(fn)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    for i in range(replays):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        out.fill_(float("nan"))
        fn()
        torch.cuda.synchronize()
        expect = host_bits(out).copy()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {i}", flush=True)
        assert host_bits(out).tobytes() == expect.tobytes(), f"replay {i} differs"


@pytest.mark.parametrize("wl", ["gqa", "llama7b"])
def test_fused_step_graph_replays(wl):
    """Matrix-core (GQA) and VALU (MHA) kernels; ordering pass, partitions and reduce."""
    w = workloads.WORKLOADS[wl](batch=48)
    print(f"[graph] {wl} B={w.num_seqs}", flush=True)
    t = workloads.make_tensors(w, DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    ctx = torch.from_numpy(w.context_lens).to(DEV)
    ws = hpkv.alloc_workspace(t.q, t.k_cache, w.max_context_len)
    out = torch.empty_like(t.q)
    slots = torch.empty(w.num_seqs, dtype=torch.int64, device=DEV)

    def step():
        hpkv.hpkv_paged_attention_decode_step(
            t.q, t.new_keys[0], t.new_values[0], t.k_cache, t.v_cache, bt, sp, ctx, w.scale,
            w.max_context_len, ws, out, slots_out=slots)

    _replays_match(step, t.q, out)


def test_noalloc_decode_graph_replays():
    w = workloads.gqa(batch=48)
    t = workloads.make_tensors(w, DEV)
    bt = torch.from_numpy(w.block_table).to(DEV)
    sp = torch.from_numpy(w.seq_ptr).to(DEV)
    ctx = torch.from_numpy(w.context_lens).to(DEV)
    out = torch.empty_like(t.q)

    def step():
        hpkv.hpkv_paged_attention_decode_noalloc(t.q, t.k_cache, t.v_cache, bt, sp, ctx, w.scale,
                                                 w.max_context_len, out)

    _replays_match(step, t.q, out)

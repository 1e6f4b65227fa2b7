"""Runs one step of the paged KV cache path on the GPU library and on the
oracle, from the same seeded inputs, for the parity tests and the smoke check.

A step is: slot mapping of the new tokens (per chunk), the store of their K/V
rows, then decode of every sequence. Inputs come from workloads.py. Pool rows
outside every sequence's context are poisoned with NaN first (the rows that
are in use are listed by the oracle's slot mapping over [0, ctx)), so a kernel
that reads past the context or into an unreferenced page shows NaN.
"""
import os

import numpy as np
import torch

import oracle
import paged_kv_cache_hpkv_amd as hpkv
import workloads

TOL_ABS = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
TOL_REL = {"f32": 1e-5, "f16": 0.0, "bf16": 0.0}


def host_threads():
    return max(1, min(16, os.cpu_count() or 1))


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's storage (bf16 carried as uint16 bit patterns)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def used_slots(w: workloads.Workload) -> np.ndarray:
    B = w.num_seqs
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(w.context_lens.astype(np.int64))
    return oracle.slot_mapping(w.block_table, w.seq_ptr, w.page_size, w.num_pages,
                               np.zeros(B, np.int32), cu)


def poison_unused(w: workloads.Workload, t: workloads.Tensors):
    dev = t.k_cache.device
    mask = torch.ones(w.num_pages * w.page_size, dtype=torch.bool, device=dev)
    mask[torch.from_numpy(used_slots(w)).to(dev)] = False
    for pool in (t.k_cache, t.v_cache):
        pool.view(w.num_pages * w.page_size, -1)[mask] = float("nan")


def host_inputs(t: workloads.Tensors):
    return dict(q=host_bits(t.q), k_cache=host_bits(t.k_cache), v_cache=host_bits(t.v_cache),
                new_keys=[host_bits(x) for x in t.new_keys],
                new_values=[host_bits(x) for x in t.new_values])


def gpu_step(w: workloads.Workload, t: workloads.Tensors, max_context_len=None):
    """Runs slot mapping + store + decode through libhpkv; returns slots and out."""
    dev = t.q.device
    bt = torch.from_numpy(w.block_table).to(dev)
    sp = torch.from_numpy(w.seq_ptr).to(dev)
    ctx = torch.from_numpy(w.context_lens).to(dev)
    slots_out = []
    for c, (start, cu) in enumerate(w.chunks):
        slots = torch.empty(int(cu[-1]), dtype=torch.int64, device=dev)
        hpkv.hpkv_slot_mapping(bt, sp, w.page_size, w.num_pages, torch.from_numpy(start).to(dev),
                               torch.from_numpy(cu).to(dev), slots)
        slots_out.append(slots.cpu().numpy())
        if w.drop_mask is not None and c == 0:
            slots[torch.from_numpy(w.drop_mask).to(dev)] = -1
        hpkv.hpkv_store_kvcache(t.new_keys[c], t.new_values[c], t.k_cache, t.v_cache, slots)
    mcl = w.max_context_len if max_context_len is None else max_context_len
    out = torch.empty_like(t.q)
    ws = hpkv.alloc_workspace(t.q, t.k_cache, mcl)
    hpkv.hpkv_paged_attention_decode(t.q, t.k_cache, t.v_cache, bt, sp, ctx, w.scale, mcl, ws,
                                     out)
    torch.cuda.synchronize(dev)
    return slots_out, out


def oracle_step(w: workloads.Workload, h: dict, threads=None):
    """The same step on the oracle, in place on the host copies `h`."""
    slots_out = []
    for c, (start, cu) in enumerate(w.chunks):
        slots = oracle.slot_mapping(w.block_table, w.seq_ptr, w.page_size, w.num_pages, start, cu)
        slots_out.append(slots.copy())
        if w.drop_mask is not None and c == 0:
            slots[w.drop_mask] = -1
        oracle.store_kvcache(h["new_keys"][c], h["new_values"][c], h["k_cache"], h["v_cache"],
                             slots)
    out, out64 = oracle.paged_attention_decode(w.dtype, h["q"], h["k_cache"], h["v_cache"],
                                               w.block_table, w.seq_ptr, w.context_lens, w.scale,
                                               threads or host_threads())
    return slots_out, out, out64


def decode_errors(dtype, got_bits, ref64):
    """(max abs error, max of error / allowed); fails on non-finite output."""
    got = oracle.widen_dtype(dtype, got_bits)
    err = np.abs(got - ref64)
    allowed = TOL_ABS[dtype] + TOL_REL[dtype] * np.abs(ref64)
    return float(np.nanmax(err)) if err.size else 0.0, \
        float(np.max(err / allowed)) if err.size else 0.0, bool(np.isfinite(got).all())


def check_step(w: workloads.Workload, device="cuda", seed_poison=True, verbose=True):
    """Full parity check of one workload; returns a dict of measured errors."""
    if verbose:
        print(f"[parity] {w.name} {w.dtype} {w.index} B={w.num_seqs} Hq={w.num_q_heads} "
              f"Hkv={w.num_kv_heads} d={w.head_dim} bs={w.page_size} pages={w.num_pages}",
              flush=True)
    t = workloads.make_tensors(w, device)
    if seed_poison:
        poison_unused(w, t)
    h = host_inputs(t)
    g_slots, g_out = gpu_step(w, t)
    o_slots, o_out, o_out64 = oracle_step(w, h)
    for gs, os_ in zip(g_slots, o_slots):
        np.testing.assert_array_equal(gs, os_)  # slot mapping: bit-exact
    for name in ("k_cache", "v_cache"):  # store: whole pools byte-for-byte
        g_pool = host_bits(getattr(t, name))
        assert g_pool.tobytes() == h[name].tobytes(), f"{name} differs after store"
    max_err, worst_ratio, finite = decode_errors(w.dtype, host_bits(g_out), o_out64)
    assert finite, "non-finite decode output"
    assert worst_ratio <= 1.0, f"decode error {max_err} above tolerance"
    return dict(max_err=max_err, worst_ratio=worst_ratio, out=g_out, oracle_out=o_out,
                oracle_out64=o_out64, tensors=t)


def decode_step_workload(w: workloads.Workload, empty_seq=None) -> workloads.Workload:
    """Copy of `w` whose store step is the decode step's: one new token per sequence at
    position ctx-1, none for an empty sequence; `empty_seq` (an index) is set to ctx 0."""
    w2 = workloads.Workload(**{**w.__dict__})
    w2.context_lens = w.context_lens.copy()
    if empty_seq is not None and w2.num_seqs > empty_seq:
        w2.context_lens[empty_seq] = 0
    w2.chunks = workloads._decode_step_chunks(w2.context_lens)
    w2.drop_mask = None
    return w2


def gpu_fused_step(w: workloads.Workload, t: workloads.Tensors):
    """hpkv_paged_attention_decode_step on the decode-step workload `w` (one new row per
    non-empty sequence in t.new_keys[0]); returns (slots [B], out)."""
    dev = t.q.device
    B = w.num_seqs
    nk = torch.zeros(B, w.num_kv_heads, w.head_dim, dtype=t.q.dtype, device=dev)
    nv = torch.zeros_like(nk)
    has = torch.from_numpy(w.context_lens > 0).to(dev)
    nk[has] = t.new_keys[0]
    nv[has] = t.new_values[0]
    out = torch.empty_like(t.q)
    slots = torch.full((B,), 7, dtype=torch.int64, device=dev)
    ws = hpkv.alloc_workspace(t.q, t.k_cache, w.max_context_len)
    hpkv.hpkv_paged_attention_decode_step(
        t.q, nk, nv, t.k_cache, t.v_cache, torch.from_numpy(w.block_table).to(dev),
        torch.from_numpy(w.seq_ptr).to(dev), torch.from_numpy(w.context_lens).to(dev), w.scale,
        w.max_context_len, ws, out, slots_out=slots)
    torch.cuda.synchronize(dev)
    return slots.cpu().numpy(), out


def check_fused_step(w: workloads.Workload, device="cuda", empty_seq=1, verbose=True):
    """The fused store-and-decode entry point against the oracle's slot mapping (position
    ctx-1), store and decode on the same inputs: slots and both pools bit-exact, output within
    tolerance; an empty sequence gets slot -1 and zeros."""
    w = decode_step_workload(w, empty_seq)
    if verbose:
        print(f"[parity fused] {w.name} {w.dtype} {w.index} B={w.num_seqs} Hq={w.num_q_heads} "
              f"Hkv={w.num_kv_heads} d={w.head_dim} bs={w.page_size}", flush=True)
    t = workloads.make_tensors(w, device)
    poison_unused(w, t)
    h = host_inputs(t)
    g_slots, g_out = gpu_fused_step(w, t)
    o_slots, _, o_out64 = oracle_step(w, h)
    want = np.full(w.num_seqs, -1, dtype=np.int64)
    want[w.context_lens > 0] = o_slots[0]
    np.testing.assert_array_equal(g_slots, want)
    for name in ("k_cache", "v_cache"):
        assert host_bits(getattr(t, name)).tobytes() == h[name].tobytes(), \
            f"{name} differs after the fused store"
    max_err, worst_ratio, finite = decode_errors(w.dtype, host_bits(g_out), o_out64)
    assert finite, "non-finite fused decode output"
    assert worst_ratio <= 1.0, f"fused decode error {max_err} above tolerance"
    if empty_seq is not None and w.num_seqs > empty_seq:
        assert not host_bits(g_out)[empty_seq].any(), "empty sequence must decode to zeros"
    return dict(max_err=max_err, worst_ratio=worst_ratio)


# ------------------------------------------------------------ chunked prefill

def max_chunk_len(cu) -> int:
    cu = np.asarray(cu, dtype=np.int64)
    return int(np.diff(cu).max()) if len(cu) > 1 else 0


def gpu_prefill(w: workloads.Workload, t: workloads.Tensors, queries, max_q_len=None):
    """Per chunk through libhpkv: slot mapping + store of the chunk's K/V rows, then
    causal prefill attention of the chunk's queries. Returns the outputs per chunk."""
    dev = t.k_cache.device
    bt = torch.from_numpy(w.block_table).to(dev)
    sp = torch.from_numpy(w.seq_ptr).to(dev)
    outs = []
    for c, (start, cu) in enumerate(w.chunks):
        start_t = torch.from_numpy(start).to(dev)
        cu_t = torch.from_numpy(cu).to(dev)
        slots = torch.empty(int(cu[-1]), dtype=torch.int64, device=dev)
        hpkv.hpkv_slot_mapping(bt, sp, w.page_size, w.num_pages, start_t, cu_t, slots)
        hpkv.hpkv_store_kvcache(t.new_keys[c], t.new_values[c], t.k_cache, t.v_cache, slots)
        out = torch.empty_like(queries[c])
        mq = max_chunk_len(cu) if max_q_len is None else max_q_len
        hpkv.hpkv_paged_attention_prefill(queries[c], t.k_cache, t.v_cache, bt, sp, start_t, cu_t,
                                          w.scale, max(mq, 1), out)
        outs.append(out)
    torch.cuda.synchronize(dev)
    return outs


def oracle_prefill_rows(w: workloads.Workload, h: dict, q_bits, start, cu, rows):
    """Oracle prefill outputs (float64 [len(rows), Hq, d]) of the given query rows of a chunk,
    computed one sequence position at a time (pools in `h` already hold the chunk)."""
    start = np.asarray(start, dtype=np.int32)
    cu = np.asarray(cu, dtype=np.int64)
    B = len(start)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    out = np.empty((len(rows), w.num_q_heads, w.head_dim), dtype=np.float64)
    pending = list(range(len(rows)))
    while pending:  # one oracle call per round, each sequence at most once per round
        taken, rest = {}, []
        for k in pending:
            if seq_of[k] in taken:
                rest.append(k)
            else:
                taken[seq_of[k]] = k
        order = sorted(taken.items())
        q_start = np.zeros(B, dtype=np.int32)
        counts = np.zeros(B, dtype=np.int64)
        for s, k in order:
            q_start[s] = start[s] + (rows[k] - cu[s])
            counts[s] = 1
        cu_s = np.zeros(B + 1, dtype=np.int64)
        cu_s[1:] = np.cumsum(counts)
        q_sel = np.ascontiguousarray(q_bits[[rows[k] for _, k in order]])
        _, o64 = oracle.paged_attention_prefill(w.dtype, q_sel, h["k_cache"], h["v_cache"],
                                                w.block_table, w.seq_ptr, q_start, cu_s, w.scale)
        for j, (_, k) in enumerate(order):
            out[k] = o64[j]
        pending = rest
    return out


def oracle_prefill(w: workloads.Workload, h: dict, q_bits_list, sample_rows=None):
    """The prefill step on the oracle, in place on the host pools of `h`: per chunk, slot
    mapping + store, then prefill of all its rows (or of sample_rows[c])."""
    outs = []
    for c, (start, cu) in enumerate(w.chunks):
        slots = oracle.slot_mapping(w.block_table, w.seq_ptr, w.page_size, w.num_pages, start, cu)
        oracle.store_kvcache(h["new_keys"][c], h["new_values"][c], h["k_cache"], h["v_cache"],
                             slots)
        if sample_rows is None:
            _, o64 = oracle.paged_attention_prefill(w.dtype, q_bits_list[c], h["k_cache"],
                                                    h["v_cache"], w.block_table, w.seq_ptr,
                                                    start, cu, w.scale)
        else:
            o64 = oracle_prefill_rows(w, h, q_bits_list[c], start, cu, sample_rows[c])
        outs.append(o64)
    return outs

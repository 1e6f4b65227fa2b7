"""GPU parity over seeded random shapes.

Each case draws a batch size, head counts, head size, page size, element and
index type and a length mix from one seed, then runs the full step (slot
mapping, store, decode) against the oracle with NaN-poisoned unused pool rows;
the quantized cases run the int8 / fp8 decode against the quantized oracle,
with NaN factors on the pages no sequence references; the prefill cases run
chunked prefill (slot mapping, store, causal attention per chunk) over groups
that alias a prefix, with chunk cuts inside pages.
The draws cover the decode's launch plans: one, two or four KV heads per
workgroup, 512- or 1024-token partitions, grids above and below the size at
which partitions are dispatched longest first, ragged tails and pages that do
not divide the partitions.
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

SEEDS = list(range(101, 141))
QSEEDS = list(range(201, 213))


def _draw(seed):
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([1, 7, 16, 64]))
    dtype = str(rng.choice(["bf16", "f16"]))
    index = str(rng.choice(["u32", "u64"]))
    B = int(rng.integers(1, 160))
    top = int(rng.choice([600, 3000, 6000]))
    ctx = rng.integers(1, top + 1, B).astype(np.int32)
    ctx[rng.random(B) < 0.1] = top  # some sequences at the longest length
    num_pages, seq_ptr, bt = workloads._random_pool_tables(rng, ctx, bs, index)
    return workloads.Workload(f"sweep{seed}", dtype, index, hkv * group, hkv, d, bs, num_pages,
                              ctx, seq_ptr, bt, d ** -0.5,
                              chunks=workloads._decode_step_chunks(ctx), seed=seed)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shape_step(seed):
    w = _draw(seed)
    print(f"[sweep] seed={seed} {w.dtype} {w.index} B={w.num_seqs} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} d={w.head_dim} bs={w.page_size} max_ctx={w.max_context_len}",
          flush=True)
    r = check_step(w)
    assert r["worst_ratio"] <= 1.0


@pytest.mark.parametrize("seed", QSEEDS)
def test_random_shape_quant_decode(seed):
    w = _draw(seed)
    kv = "fp8" if seed % 2 else "i8"
    print(f"[sweep quant] seed={seed} {kv} {w.dtype} B={w.num_seqs} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} d={w.head_dim} bs={w.page_size} max_ctx={w.max_context_len}",
          flush=True)
    t = workloads.make_tensors(w, DEV)
    qt = workloads.make_quant_tensors(w, kv, DEV)
    used = torch.zeros(w.num_pages * w.page_size, dtype=torch.bool)
    used[torch.from_numpy(used_slots(w))] = True
    pages = used.view(w.num_pages, w.page_size).any(1).to(DEV)
    for sc in (qt.k_scale, qt.v_scale):
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


PSEEDS = list(range(301, 313))


def _draw_prefill(seed):
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 4]))
    group = int(rng.choice([1, 2, 3, 4, 8]))
    d = int(rng.choice([32, 64, 128, 256]))
    bs = int(rng.choice([4, 12, 16, 64]))
    prefix_pages = int(rng.integers(0, 6))
    return workloads.chunked_prefill(
        f"psweep{seed}", str(rng.choice(["bf16", "f16"])), str(rng.choice(["u32", "u64"])), seed,
        groups=int(rng.integers(1, 4)), group_size=int(rng.integers(1, 4)),
        prefix_tokens=prefix_pages * bs, n_chunks=int(rng.integers(1, 4)),
        num_q_heads=hkv * group, num_kv_heads=hkv, head_dim=d, bs=bs,
        tail_lo=int(rng.integers(1, 50)), tail_hi=int(rng.integers(50, 500)))


@pytest.mark.parametrize("seed", PSEEDS)
def test_random_shape_prefill(seed):
    from test_gpu_prefill import _run
    w = _draw_prefill(seed)
    _run(w)

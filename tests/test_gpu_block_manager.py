"""The host block manager as a table generator for the GPU path: sequences
admitted with shared prompt prefixes (aliased pages), then decode steps that
append one token each. The K/V rows of every step go to the slots the manager
returns; those slots must equal the library's slot mapping over the exported
tables, and decode over those tables must match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_hpkv_amd as hpkv
from paths import decode_errors, host_bits, host_threads

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("index", ["u32", "u64"])
def test_block_manager_tables_drive_decode(index):
    rng = np.random.default_rng(11)
    bs, num_pages, Hq, Hkv, d = 16, 512, 8, 2, 128
    bm = hpkv.BlockManager(num_pages, bs)
    prompts = [list(rng.integers(0, 1000, 200)) for _ in range(3)]
    ids = []
    for g, p in enumerate(prompts):
        for j in range(4):  # four sequences per prompt, each with its own tail
            sid = 10 * g + j
            bm.admit(sid, p + list(rng.integers(0, 1000, int(rng.integers(1, 60)))))
            ids.append(sid)
    assert bm.check() == hpkv.OK
    gen = torch.Generator(device=DEV).manual_seed(5)
    kc = torch.randn(num_pages, bs, Hkv, d, generator=gen, device=DEV, dtype=torch.bfloat16)
    vc = torch.randn(num_pages, bs, Hkv, d, generator=gen, device=DEV, dtype=torch.bfloat16)
    for step in range(3):
        slots = np.array([bm.append(s, int(rng.integers(0, 1000))) for s in ids], np.int64)
        assert bm.check() == hpkv.OK
        bt, sp, ctx = bm.export(ids, index)
        # the library's slot mapping of position ctx-1 gives the manager's slots
        g_slots = torch.empty(len(ids), dtype=torch.int64, device=DEV)
        hpkv.hpkv_slot_mapping(torch.from_numpy(bt).to(DEV), torch.from_numpy(sp).to(DEV), bs,
                               bm.num_pages,
                               torch.from_numpy(ctx - 1).to(DEV),
                               torch.arange(len(ids) + 1, device=DEV), g_slots)
        assert np.array_equal(g_slots.cpu().numpy(), slots)
        nk = torch.randn(len(ids), Hkv, d, generator=gen, device=DEV, dtype=torch.bfloat16)
        nv = torch.randn(len(ids), Hkv, d, generator=gen, device=DEV, dtype=torch.bfloat16)
        hpkv.hpkv_store_kvcache(nk, nv, kc, vc, g_slots)
        q = torch.randn(len(ids), Hq, d, generator=gen, device=DEV, dtype=torch.bfloat16)
        out = torch.empty_like(q)
        mcl = int(ctx.max())
        ws = hpkv.alloc_workspace(q, kc, mcl)
        hpkv.hpkv_paged_attention_decode(q, kc, vc, torch.from_numpy(bt).to(DEV),
                                         torch.from_numpy(sp).to(DEV),
                                         torch.from_numpy(ctx).to(DEV), d ** -0.5, mcl, ws, out)
        torch.cuda.synchronize()
        _, ref = oracle.paged_attention_decode("bf16", host_bits(q), host_bits(kc), host_bits(vc),
                                               bt, sp, ctx, d ** -0.5, host_threads())
        max_err, ratio, finite = decode_errors("bf16", host_bits(out), ref)
        assert finite and ratio <= 1.0, (step, max_err)
    st = bm.stats()
    # 3 prompts x 12 shared full pages, plus private pages per sequence
    assert st["allocated"] < 12 * len(ids)

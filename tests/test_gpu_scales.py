"""GPU parity at softmax scales other than 1/sqrt(d), through the C ABI against the
oracle: negative (the kernels fold the sign into q), zero (uniform weights), large
(peaked weights: the running max grows often, so the rescale of the accumulators runs
on many tiles) and tiny. Covers the full decode step on the VALU kernel (MHA, and fp32)
and on the matrix cores (GQA), the quantized decode (int8 and fp8, both kernels) and
chunked prefill (bf16 and f16). The scale enters every score as written in
"Paged KV Cache · AI infra interview lesson", section "Step 2: paged_attention_decode".
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_hpkv_amd as hpkv
import workloads
from paths import check_step, decode_errors, host_bits, host_threads, used_slots

pytestmark = pytest.mark.gpu
DEV = "cuda"

# scale as a multiple of 1/sqrt(d), or an absolute value
SCALES = {"neg": ("rel", -1.0), "zero": ("abs", 0.0), "large": ("abs", 3.0),
          "tiny": ("abs", 1e-3)}


def _scale(kind, d):
    how, v = SCALES[kind]
    return v * d ** -0.5 if how == "rel" else v


def _decode_workload(name, dtype, hq, hkv, d, scale, seed):
    """24 sequences, contexts up to 2500 tokens (several partitions), 16-token pages."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, 2501, 24).astype(np.int32)
    ctx[0] = 2500
    num_pages, seq_ptr, bt = workloads._random_pool_tables(rng, ctx, 16, "u32")
    return workloads.Workload(name, dtype, "u32", hq, hkv, d, 16, num_pages, ctx, seq_ptr, bt,
                              scale, chunks=workloads._decode_step_chunks(ctx), seed=seed)


DECODE_SHAPES = {"mha_bf16": ("bf16", 8, 8, 128), "gqa_bf16": ("bf16", 16, 4, 128),
                 "gqa_f32": ("f32", 4, 2, 64)}


@pytest.mark.parametrize("kind", sorted(SCALES))
@pytest.mark.parametrize("shape", sorted(DECODE_SHAPES))
def test_decode_step_scales(shape, kind):
    dtype, hq, hkv, d = DECODE_SHAPES[shape]
    w = _decode_workload(f"scale_{shape}_{kind}", dtype, hq, hkv, d, _scale(kind, d), 401)
    print(f"[scales decode] {shape} {kind} scale={w.scale:g}", flush=True)
    r = check_step(w)
    assert r["worst_ratio"] <= 1.0


QUANT_SHAPES = {"gqa": (16, 4), "g2": (16, 8), "mha": (8, 8)}


def _quant_decode_check(w, kv, qmul=1.0, spread=None):
    t = workloads.make_tensors(w, DEV)
    if qmul != 1.0:  # a power of two: exact in bf16
        t.q.mul_(qmul)
    qt = workloads.make_quant_tensors(w, kv, DEV)
    if spread is not None:  # per-page scales 2^-u, u uniform in the given ranges
        g = torch.Generator(device="cpu")
        g.manual_seed(405)
        for sc, (lo, hi) in ((qt.k_scale, spread[0]), (qt.v_scale, spread[1])):
            u = lo + (hi - lo) * torch.rand(sc.shape, generator=g)
            sc.copy_(torch.exp2(-u).to(sc.device))
    used = torch.zeros(w.num_pages * w.page_size, dtype=torch.bool)
    used[torch.from_numpy(used_slots(w))] = True
    pages = used.view(w.num_pages, w.page_size).any(1).to(DEV)
    for sc in (qt.k_scale, qt.v_scale):  # pages no sequence references: NaN factors
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


@pytest.mark.parametrize("kind", sorted(SCALES))
@pytest.mark.parametrize("kv", ["fp8", "i8"])
@pytest.mark.parametrize("shape", sorted(QUANT_SHAPES))
def test_quant_decode_scales(shape, kv, kind):
    hq, hkv = QUANT_SHAPES[shape]
    w = _decode_workload(f"qscale_{shape}_{kind}", "bf16", hq, hkv, 128, _scale(kind, 128), 402)
    print(f"[scales quant] {shape} {kv} {kind} scale={w.scale:g}", flush=True)
    _quant_decode_check(w, kv)


@pytest.mark.parametrize("qmul", [2.0 ** 24, 2.0 ** -24])
@pytest.mark.parametrize("kv", ["fp8", "i8"])
@pytest.mark.parametrize("shape", sorted(QUANT_SHAPES))
def test_quant_decode_query_magnitudes(shape, kv, qmul):
    """Queries far outside f16's range (the VALU kernel takes int8 products in f16 after
    scaling a bf16 q by a power of two per head), with the scale divided by the same
    factor so the weights stay those of an ordinary batch."""
    hq, hkv = QUANT_SHAPES[shape]
    w = _decode_workload(f"qmag_{shape}", "bf16", hq, hkv, 128, 128 ** -0.5 / qmul, 404)
    print(f"[q magnitude quant] {shape} {kv} q x {qmul:g}", flush=True)
    _quant_decode_check(w, kv, qmul)


# exponent ranges of the K and V page scales: V values stay within a few units, so the
# 16-bit output rounding stays far inside the tolerance
SPREAD = {"fp8": ((4.0, 12.0), (8.0, 20.0)), "i8": ((4.0, 12.0), (6.0, 20.0))}


@pytest.mark.parametrize("kv", ["fp8", "i8"])
@pytest.mark.parametrize("shape", sorted(QUANT_SHAPES))
def test_quant_decode_page_scale_spread(shape, kv):
    """Page scales that differ by up to 2^12 between the pages one partition reads (the
    VALU kernel pairs rows of different pages in one v_dot2 with fp8 codes, each with its
    own weight times V scale), against the oracle's per-page dequantization."""
    hq, hkv = QUANT_SHAPES[shape]
    w = _decode_workload(f"qspread_{shape}", "bf16", hq, hkv, 128, 128 ** -0.5, 406)
    print(f"[page scale spread quant] {shape} {kv}", flush=True)
    _quant_decode_check(w, kv, spread=SPREAD[kv])


@pytest.mark.parametrize("kind", sorted(SCALES))
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_scales(dtype, kind):
    from test_gpu_prefill import _run
    w = workloads.chunked_prefill(f"pscale_{dtype}_{kind}", dtype, "u32", 403, groups=2,
                                  group_size=2, prefix_tokens=32, n_chunks=2, num_q_heads=8,
                                  num_kv_heads=2, head_dim=128, bs=16, tail_lo=20, tail_hi=200)
    w = dataclasses.replace(w, scale=_scale(kind, 128))
    print(f"[scales prefill] {dtype} {kind} scale={w.scale:g}", flush=True)
    _run(w)

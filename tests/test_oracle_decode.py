"""Pins of the oracle's paged decode attention.

"Paged KV Cache · AI infra interview lesson", Step 2: the paged result must
equal softmax attention over the same K/V stored contiguously; the page checks
it against torch's scaled_dot_product_attention on pools pre-filled with
garbage, for bs in {4, 16, 256} and lengths [1, bs, 2bs+3]. Here the oracle's
paged decode is compared with (a) its own dense routine, (b) torch's SDPA in
float64 (an independent library implementation), plus closed forms (ctx=1
gives v_0; q=0 gives mean(V)), the consecutive GQA grouping of the same Step
(query head h reads KV head h // (Hq/Hkv)), invariance under a permutation of
physical pages, u32 == u64 tables, ctx=0 and NaN garbage outside the context.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def _build_case(bs, dtype="f32", lens=None, Hq=4, Hkv=2, d=8, nb=12, seed=0, index=np.uint32):
    """Step 2's test layout: garbage pools, pages popped from a permutation."""
    g = torch.Generator().manual_seed(seed)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    lens = lens or [1, bs, 2 * bs + 3]
    k_cache = torch.randn(nb, bs, Hkv, d, generator=g).to(tdt)
    v_cache = torch.randn(nb, bs, Hkv, d, generator=g).to(tdt)
    free = torch.randperm(nb, generator=g).tolist()
    tables, Ks, Vs = [], [], []
    for L in lens:
        bt = [free.pop() for _ in range((L + bs - 1) // bs)]
        K = torch.randn(L, Hkv, d, generator=g).to(tdt)
        V = torch.randn(L, Hkv, d, generator=g).to(tdt)
        for p in range(L):
            k_cache[bt[p // bs], p % bs] = K[p]
            v_cache[bt[p // bs], p % bs] = V[p]
        tables.append(bt)
        Ks.append(K)
        Vs.append(V)
    sp = np.zeros(len(lens) + 1, dtype=np.int64)
    sp[1:] = np.cumsum([len(t) for t in tables])
    flat = np.array([p for t in tables for p in t], dtype=np.int64)
    q = torch.randn(len(lens), Hq, d, generator=g).to(tdt)
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, tables=tables, Ks=Ks, Vs=Vs,
                seq_ptr=sp.astype(index), block_table=flat.astype(index),
                ctx=np.array(lens, dtype=np.int32), scale=d ** -0.5, dtype=dtype)


def _paged(c, **over):
    c = {**c, **over}
    return oracle.paged_attention_decode(c["dtype"], _bits(c["q"]), _bits(c["k_cache"]),
                                         _bits(c["v_cache"]), c["block_table"], c["seq_ptr"],
                                         c["ctx"], c["scale"])


def _sdpa64(q, K, V, scale):
    Hq, Hkv = q.shape[0], K.shape[1]
    Kr = K.double().repeat_interleave(Hq // Hkv, 1).transpose(0, 1).contiguous()
    Vr = V.double().repeat_interleave(Hq // Hkv, 1).transpose(0, 1).contiguous()
    return F.scaled_dot_product_attention(q.double()[:, None], Kr, Vr, scale=scale)[:, 0].numpy()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("bs", [4, 16, 256])
def test_paged_equals_dense_and_sdpa(bs, dtype):
    c = _build_case(bs, dtype, seed=bs)
    out, out64 = _paged(c)
    for b in range(len(c["ctx"])):
        dense = oracle.dense_attention(dtype, _bits(c["q"][b]), _bits(c["Ks"][b]),
                                       _bits(c["Vs"][b]), c["scale"])
        ref = _sdpa64(c["q"][b], c["Ks"][b], c["Vs"][b], c["scale"])
        np.testing.assert_allclose(out64[b], dense, rtol=0, atol=1e-12)
        np.testing.assert_allclose(out64[b], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dense, ref, rtol=1e-12, atol=1e-12)
    # the stored output is the double result rounded once to the storage type
    assert out.tobytes() == oracle.round_to_dtype(dtype, out64).tobytes()


def test_gqa_mapping_is_consecutive():
    """Hq=4, Hkv=2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1."""
    bs, Hq, Hkv, d = 4, 4, 2, 8
    c = _build_case(bs, "f32", lens=[5], Hq=Hq, Hkv=Hkv, d=d, seed=3)
    v = c["v_cache"].clone()
    v[..., 0, :] = 1.0
    v[..., 1, :] = -1.0
    _, out64 = _paged(c, v_cache=v)
    np.testing.assert_array_equal(out64[0, 0:2], np.ones((2, d)))
    np.testing.assert_array_equal(out64[0, 2:4], -np.ones((2, d)))


def test_mha_case_matches_sdpa_without_grouping():
    c = _build_case(16, "f32", lens=[3, 16, 40], Hq=2, Hkv=2, d=16, nb=8, seed=9)
    _, out64 = _paged(c)
    for b in range(3):
        K = c["Ks"][b].double().transpose(0, 1).contiguous()
        V = c["Vs"][b].double().transpose(0, 1).contiguous()
        ref = F.scaled_dot_product_attention(c["q"][b].double()[:, None], K, V,
                                             scale=c["scale"])[:, 0].numpy()
        np.testing.assert_allclose(out64[b], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_closed_forms(dtype):
    c = _build_case(4, dtype, lens=[1, 7, 9], seed=5)
    out, out64 = _paged(c)
    # one token: the softmax weight is exactly 1, so the output is v_0 bit for bit
    v0 = c["Vs"][0][0]
    np.testing.assert_array_equal(out64[0], np.repeat(v0.double().numpy(), 2, axis=0))
    assert out[0].tobytes() == _bits(v0.repeat_interleave(2, 0)).tobytes()
    # zero query (and zero scale): uniform weights, the output is the mean of V
    zq = torch.zeros_like(c["q"])
    _, z64 = _paged(c, q=zq)
    _, s64 = _paged(c, scale=0.0)
    for b in range(3):
        mean = c["Vs"][b].double().mean(0).repeat_interleave(2, 0).numpy()
        np.testing.assert_allclose(z64[b], mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(s64[b], mean, rtol=0, atol=1e-13)


def test_zero_length_context_gives_zeros():
    c = _build_case(4, "f32", lens=[3, 6], seed=2)
    ctx = c["ctx"].copy()
    ctx[0] = 0
    _, out64 = _paged(c, ctx=ctx)
    np.testing.assert_array_equal(out64[0], 0.0)
    assert np.all(np.isfinite(out64[1]))


def test_nan_garbage_outside_context_never_reaches_output():
    c = _build_case(4, "f32", lens=[2, 5, 11], seed=4)
    _, ref = _paged(c)
    used = set()
    for t, L in zip(c["tables"], c["ctx"]):
        for p in range(L):
            used.add((t[p // 4], p % 4))
    k, v = c["k_cache"].clone(), c["v_cache"].clone()
    for page in range(k.shape[0]):
        for r in range(4):
            if (page, r) not in used:
                k[page, r] = float("nan")
                v[page, r] = float("nan")
    _, got = _paged(c, k_cache=k, v_cache=v)
    np.testing.assert_array_equal(got, ref)


def test_page_permutation_invariance_and_index_width():
    c = _build_case(4, "bf16", lens=[3, 9, 12], seed=8, nb=12)
    _, ref = _paged(c)
    perm = torch.randperm(12, generator=torch.Generator().manual_seed(1))
    inv = torch.argsort(perm)
    # new page i holds old page perm[i]; old page id p is now inv[p]
    k2, v2 = c["k_cache"][perm].contiguous(), c["v_cache"][perm].contiguous()
    bt2 = inv.numpy()[c["block_table"].astype(np.int64)].astype(np.uint32)
    _, got = _paged(c, k_cache=k2, v_cache=v2, block_table=bt2)
    np.testing.assert_array_equal(got, ref)
    _, got64 = _paged(c, block_table=c["block_table"].astype(np.uint64),
                      seq_ptr=c["seq_ptr"].astype(np.uint64))
    np.testing.assert_array_equal(got64, ref)


def test_extra_pages_in_slice_are_ignored_and_overlong_ctx_refused():
    c = _build_case(4, "f32", lens=[5], seed=6)
    _, ref = _paged(c)
    bt = np.concatenate([c["block_table"], np.array([11], dtype=np.uint32)])
    sp = np.array([0, len(bt)], dtype=np.uint32)
    _, got = _paged(c, block_table=bt, seq_ptr=sp)
    np.testing.assert_array_equal(got, ref)
    with pytest.raises(ValueError):
        _paged(c, ctx=np.array([9], dtype=np.int32))  # 2 pages of 4 hold at most 8 tokens

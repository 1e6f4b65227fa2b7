"""Pins of the oracle's causal chunked-prefill attention over the paged cache.

"Paged KV Cache · AI infra interview lesson", Step 1: a prefill chunk may start
part-way into a page (prefix hit / second half of a chunked prefill); its
queries attend causally to the sequence's earlier tokens. Pinned to torch's
scaled_dot_product_attention in float64 with an explicit causal mask aligned to
the chunk's positions (an independent library implementation) over K/V stored
contiguously, to the decode oracle for one-token chunks, to the closed form
at position 0, and to the dense result being independent of how the chunk is
split.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().numpy()


def _case(dtype="f32", bs=4, lens=(7, 13, 3), Hq=4, Hkv=2, d=8, seed=0):
    g = torch.Generator().manual_seed(seed)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    nb = sum(-(-L // bs) for L in lens) + 3
    kc = torch.randn(nb, bs, Hkv, d, generator=g).to(tdt)
    vc = torch.randn(nb, bs, Hkv, d, generator=g).to(tdt)
    free = torch.randperm(nb, generator=g).tolist()
    tables, Ks, Vs = [], [], []
    for L in lens:
        bt = [free.pop() for _ in range(-(-L // bs))]
        K = torch.randn(L, Hkv, d, generator=g).to(tdt)
        V = torch.randn(L, Hkv, d, generator=g).to(tdt)
        for p in range(L):
            kc[bt[p // bs], p % bs] = K[p]
            vc[bt[p // bs], p % bs] = V[p]
        tables.append(bt)
        Ks.append(K)
        Vs.append(V)
    sp = np.zeros(len(lens) + 1, dtype=np.int64)
    sp[1:] = np.cumsum([len(t) for t in tables])
    return dict(kc=kc, vc=vc, Ks=Ks, Vs=Vs, tables=tables, sp=sp.astype(np.uint32),
                bt=np.array([p for t in tables for p in t], dtype=np.uint32), lens=lens,
                Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, tdt=tdt, g=g, scale=d ** -0.5)


def _chunk(c, starts, counts):
    cu = np.zeros(len(counts) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(counts)
    q = torch.randn(int(cu[-1]), c["Hq"], c["d"], generator=c["g"]).to(c["tdt"])
    return q, np.array(starts, dtype=np.int32), cu


def _sdpa_causal(q, K, V, start, scale):
    """Chunk queries at positions start.. over keys 0..start+n-1, float64."""
    n, Hq = q.shape[0], q.shape[1]
    L, Hkv = K.shape[0], K.shape[1]
    Kr = K.double().repeat_interleave(Hq // Hkv, 1).transpose(0, 1).contiguous()  # [Hq, L, d]
    Vr = V.double().repeat_interleave(Hq // Hkv, 1).transpose(0, 1).contiguous()
    qp = torch.arange(start, start + n)[:, None]
    mask = torch.arange(L)[None, :] <= qp                                           # [n, L]
    out = F.scaled_dot_product_attention(q.double().transpose(0, 1), Kr[:, :start + n],
                                         Vr[:, :start + n], attn_mask=mask[:, :start + n],
                                         scale=scale)
    return out.transpose(0, 1).numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [4, 16])
def test_prefill_matches_causal_sdpa(dtype, bs):
    c = _case(dtype, bs=bs, lens=(7, 2 * bs + 5, 3), seed=bs)
    # chunks: a full prefill, a chunk starting mid-page, a single token at the end
    starts, counts = [0, bs // 2 + 1, 2], [7, bs + 3, 1]
    q, qs, cu = _chunk(c, starts, counts)
    out, out64 = oracle.paged_attention_prefill(dtype, _bits(q), _bits(c["kc"]), _bits(c["vc"]),
                                                c["bt"], c["sp"], qs, cu, c["scale"])
    for s in range(3):
        ref = _sdpa_causal(q[cu[s]:cu[s + 1]], c["Ks"][s], c["Vs"][s], starts[s], c["scale"])
        np.testing.assert_allclose(out64[cu[s]:cu[s + 1]], ref, rtol=1e-12, atol=1e-12)
    assert out.tobytes() == oracle.round_to_dtype(dtype, out64).tobytes()


def test_single_token_chunks_equal_decode_and_position_zero_is_v0():
    c = _case("f32", bs=4, lens=(9, 5), seed=3)
    q, qs, cu = _chunk(c, [8, 4], [1, 1])   # the last token of each sequence
    _, pre = oracle.paged_attention_prefill("f32", _bits(q), _bits(c["kc"]), _bits(c["vc"]),
                                            c["bt"], c["sp"], qs, cu, c["scale"])
    _, dec = oracle.paged_attention_decode("f32", _bits(q), _bits(c["kc"]), _bits(c["vc"]),
                                           c["bt"], c["sp"], np.array([9, 5], np.int32),
                                           c["scale"])
    np.testing.assert_array_equal(pre, dec)
    q0, qs0, cu0 = _chunk(c, [0, 0], [1, 1])
    _, p0 = oracle.paged_attention_prefill("f32", _bits(q0), _bits(c["kc"]), _bits(c["vc"]),
                                           c["bt"], c["sp"], qs0, cu0, c["scale"])
    for s in range(2):
        np.testing.assert_array_equal(p0[s], c["Vs"][s][0].double().repeat_interleave(2, 0))


def test_chunk_split_does_not_change_results():
    c = _case("f32", bs=4, lens=(11,), seed=5)
    q, _, _ = _chunk(c, [0], [11])
    one = oracle.paged_attention_prefill("f32", _bits(q), _bits(c["kc"]), _bits(c["vc"]), c["bt"],
                                         c["sp"], np.array([0], np.int32),
                                         np.array([0, 11]), c["scale"])[1]
    parts = []
    for a, b in [(0, 3), (3, 9), (9, 11)]:
        parts.append(oracle.paged_attention_prefill(
            "f32", _bits(q[a:b]), _bits(c["kc"]), _bits(c["vc"]), c["bt"], c["sp"],
            np.array([a], np.int32), np.array([0, b - a]), c["scale"])[1])
    np.testing.assert_array_equal(np.concatenate(parts), one)


def test_prefill_refuses_positions_past_the_slice():
    c = _case("f32", bs=4, lens=(5,), seed=1)
    q, qs, cu = _chunk(c, [6], [3])          # positions 6..8 need 9 tokens; 2 pages hold 8
    with pytest.raises(ValueError):
        oracle.paged_attention_prefill("f32", _bits(q), _bits(c["kc"]), _bits(c["vc"]), c["bt"],
                                       c["sp"], qs, cu, c["scale"])

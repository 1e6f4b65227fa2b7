"""Pins of the oracle's quantized pools ("Block-Paged KV Cache", section
"Quantization compatibility": per-block-affine quantization along the paged
axis with one block per page, so each physical page carries its own scales).

Reading (the dequantization formula is not on the pages): int8 or OCP fp8
E4M3 ("e4m3fn") codes; per (page, KV head) an fp32 scale and zero point for K
and for V; a code q stands for scale * (value(q) - zero); the store quantizes
t = x / scale + zero (fp32) to the nearest code, ties to even, saturating.

Pins: torch's float8_e4m3fn type (an independent library implementation of the
OCP format) for decoding and in-range rounding; numpy rint for int8; printed
anchors of the format; the plain decode oracle on exactly representable
dequantized pools; brute-force numpy softmax on a tiny case.
"""
import numpy as np
import pytest
import torch

import oracle


def test_fp8_decode_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.fp8_e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    # anchors of the format: max 448, smallest normal 2^-6, smallest subnormal 2^-9, 1.0
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9 and ours[0x38] == 1.0
    assert ours[0x00] == 0.0 and np.signbit(ours[0x80])


def _codes_torch_fp8(t):
    t = np.clip(np.asarray(t, dtype=np.float32), -448.0, 448.0)  # saturating conversion
    return torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_quantize_matches_torch_including_ties_and_saturation():
    rng = np.random.default_rng(0)
    t = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 100, 20000),
                        rng.uniform(-2 ** -6, 2 ** -6, 5000)]).astype(np.float32)
    np.testing.assert_array_equal(oracle.quantize("fp8", t), _codes_torch_fp8(t))
    # exact midpoints between consecutive positive codes go to the even code
    vals = oracle.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)  # exact in fp32
    got = oracle.quantize("fp8", mids)
    want = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    np.testing.assert_array_equal(got, want.astype(np.uint8))
    np.testing.assert_array_equal(got, _codes_torch_fp8(mids))
    # saturation, signed zero, NaN
    assert list(oracle.quantize("fp8", [449.0, 1e6, np.inf, -1e6, -0.0, np.nan])) == \
        [0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x7F]


def test_int8_quantize_matches_numpy_rint_and_clip():
    rng = np.random.default_rng(1)
    t = np.concatenate([rng.normal(0, 60, 20000), np.arange(-140, 140) + 0.5,
                        [-0.5, 0.5, 1.5, 2.5, -1.5, 1e9, -1e9]]).astype(np.float32)
    want = np.clip(np.rint(t.astype(np.float64)), -128, 127).astype(np.int8).view(np.uint8)
    np.testing.assert_array_equal(oracle.quantize("i8", t), want)
    assert oracle.quantize("i8", [np.nan])[0] == 0


def _pools(kv, num_pages=6, bs=4, H=2, d=8, seed=3):
    rng = np.random.default_rng(seed)
    shape = (num_pages, bs, H, d)
    kc = rng.integers(0, 256, size=shape, dtype=np.uint8)
    vc = rng.integers(0, 256, size=shape, dtype=np.uint8)
    if kv == "fp8":  # no NaN codes in the pools of these pins
        kc[(kc & 0x7F) == 0x7F] = 0x3F
        vc[(vc & 0x7F) == 0x7F] = 0x3F
    return kc, vc


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_store_quant_matches_numpy_formulation(kv, dtype):
    rng = np.random.default_rng(5)
    num_pages, bs, H, d = 6, 4, 2, 8
    kc, vc = _pools(kv, num_pages, bs, H, d)
    k0, v0 = kc.copy(), vc.copy()
    n = 9
    x = torch.from_numpy(rng.normal(0, 3, (2, n, H, d)).astype(np.float32))
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
        xb = x.view(torch.int16).numpy().view(np.uint16)
    else:
        xb = x.numpy()
    xf = x.to(torch.float32).numpy()
    ks, kz, vs, vz = [rng.uniform(0.02, 0.5, (num_pages, H)).astype(np.float32),
                      rng.uniform(-3, 3, (num_pages, H)).astype(np.float32),
                      rng.uniform(0.02, 0.5, (num_pages, H)).astype(np.float32),
                      rng.uniform(-3, 3, (num_pages, H)).astype(np.float32)]
    slots = np.array([5, -1, 0, 23, 7, 30, 12, 13, 2], dtype=np.int64)  # 30 is past the pool
    skipped = oracle.store_kvcache_quant(dtype, kv, xb[0], xb[1], kc, vc, ks, kz, vs, vz, slots)
    assert skipped == 2
    kw, vw = k0.copy(), v0.copy()
    for i, sl in enumerate(slots):
        if sl < 0 or sl >= num_pages * bs:
            continue
        p = sl // bs
        for pool, xx, sc, zr in ((kw, xf[0], ks, kz), (vw, xf[1], vs, vz)):
            t = (xx[i] / sc[p][:, None]).astype(np.float32) + zr[p][:, None]
            t = t.astype(np.float32)
            if kv == "i8":
                code = np.clip(np.rint(t.astype(np.float64)), -128, 127).astype(np.int8)
                code = code.view(np.uint8)
            else:
                code = _codes_torch_fp8(t)
            pool[p, sl % bs] = code
    np.testing.assert_array_equal(kc, kw)
    np.testing.assert_array_equal(vc, vw)


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_decode_quant_equals_decode_on_dequantized_pools(kv):
    """Power-of-two scales and integer zero points make every dequantized value
    exact in fp32, so the plain decode oracle over those values must agree bit
    for bit (the same double arithmetic on the same numbers)."""
    rng = np.random.default_rng(7)
    num_pages, bs, H, d, Hq = 6, 4, 2, 8, 4
    kc, vc = _pools(kv, num_pages, bs, H, d, seed=8)
    ks = (2.0 ** rng.integers(-6, 0, (num_pages, H))).astype(np.float32)
    vs = (2.0 ** rng.integers(-6, 0, (num_pages, H))).astype(np.float32)
    kz = rng.integers(-4, 5, (num_pages, H)).astype(np.float32)
    vz = rng.integers(-4, 5, (num_pages, H)).astype(np.float32)
    val = (lambda c: c.view(np.int8).astype(np.float64)) if kv == "i8" else oracle.fp8_e4m3_decode
    kf = (ks[:, None, :, None] * (val(kc) - kz[:, None, :, None])).astype(np.float32)
    vf = (vs[:, None, :, None] * (val(vc) - vz[:, None, :, None])).astype(np.float32)
    assert np.array_equal(kf.astype(np.float64), ks[:, None, :, None] *
                          (val(kc) - kz[:, None, :, None]))  # exact
    sp = np.array([0, 2, 3, 6], dtype=np.uint32)
    bt = np.array([4, 1, 0, 5, 3, 2], dtype=np.uint32)
    ctx = np.array([7, 1, 10], dtype=np.int32)
    q = rng.normal(0, 1, (3, Hq, d)).astype(np.float32)
    _, ref = oracle.paged_attention_decode("f32", q, kf, vf, bt, sp, ctx, d ** -0.5)
    _, got = oracle.paged_attention_decode_quant("f32", kv, q, kc, vc, ks, kz, vs, vz, bt, sp,
                                                 ctx, d ** -0.5)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("kv", ["i8", "fp8"])
def test_decode_quant_brute_force(kv):
    """General scales and zero points against numpy softmax written out."""
    rng = np.random.default_rng(9)
    num_pages, bs, H, d, Hq = 5, 4, 1, 8, 2
    kc, vc = _pools(kv, num_pages, bs, H, d, seed=10)
    ks, vs = rng.uniform(0.01, 0.1, (2, num_pages, H)).astype(np.float32)
    kz, vz = rng.uniform(-2, 2, (2, num_pages, H)).astype(np.float32)
    val = (lambda c: c.view(np.int8).astype(np.float64)) if kv == "i8" else oracle.fp8_e4m3_decode
    sp = np.array([0, 3], dtype=np.uint64)
    table = [3, 0, 4]
    bt = np.array(table, dtype=np.uint64)
    n = 11
    q = rng.normal(0, 1, (1, Hq, d)).astype(np.float32)
    _, got = oracle.paged_attention_decode_quant("f32", kv, q, kc, vc, ks, kz, vs, vz, bt, sp,
                                                 np.array([n], np.int32), 0.3)
    for h in range(Hq):
        K = np.stack([ks[table[t // bs], 0] * (val(kc[table[t // bs], t % bs, 0]) -
                                                kz[table[t // bs], 0]) for t in range(n)])
        V = np.stack([vs[table[t // bs], 0] * (val(vc[table[t // bs], t % bs, 0]) -
                                                vz[table[t // bs], 0]) for t in range(n)])
        z = 0.3 * (K @ q[0, h].astype(np.float64))
        w = np.exp(z - z.max())
        np.testing.assert_allclose(got[0, h], (w / w.sum()) @ V, rtol=1e-12, atol=1e-12)

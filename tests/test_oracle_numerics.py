"""Pins of the oracle's storage-type conversions and of the KV byte accounting.

Widening is checked exhaustively (all 65536 bit patterns) against numpy's
float16 and torch's bfloat16 conversions; rounding to nearest-even is checked
against numpy (float64 -> float16 / float32, both correctly rounded in one
step), against torch for bfloat16 on values exact in float32, and on hand
cases where rounding through float32 first would give a different answer.
The KV-size arithmetic the pages print (tests/golden/kv_bytes.txt) pins the
byte count the benchmark divides by.
"""
import numpy as np
import torch

import oracle
import workloads
from conftest import read_golden


def test_widen_f16_exhaustive():
    bits = np.arange(2 ** 16, dtype=np.uint16)
    got = oracle.widen_dtype("f16", bits)
    want = bits.view(np.float16).astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()


def test_widen_bf16_exhaustive():
    bits = np.arange(2 ** 16, dtype=np.uint16)
    got = oracle.widen_dtype("bf16", bits)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0 and got[0x0001] == 2.0 ** -133


def test_round_f16_and_f32_match_numpy():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -25, 2.0 ** -24 * 1.5,
         5.960464477539063e-08, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 3.4e38, 3.5e38],
    ])
    got16 = oracle.round_to_dtype("f16", x)
    with np.errstate(over="ignore"):
        want16 = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(got16, want16)
    got32 = oracle.round_to_dtype("f32", x)
    with np.errstate(over="ignore"):
        want32 = x.astype(np.float32).view(np.uint32)
    np.testing.assert_array_equal(got32, want32)


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    x32 = np.concatenate([x32, np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                                         3.3895314e38, 3.4e38, 1e-40], dtype=np.float32)])
    got = oracle.round_to_dtype("bf16", x32.astype(np.float64))
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)


def test_round_bf16_is_single_rounding_from_double():
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties go to the even value 1.
    # A tiny excess puts it above the midpoint, which a detour through float32
    # would erase (float32 cannot hold 2^-40 next to 1).
    one = 0x3F80
    got = oracle.round_to_dtype("bf16", np.array([1 + 2 ** -8, 1 + 2 ** -8 + 2 ** -40,
                                                  1 + 2 ** -8 - 2 ** -40]))
    assert got.tolist() == [one, one + 1, one]
    # overflow to infinity and the largest finite value
    big = oracle.round_to_dtype("bf16", np.array([3.3961e38, 3.4e38, -1e39]))
    assert big.tolist() == [0x7F7F, 0x7F80, 0xFF80]


def test_printed_kv_sizes_and_workload_accounting():
    n = 0
    for line in read_golden("kv_bytes.txt"):
        lhs, want = line.split("->")
        _, L, hkv, d, b, T = lhs.split()
        L, hkv, d, b, T, want = int(L), int(hkv), int(d), int(b), int(T), int(want)
        # one layer of a workload with exactly T cached tokens, times L layers
        dtype = "bf16" if b == 2 else "f32"
        w = workloads.Workload("probe", dtype, "u32", hkv, hkv, d, 16, 1,
                               np.array([T], dtype=np.int32), np.array([0, 1], np.uint32),
                               np.array([0], np.uint32), 1.0)
        assert L * w.kv_bytes_logical() == want
        n += 1
    assert n == 7

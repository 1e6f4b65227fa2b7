"""Pins of the oracle's slot mapping and store.

"Paged KV Cache · AI infra interview lesson": the printed slots of Step 1 and
the fifth-token question of "Why It Matters" (tests/golden/slot_mapping.txt),
Step 1's property test (slots emitted page by page equal the per-token rule
for bs in {4, 16, 256}) and store test (a -1 slot leaves its row untouched, n-1
rows written), the decode-slot pitfall of "Common Pitfalls" and the new-page
rule of "Walk the Shapes First". Independently of any formula, slots are also
checked against a numpy gather over a table of slot ids laid out like the pool.
"""
import numpy as np
import pytest

import oracle
from conftest import ints, read_golden


def _csr(tables, dtype=np.uint32):
    sp = np.zeros(len(tables) + 1, dtype=np.int64)
    sp[1:] = np.cumsum([len(t) for t in tables])
    return sp.astype(dtype), np.array([p for t in tables for p in t], dtype=dtype)


def _per_token(bt, start, end, bs, num_pages=1 << 40):
    """CSR slot mapping of one sequence's positions [start, end)."""
    sp, flat = _csr([bt])
    return oracle.slot_mapping(flat, sp, bs, num_pages, [start],
                               [0, max(0, end - start)]).tolist()


def _page_runs(bt, start, end, bs):
    """Slots of positions [start, end) written as one contiguous run per logical page: page k
    of the table contributes the offsets of [start, end) that fall inside [k*bs, (k+1)*bs)."""
    out = []
    for k, page in enumerate(bt):
        lo, hi = max(start, k * bs), min(end, (k + 1) * bs)
        out.extend(range(page * bs + lo - k * bs, page * bs + hi - k * bs))
    return out


def test_printed_slots():
    n = 0
    for line in read_golden("slot_mapping.txt"):
        lhs, want = line.split("->")
        kind, bt, *nums = lhs.split()
        want, bt, nums = ints(want.strip()), ints(bt), [int(x) for x in nums]
        if kind == "ranges":
            a, b, bs = nums
            assert _page_runs(bt, a, b, bs) == want
            assert _per_token(bt, a, b, bs) == want
        else:  # one token at a position
            p, bs = nums
            assert _per_token(bt, p, p + 1, bs) == want
        n += 1
    assert n == 2


@pytest.mark.parametrize("bs", [4, 16, 256])
def test_range_emission_equals_per_token_rule(bs):
    bt = [7, 2, 5]
    for start, end in [(0, 2 * bs + 2), (bs // 2 + 1, 2 * bs + 1), (bs, 2 * bs), (3, 3)]:
        ranges = _page_runs(bt, start, end, bs)
        assert ranges == _per_token(bt, start, end, bs)
        # independent of both: gather from a pool-shaped table of slot ids
        slot_ids = np.arange(8 * bs).reshape(8, bs)
        logical = slot_ids[np.array(bt)].reshape(-1)
        assert ranges == logical[start:end].tolist()
    assert _per_token(bt, 5, 5, bs) == [] and _page_runs(bt, 5, 5, bs) == []
    assert _per_token(bt, 7, 3, bs) == []


def test_batch_slot_mapping_matches_gather():
    rng = np.random.default_rng(11)
    for trial in range(25):
        bs = int(rng.choice([1, 2, 3, 4, 5, 16]))
        num_pages = 40
        B = int(rng.integers(1, 6))
        tables = [rng.permutation(num_pages)[:int(rng.integers(0, 5))].tolist() for _ in range(B)]
        for index in (np.uint32, np.uint64):
            sp, flat = _csr(tables, index)
            start = rng.integers(0, 3 * bs, size=B).astype(np.int32)
            counts = rng.integers(0, 2 * bs + 1, size=B)
            cu = np.zeros(B + 1, dtype=np.int64)
            cu[1:] = np.cumsum(counts)
            # a pool smaller than the ids in use: ids >= pool_pages have no slot
            pool_pages = num_pages if trial % 2 else int(rng.integers(1, num_pages))
            got = oracle.slot_mapping(flat, sp, bs, pool_pages, start, cu)
            slot_ids = np.arange(num_pages * bs).reshape(num_pages, bs)
            want = []
            for s, t in enumerate(tables):
                logical = slot_ids[np.array(t, dtype=np.int64)].reshape(-1) if t else []
                for p in range(start[s], start[s] + counts[s]):
                    ok = p < len(logical) and t[p // bs] < pool_pages
                    want.append(int(logical[p]) if ok else -1)
            assert got.tolist() == want


@pytest.mark.parametrize("bs", [4, 16, 256])
def test_decode_slot_is_at_len_minus_one(bs):
    """Appending token number `length` writes position length-1, not one past it."""
    rng = np.random.default_rng(bs)
    pages = rng.permutation(64)[:6].tolist()
    for length in range(1, 5 * bs + 1):
        n_pages = -(-length // bs)
        table = pages[:n_pages]
        got = _per_token(table, length - 1, length, bs)[0]
        # the pitfall: last page base plus the number of tokens in the last page
        tokens_in_last = length - (n_pages - 1) * bs
        pitfall = table[-1] * bs + tokens_in_last
        assert got == pitfall - 1


@pytest.mark.parametrize("bs", [4, 16, 256])
def test_new_page_needed_exactly_when_len_mod_bs_is_one(bs):
    """With the pages of length-1 tokens only, the new token has a slot iff len % bs != 1."""
    pages = list(range(10, 20))
    for length in range(2, 4 * bs + 2):
        table = pages[:-(-(length - 1) // bs)]
        slot = _per_token(table, length - 1, length, bs)[0]
        assert (slot == -1) == (length % bs == 1 or bs == 1)


@pytest.mark.parametrize("bs", [4, 16, 256])
def test_store_matches_printed_test_and_numpy_scatter(bs):
    rng = np.random.default_rng(100 + bs)
    H, d, n = 2, 4, 2 * bs + 2
    bt = [7, 2, 5]
    k_cache = np.zeros((8, bs, H, d), dtype=np.float32)
    v_cache = np.zeros((8, bs, H, d), dtype=np.float32)
    key = rng.standard_normal((n, H, d)).astype(np.float32)
    value = rng.standard_normal((n, H, d)).astype(np.float32)
    slots = np.array(_per_token(bt, 0, n, bs), dtype=np.int64)
    slots[1] = -1
    assert oracle.store_kvcache(key, value, k_cache, v_cache, slots) == 0
    for p in range(n):
        want = np.zeros((H, d), np.float32) if p == 1 else key[p]
        np.testing.assert_array_equal(k_cache[bt[p // bs], p % bs], want)
    assert int((np.abs(k_cache).sum((-1, -2)) != 0).sum()) == n - 1
    # numpy's scatter by slot over the [num_pages*bs, H*d] view
    kc2 = np.zeros_like(k_cache)
    vc2 = np.zeros_like(v_cache)
    mask = slots != -1
    kc2.reshape(-1, H * d)[slots[mask]] = key.reshape(n, -1)[mask]
    vc2.reshape(-1, H * d)[slots[mask]] = value.reshape(n, -1)[mask]
    assert k_cache.tobytes() == kc2.tobytes() and v_cache.tobytes() == vc2.tobytes()


def test_store_is_bitwise_and_skips_invalid():
    rng = np.random.default_rng(5)
    num_pages, bs, H, d = 3, 4, 2, 8
    kc = rng.integers(0, 2 ** 16, size=(num_pages, bs, H, d), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, size=(num_pages, bs, H, d), dtype=np.uint16)
    before_k, before_v = kc.copy(), vc.copy()
    key = rng.integers(0, 2 ** 16, size=(6, H, d), dtype=np.uint16)
    key[0, 0, 0] = 0x7FC1  # a NaN payload must be copied unchanged
    value = rng.integers(0, 2 ** 16, size=(6, H, d), dtype=np.uint16)
    slots = np.array([5, -1, 12, -7, 0, 5], dtype=np.int64)  # 12 == num_pages*bs, -7 invalid
    invalid = oracle.store_kvcache(key, value, kc, vc, slots)
    assert invalid == 2
    flat_k, flat_v = kc.reshape(-1, H * d), vc.reshape(-1, H * d)
    np.testing.assert_array_equal(flat_k[5], key[5].reshape(-1))   # last writer wins
    np.testing.assert_array_equal(flat_v[5], value[5].reshape(-1))
    np.testing.assert_array_equal(flat_k[0], key[4].reshape(-1))
    untouched = [r for r in range(num_pages * bs) if r not in (0, 5)]
    np.testing.assert_array_equal(flat_k[untouched], before_k.reshape(-1, H * d)[untouched])
    np.testing.assert_array_equal(flat_v[untouched], before_v.reshape(-1, H * d)[untouched])

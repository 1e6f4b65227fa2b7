"""Pins of the oracle's block-table addressing and index validation.

Pinned to the worked examples of "Block-Paged KV Cache" (Hurray docs),
sections "Element lookup through the block table" and "Validating the storage
invariants" (fixtures in tests/golden/), and to a brute-force gather that
builds each sequence's logical tensor by concatenating its pages with numpy.
"""
import itertools

import numpy as np
import pytest

import oracle
from conftest import ints, read_golden


def _golden_offset_case():
    lines = read_golden("element_offset.txt")
    params = dict(kv.split("=") for kv in lines[0].split())
    sp = np.array(ints(lines[1].split("=")[1]), dtype=np.uint32)
    bt = np.array(ints(lines[2].split("=")[1]), dtype=np.uint32)
    geo = {k: int(v) for k, v in params.items()}
    return geo, sp, bt, lines[3:]


@pytest.mark.parametrize("index", [np.uint32, np.uint64])
def test_printed_element_offset(index):
    geo, sp, bt, cases = _golden_offset_case()
    sp, bt = sp.astype(index), bt.astype(index)
    n_checked = 0
    for line in cases:
        kind, rest = line.split(None, 1)
        if kind == "offset":
            s, t, h, d, want = (int(x) for x in rest.split())
            st, flat = oracle.element_offset(s, t, h, d, geo["page_size"], geo["num_pages"],
                                             geo["num_heads"], geo["head_dim"], bt, sp)
            assert st == oracle.OK and flat == want
            n_checked += 1
        elif kind == "alias":
            a, b = ([int(x) for x in part.split()] for part in rest.split("|"))
            sa, fa = oracle.element_offset(*a, geo["page_size"], geo["num_pages"],
                                           geo["num_heads"], geo["head_dim"], bt, sp)
            sb, fb = oracle.element_offset(*b, geo["page_size"], geo["num_pages"],
                                           geo["num_heads"], geo["head_dim"], bt, sp)
            assert sa == sb == oracle.OK and fa == fb
            n_checked += 1
    assert n_checked == 2


def test_element_offset_matches_page_concatenation():
    """Brute force: every logical element equals the pool element at its offset."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        ps = int(rng.integers(1, 6))
        H = int(rng.integers(1, 4))
        D = int(rng.integers(1, 5))
        num_pages = int(rng.integers(3, 9))
        B = int(rng.integers(1, 4))
        tables = [rng.integers(0, num_pages, size=int(rng.integers(0, 4))).tolist()
                  for _ in range(B)]
        sp = np.zeros(B + 1, dtype=np.uint64)
        sp[1:] = np.cumsum([len(t) for t in tables])
        bt = np.array([p for t in tables for p in t], dtype=np.uint64)
        pool = np.arange(num_pages * ps * H * D).reshape(num_pages, ps, H, D)
        for s, table in enumerate(tables):
            logical = pool[np.array(table, dtype=np.int64)].reshape(-1, H, D) if table else \
                np.zeros((0, H, D), dtype=pool.dtype)
            for t, h, d in itertools.product(range(len(logical)), range(H), range(D)):
                st, flat = oracle.element_offset(s, t, h, d, ps, num_pages, H, D, bt, sp)
                assert st == oracle.OK
                assert pool.reshape(-1)[flat] == logical[t, h, d]
            # one past the slice is refused, as are out-of-range heads and dims
            st, _ = oracle.element_offset(s, len(logical), 0, 0, ps, num_pages, H, D, bt, sp)
            assert st == oracle.OUT_OF_RANGE
        st, _ = oracle.element_offset(0, 0, H, 0, ps, num_pages, H, D, bt, sp)
        assert st == oracle.OUT_OF_RANGE
        st, _ = oracle.element_offset(0, 0, 0, D, ps, num_pages, H, D, bt, sp)
        assert st == oracle.OUT_OF_RANGE
        st, _ = oracle.element_offset(B, 0, 0, 0, ps, num_pages, H, D, bt, sp)
        assert st == oracle.OUT_OF_RANGE


@pytest.mark.parametrize("index", [np.uint32, np.uint64])
def test_printed_validator_cases(index):
    seen = set()
    for line in read_golden("validate.txt"):
        verdict, num_pages, sp, bt = line.split()
        st = oracle.validate_index_buffers(np.array(ints(sp), dtype=index),
                                           np.array(ints(bt), dtype=index), int(num_pages))
        assert (st == oracle.OK) == (verdict == "ok"), line
        seen.add(verdict)
    assert seen == {"ok", "bad"}


def test_validator_each_invariant():
    u = np.uint32
    ok = oracle.validate_index_buffers(np.array([0, 2, 3], u), np.array([0, 1, 0], u), 5)
    assert ok == oracle.OK
    assert oracle.validate_index_buffers(np.array([1, 2, 3], u), np.array([0, 1, 0], u), 5) \
        == oracle.SEQ_PTR_FIRST
    assert oracle.validate_index_buffers(np.array([0, 3, 2, 3], u), np.array([0, 1, 0], u), 5) \
        == oracle.SEQ_PTR_ORDER
    assert oracle.validate_index_buffers(np.array([0, 2, 2], u), np.array([0, 1, 0], u), 5) \
        == oracle.SEQ_PTR_LAST
    assert oracle.validate_index_buffers(np.array([0, 2, 3], u), np.array([0, 1, 0], u), 1) \
        == oracle.PAGE_RANGE
    # aliasing (the same page in two slices) is accepted
    assert oracle.validate_index_buffers(np.array([0, 1, 2], u), np.array([4, 4], u), 5) \
        == oracle.OK
    # context lengths: must fit pages*page_size and be non-negative
    sp, bt = np.array([0, 2, 3], u), np.array([0, 1, 0], u)
    assert oracle.validate_index_buffers(sp, bt, 5, context_lens=[8, 4], page_size=4) == oracle.OK
    assert oracle.validate_index_buffers(sp, bt, 5, context_lens=[9, 4], page_size=4) \
        == oracle.CTX_RANGE
    assert oracle.validate_index_buffers(sp, bt, 5, context_lens=[-1, 4], page_size=4) \
        == oracle.CTX_RANGE
    # u32 wrap of -1 (the padded-table filler) is an out-of-range page id
    assert oracle.validate_index_buffers(np.array([0, 1], u), np.array([0xFFFFFFFF], u), 5) \
        == oracle.PAGE_RANGE

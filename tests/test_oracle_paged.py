"""Pins of the oracle's paged-store bookkeeping (oracle/paged.py).

The model is pinned to things it does not compute itself: the contiguous
layout the C oracle computes (oracle.prefill_layout, 64-row alignment),
which one whole-batch admission after init must reproduce page for page;
hand-worked stack states; and the conservation invariant under random
sequences of operations."""
import numpy as np
import pytest

import oracle
import workload
from oracle.paged import PAGE_ROWS, PagedBook, pages_for


def test_pages_for():
    assert [pages_for(r) for r in (0, 1, 63, 64, 65, 128, 129)] == [0, 1, 1, 1, 2, 2, 3]


@pytest.mark.parametrize("W,reserve,T", [(16, 5, 300), (64, 0, 1000), (0, 64, 200), (100, 3, 90)])
def test_first_admission_is_the_contiguous_layout(W, reserve, T):
    cfg = workload.custom(B=3, Hkv=2, T=T, W=W, keep_lo=0.1, keep_hi=0.6, seed=9)
    keep = workload.make_layer(cfg, 0).keep
    lay = oracle.prefill_layout(keep, T, W, reserve, align=PAGE_ROWS)
    n_pages = int(lay["seg_base"][-1]) // PAGE_ROWS + 5
    book = PagedBook(n_pages, cfg.B, cfg.Hkv, W, max_pages=64)
    assert book.admit(0, cfg.B, lay["comp_len"], reserve)
    for i in range(cfg.B * cfg.Hkv):
        first = int(lay["seg_base"][i]) // PAGE_ROWS
        size = (int(lay["seg_base"][i + 1]) - int(lay["seg_base"][i])) // PAGE_ROWS
        assert book.table[i] == list(range(first, first + size))
        assert book.seg_cap(i) == size * PAGE_ROWS - W >= int(lay["seg_cap"][i])
    assert book.free == list(range(n_pages - 1, int(lay["seg_base"][-1]) // PAGE_ROWS - 1, -1))
    book.check()


def test_hand_worked_stack():
    book = PagedBook(8, B=2, Hkv=1, W=0, max_pages=4)
    assert book.admit(0, 1, [130], 0)              # 3 pages
    assert book.table[0] == [0, 1, 2]
    assert book.admit(1, 1, [10], 0)               # 1 page
    assert book.table[1] == [3]
    book.release(0, 1)                             # 0, 1, 2 pushed in that order
    assert book.free == [7, 6, 5, 4, 0, 1, 2] and book.table[0] == []
    assert book.admit(0, 1, [64], 0)               # last released first
    assert book.table[0] == [2]
    book.refill([64, 10], reserve=64)              # 128 and 74 rows: 2 pages each
    assert book.table == [[2, 1], [3, 0]] and book.free == [7, 6, 5, 4]
    assert not book.pages_error
    book.check()


def test_admission_is_all_or_nothing():
    book = PagedBook(5, B=2, Hkv=2, W=0, max_pages=8)
    assert not book.admit(0, 2, [64, 64, 64, 129], 0)  # needs 1 + 1 + 1 + 3 > 5 pages
    assert book.pages_error and book.free == [4, 3, 2, 1, 0]
    assert all(row == [] for row in book.table) and book.live == [False, False]
    book2 = PagedBook(50, B=1, Hkv=1, W=0, max_pages=2)
    assert not book2.admit(0, 1, [129], 0)              # 3 pages > max_pages
    assert book2.pages_error and len(book2.free) == 50


def test_refill_serves_earlier_segments_first():
    book = PagedBook(6, B=1, Hkv=3, W=0, max_pages=8)
    assert book.admit(0, 1, [0, 0, 0], 64)            # one page each
    book.refill([64, 64, 64], reserve=64)              # each wants 2: only 3 pages left
    assert [len(r) for r in book.table] == [2, 2, 2] and not book.pages_error
    book.refill([128, 128, 128], reserve=64)           # each wants 3; stack is empty
    assert [len(r) for r in book.table] == [2, 2, 2] and book.pages_error
    book.check()


def test_refill_skips_idle_and_caps_at_max_pages():
    book = PagedBook(20, B=2, Hkv=1, W=32, max_pages=3)
    assert book.admit(0, 1, [0], 0)
    book.refill([1000, 1000], reserve=64)
    assert len(book.table[0]) == 3 and book.table[1] == []   # capped; sequence 1 idle
    book.check()


def test_random_serving_mix_keeps_every_page_accounted():
    rng = np.random.default_rng(3)
    B, Hkv, W = 4, 2, 32
    book = PagedBook(40, B, Hkv, W, max_pages=12)
    comp = np.zeros(B * Hkv, int)
    for _ in range(400):
        b = int(rng.integers(B))
        op = rng.integers(4)
        if op == 0 and not book.live[b]:
            c = rng.integers(0, 300, Hkv)
            if book.admit(b, 1, c, int(rng.integers(0, 70))):
                comp[b * Hkv:(b + 1) * Hkv] = c
        elif op == 1 and book.live[b]:
            book.release(b, 1)
            comp[b * Hkv:(b + 1) * Hkv] = 0
        elif op == 2:
            for i in range(B * Hkv):
                if book.live[i // Hkv]:
                    comp[i] = min(comp[i] + int(rng.integers(0, 20)), book.seg_cap(i))
            book.refill(comp, 64)
        book.check()
        for i in range(B * Hkv):
            if book.live[i // Hkv]:
                assert comp[i] <= book.seg_cap(i)
            else:
                assert book.table[i] == []

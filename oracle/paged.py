"""Oracle model of the paged compact store's page bookkeeping (test
infrastructure only: the tests may import it, the product never does).

What it models.  FastDMS page ("FastDMS: 6.4X KV-cache compression running
faster than vLLM BF16/FP8"), release paragraph: the compact store gives the
memory of evicted tokens back to the allocator.  Carried across requests,
that is a pool of fixed-size pages shared by every (sequence, KV head)
segment, a page table per segment, and a free list that pages of finished
requests return to.  The pages fix none of the details; the ones here are
the library's stated rules, written out plainly:

  * a page is 64 rows; the free pages are a stack (taken from the top);
  * init: every page free, stacked so that pages are first taken in
    ascending order; every segment idle with no page;
  * admission of a range of sequences: each segment of the range needs
    ceil((W + comp_len + reserve) / 64) pages; the range gets all of them
    (segments in index order, pages in row order, each the top of the
    stack) or, if the stack is short or a segment needs more than
    max_pages, none;
  * refill: every live segment, in index order, takes pages until its
    pages cover W + comp_len + reserve rows (at most max_pages); a short
    stack serves the earlier segments first;
  * release of a range: its segments' pages go back onto the stack
    (segments in index order, pages in row order) and the segments become
    idle.

Segment contents are not modelled here: the rows a segment holds are those
of the contiguous store (``oracle.OracleCache``), only their placement in
the pool changes.
"""
from __future__ import annotations

PAGE_ROWS = 64


def pages_for(rows: int) -> int:
    """Pages that hold `rows` rows."""
    return -(-rows // PAGE_ROWS)


class PagedBook:
    """Free stack and page tables of a paged store with `n_pages` pages,
    `nh` = B * Hkv segments of `max_pages` page-table entries each."""

    def __init__(self, n_pages: int, B: int, Hkv: int, W: int, max_pages: int):
        self.n_pages, self.B, self.Hkv, self.W, self.max_pages = n_pages, B, Hkv, W, max_pages
        self.nh = B * Hkv
        # the top of the stack is the end of the list; page 0 is on top
        self.free = list(range(n_pages - 1, -1, -1))
        self.table = [[] for _ in range(self.nh)]   # pages held, in row order
        self.live = [False] * B
        self.pages_error = False

    # -- queries
    def table_array(self):
        """Page-table rows padded with -1 to max_pages entries."""
        return [row + [-1] * (self.max_pages - len(row)) for row in self.table]

    def seg_cap(self, i: int) -> int:
        return max(PAGE_ROWS * len(self.table[i]) - self.W, 0)

    def segs(self, b0: int, nb: int):
        return range(b0 * self.Hkv, (b0 + nb) * self.Hkv)

    # -- operations
    def admit(self, b0: int, nb: int, comp_len, reserve: int) -> bool:
        """Pages for sequences [b0, b0 + nb), whose segments hold comp_len[j]
        compact rows (j = index within the range).  All or nothing."""
        need = [pages_for(self.W + int(comp_len[j]) + reserve)
                for j in range(nb * self.Hkv)]
        if any(n > self.max_pages for n in need) or sum(need) > len(self.free):
            self.pages_error = True
            for i in self.segs(b0, nb):
                self.table[i] = []
            return False
        for j, i in enumerate(self.segs(b0, nb)):
            self.table[i] = [self.free.pop() for _ in range(need[j])]
        for b in range(b0, b0 + nb):
            self.live[b] = True
        return True

    def refill(self, comp_len, reserve: int) -> None:
        """comp_len[i] for every segment i of the batch."""
        for i in range(self.nh):
            if not self.live[i // self.Hkv]:
                continue
            want = min(pages_for(self.W + int(comp_len[i]) + reserve), self.max_pages)
            while len(self.table[i]) < want:
                if not self.free:
                    self.pages_error = True
                    break
                self.table[i].append(self.free.pop())

    def release(self, b0: int, nb: int) -> None:
        for i in self.segs(b0, nb):
            self.free.extend(self.table[i])
            self.table[i] = []
        for b in range(b0, b0 + nb):
            self.live[b] = False

    # -- the invariant every state keeps
    def check(self) -> None:
        held = [p for row in self.table for p in row]
        every = sorted(held + self.free)
        assert every == list(range(self.n_pages)), "a page is lost or held twice"
        for row in self.table:
            assert len(row) <= self.max_pages

"""Paged retrieval rows and prefix sharing (oracle; test infrastructure only).

What is modelled.  "Attention Variants and Memory Efficiency", "What the
Inference Runtime Can Change", lists paging among the runtime's storage
choices: a request's rows are cut into equal blocks that may sit anywhere in
memory, which makes allocation and sharing easier while the set of cached
values stays what the attention rule needs; prefix sharing stores the blocks
of a common prefix once.  Its section "A Closer Look at Attention Memory"
contrasts padding every request to the longest one with a ragged layout that
sizes each request's cache to its own length.

Readings taken where the pages leave a step open:
  * a page holds P consecutive positions of one request (batch row), for
    every retrieval head of a layer (one page table per row and layer);
  * a row that holds n tokens holds ceil(n / P) pages, taken from a pool of
    fixed size as the row grows;
  * a fork makes an empty row a copy of another row: the full pages of the
    source are shared (held by both rows, stored once); a partly filled last
    page is copied into a page of the new row's own;
  * a row only writes the positions past its own count, so a shared page (a
    full one) is never written again;
  * a reset empties a row; a page returns to the pool when no row holds it.

Attention over a paged cache is attention over the logical rows
(oracle.attention): paging changes where rows live, not which rows a query
sees.  This module models the page accounting and what each position of a row
holds; the pins in tests/oracle_checks.py are closed-form page counts and the
content of forked rows.
"""
from __future__ import annotations

from typing import List, Tuple


class _Page:
    """One page: slot i holds (origin row, position) of the token stored there,
    or None."""

    def __init__(self, P: int):
        self.slots: List = [None] * P


class PagedRows:
    """B rows over a pool of n_pages pages of P positions each."""

    def __init__(self, P: int, n_pages: int, B: int):
        assert P >= 1 and n_pages >= 0 and B >= 1
        self.P, self.n_pages, self.B = P, n_pages, B
        self.rows: List[List[_Page]] = [[] for _ in range(B)]
        self.count = [0] * B

    def pages_needed(self, n: int) -> int:
        """Pages a row of n tokens holds."""
        return -(-n // self.P)

    def pages_in_use(self) -> int:
        """Pages held by at least one row (a shared page counts once)."""
        return len({id(pg) for r in self.rows for pg in r})

    def free_pages(self) -> int:
        return self.n_pages - self.pages_in_use()

    def _grow_need(self, rows_and_counts) -> int:
        return sum(max(0, self.pages_needed(self.count[b] + n) - len(self.rows[b])) for b, n in rows_and_counts)

    def append(self, b: int, n: int, origin: int = None) -> None:
        """Row b takes n more tokens at positions count .. count + n - 1 (their
        content is recorded as coming from row `origin`, default b).  Raises
        MemoryError, changing nothing, if the pool is short of pages."""
        self.append_rows([(b, n)], origin)

    def append_rows(self, rows_and_counts, origin: int = None) -> None:
        """Several rows grow at once (all or none)."""
        if self._grow_need(rows_and_counts) > self.free_pages():
            raise MemoryError("not enough free pages")
        for b, n in rows_and_counts:
            while len(self.rows[b]) < self.pages_needed(self.count[b] + n):
                self.rows[b].append(_Page(self.P))
            for p in range(self.count[b], self.count[b] + n):
                self.rows[b][p // self.P].slots[p % self.P] = (b if origin is None else origin, p)
            self.count[b] += n

    def fork(self, src: int, dst: int) -> None:
        """Empty row dst becomes a copy of row src: src's full pages are
        shared; a partly filled last page is copied."""
        assert self.count[dst] == 0 and src != dst
        n = self.count[src]
        full = n // self.P
        pages = list(self.rows[src][:full])
        if n % self.P:
            if self.free_pages() < 1:
                raise MemoryError("no free page for the copy of the last page")
            copy = _Page(self.P)
            copy.slots = list(self.rows[src][full].slots)
            pages.append(copy)
        self.rows[dst] = pages
        self.count[dst] = n

    def reset(self, b: int) -> None:
        self.rows[b] = []
        self.count[b] = 0

    def content(self, b: int) -> List[Tuple[int, int]]:
        """(origin row, position) of the token at each position of row b."""
        return [self.rows[b][p // self.P].slots[p % self.P] for p in range(self.count[b])]

    def shared_pages(self, b1: int, b2: int) -> int:
        """Pages rows b1 and b2 both hold."""
        return len({id(pg) for pg in self.rows[b1]} & {id(pg) for pg in self.rows[b2]})

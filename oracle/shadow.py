"""The page-table semantics with no pages at all, and the page counts it implies.

``ShadowCache`` keeps every request's rows as a plain list, which is the
shadow model the silicon-compiler chapter 15 page checks a page table against
(section "Tests", check 1): whatever the table does with pages, the rows a
request reads back through it must equal the list.  Window trimming does not
change the list; it only says which rows may no longer be read.

Closed forms of the window rule (same chapter, section "The problem" and
"Tests", check 3):

* a request holding ``rows`` rows, trimmed at ``keep_from``, holds exactly
  ``ceil(rows / P) - floor(keep_from / P)`` pages (0 if it holds no rows);
* with a window of ``W`` tokens, after the trim that follows each step a
  request holds at most ``ceil((W - 1) / P) + 1`` pages.

With ``S`` attention-sink rows kept besides a window of ``W - S`` (same
chapter, section "Exercises", exercise 3) the first ``h = ceil(S / P)`` pages
are never released, and the trim at ``L + 1 - (W - S)`` keeps at most
``ceil((W - S - 1) / P) + 1`` pages after them, so a request holds at most
``h + ceil((W - S - 1) / P) + 1`` pages.
"""
from __future__ import annotations


class ShadowCache:
    def __init__(self):
        self.rows: dict = {}
        self.keep_from: dict = {}

    def new(self, rid):
        self.rows[rid] = []
        self.keep_from[rid] = 0

    def append(self, rid, row):
        self.rows[rid].append(row)

    def fork(self, src, dst):
        self.rows[dst] = list(self.rows[src])
        self.keep_from[dst] = self.keep_from[src]

    def trim(self, rid, keep_from):
        self.keep_from[rid] = max(self.keep_from[rid], keep_from)

    def release(self, rid):
        del self.rows[rid]
        del self.keep_from[rid]

    def readable(self, rid):
        """Rows still readable: everything from the first row of the first kept page."""
        return self.rows[rid]


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def pages_exact(rows: int, keep_from: int, page: int) -> int:
    """Pages held by a request with ``rows`` rows after a trim at ``keep_from``."""
    if rows <= 0:
        return 0
    return max(ceil_div(rows, page) - keep_from // page, 0)


def window_bound(window: int, page: int) -> int:
    """Most pages a request holds after each step's trim, with a window."""
    return ceil_div(window - 1, page) + 1


def pages_exact_sinks(rows: int, keep_from: int, head: int, page: int) -> int:
    """Pages held when the first ``head`` pages are never released: every
    page of the rows, less those after the head that end at or before
    ``keep_from``."""
    if rows <= 0:
        return 0
    total = ceil_div(rows, page)
    released = min(max(keep_from // page - head, 0), max(total - head, 0))
    return total - released


def sink_bound(window: int, sinks: int, page: int) -> int:
    """Most pages a request with ``sinks`` sink rows holds after each step's trim."""
    return ceil_div(sinks, page) + ceil_div(window - sinks - 1, page) + 1

"""Host block allocator: free list, reference counts, copy-on-write, window trim.

Plain host code.  It decides where each new K/V row goes and which pages must
be copied first; it never touches K/V data.  Its output is what the kernels
consume: int32 block tables (-1 where a page was released), raw token-slot
tables, the slot of every new row and the list of pages to copy.

Semantics follow the page table of the silicon-compiler chapter 15 (section
"The model"):

* ``append`` takes a fresh page when the new row opens a page (row index a
  multiple of the page size); otherwise, if the tail page is shared
  (reference count above one), it takes a fresh page, schedules a whole-page
  copy of the shared one into it, drops one reference to the shared page and
  maps the copy in its place (lazy copy-on-write).  A failed allocation raises
  ``OutOfPages`` and leaves the request unchanged.
* ``trim(keep_from)`` releases front pages while the page after the last
  released one ends at or before ``keep_from``, so a page that still holds a
  needed row stays.  After a decode step at context ``L`` with window ``W``
  the next step needs rows ``>= L + 1 - W``.
* with ``sinks`` rows kept at the start (the attention-sink exercise of that
  chapter, section "Exercises"), the first ``ceil(sinks / P)`` pages are never
  trimmed: the released pages then form a hole between them and the window,
  and the table reads -1 there.
* ``fork`` shares every page, a partial tail included, adding one reference
  each; ``release`` drops one reference to each page of the request.
* a page whose count reaches zero goes back on the free list.

The free list is LIFO by default, handing out page 0 first and reusing the
page freed last first, as in that chapter, so its printed traces reproduce;
``policy="fifo"`` gives the deque order of the llm-systems-cookbook notebook
"PagedAttention block allocator" (section "Block allocator").  ``free_order``
seeds any initial order (a shuffled placement).

``rewind`` (drop the newest rows, freeing pages that no longer hold any) is
the lifecycle hook of the tiny-llm page "Paged KV Cache" (Task 2), and
``pages_needed`` is the page-boundary difference of the mini-sglang page
(section on paged allocation).

Every change to a request's table (a page mapped, remapped by copy-on-write or
released) is also recorded as an update ``(request, logical page, physical
page or -1)``; ``take_table_updates`` hands them over as index lists for one
device scatter (``pa_update_tables``), the way the mini-sglang page writes new
table cells with one scatter instead of rebuilding tables on the host.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass
from typing import Dict, Hashable, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class OutOfPages(RuntimeError):
    """No free page is left in the pool."""


@dataclass
class AppendPlan:
    """Where one new row goes, and the copy that must run before it is written."""
    rid: Hashable
    row: int                      # logical row index of the new row
    page: int                     # physical page it goes to
    offset: int                   # row within the page
    slot: int                     # page * page_size + offset
    copy: Optional[Tuple[int, int]] = None   # (shared source page, private target page)
    new_page: bool = False        # the row opened a fresh page


@dataclass
class StepPlan:
    """The device operands of one decode step for a batch of requests."""
    rids: List[Hashable]
    slots: np.ndarray             # int32 [B]
    copy_src: np.ndarray          # int32 [C]
    copy_dst: np.ndarray          # int32 [C]
    context_lens: np.ndarray      # int32 [B], including the new row


class BlockAllocator:
    """Pages of one pool, with reference counts and a free list."""

    def __init__(self, num_pages: int, policy: str = "lifo",
                 free_order: Optional[Sequence[int]] = None):
        if num_pages <= 0:
            raise ValueError("a pool needs at least one page")
        if policy not in ("lifo", "fifo"):
            raise ValueError(policy)
        self.num_pages = num_pages
        self.policy = policy
        self.ref = [0] * num_pages
        order = list(free_order) if free_order is not None else list(range(num_pages))
        if sorted(order) != list(range(num_pages)):
            raise ValueError("free_order must be a permutation of the pages")
        # the next page handed out is order[0] under both policies
        self._free = deque(order) if policy == "fifo" else list(reversed(order))

    @property
    def free(self) -> List[int]:
        return list(self._free)

    def free_count(self) -> int:
        return len(self._free)

    def used(self) -> int:
        return self.num_pages - len(self._free)

    def alloc(self) -> int:
        if not self._free:
            raise OutOfPages("no free page")
        p = self._free.popleft() if self.policy == "fifo" else self._free.pop()
        self.ref[p] = 1
        return p

    def incref(self, p: int) -> None:
        if self.ref[p] <= 0:
            raise ValueError(f"page {p} is not held")
        self.ref[p] += 1

    def unref(self, p: int) -> None:
        if self.ref[p] <= 0:
            raise ValueError(f"page {p} is not held")
        self.ref[p] -= 1
        if self.ref[p] == 0:
            self._free.append(p)


class PagedKVCache:
    """Per-request block tables over one ``BlockAllocator``."""

    def __init__(self, num_pages: int, page_size: int, policy: str = "lifo",
                 free_order: Optional[Sequence[int]] = None):
        if page_size <= 0:
            raise ValueError("page_size must be positive")
        self.page_size = page_size
        self.pool = BlockAllocator(num_pages, policy, free_order)
        self.pages: Dict[Hashable, List[int]] = {}    # live pages, oldest first
        self.length: Dict[Hashable, int] = {}
        self.dropped: Dict[Hashable, int] = {}        # pages released by trim
        self.head: Dict[Hashable, int] = {}           # leading pages kept for sink rows
        self._updates: List[Tuple[Hashable, int, int]] = []   # (request, logical page, page)

    # -- lifecycle -------------------------------------------------------------
    def new(self, rid: Hashable, sinks: int = 0) -> None:
        if rid in self.pages:
            raise KeyError(f"request {rid!r} exists")
        if sinks < 0:
            raise ValueError("sinks must be >= 0")
        self.pages[rid] = []
        self.length[rid] = 0
        self.dropped[rid] = 0
        self.head[rid] = -(-sinks // self.page_size)

    def append(self, rid: Hashable) -> AppendPlan:
        """Place one new row at the end of request ``rid``."""
        P = self.page_size
        row = self.length[rid]
        off = row % P
        pages = self.pages[rid]
        plan_copy = None
        new_page = False
        if off == 0:
            pages.append(self.pool.alloc())
            new_page = True
            self._updates.append((rid, row // P, pages[-1]))
        else:
            tail = pages[-1]
            if self.pool.ref[tail] > 1:
                fresh = self.pool.alloc()
                self.pool.unref(tail)
                pages[-1] = fresh
                plan_copy = (tail, fresh)
                self._updates.append((rid, row // P, fresh))
        page = pages[-1]
        self.length[rid] = row + 1
        return AppendPlan(rid, row, page, off, page * P + off, plan_copy, new_page)

    def trim(self, rid: Hashable, keep_from: int) -> List[int]:
        """Release pages lying wholly before row ``keep_from``, sink pages
        excepted; returns them."""
        P = self.page_size
        pages = self.pages[rid]
        h = self.head[rid]
        out = []
        while len(pages) > h and (h + self.dropped[rid] + 1) * P <= keep_from:
            p = pages.pop(h)
            self.pool.unref(p)
            self._updates.append((rid, h + self.dropped[rid], -1))
            self.dropped[rid] += 1
            out.append(p)
        return out

    def fork(self, src: Hashable, dst: Hashable) -> None:
        if dst in self.pages:
            raise KeyError(f"request {dst!r} exists")
        self.pages[dst] = list(self.pages[src])
        self.length[dst] = self.length[src]
        self.dropped[dst] = self.dropped[src]
        self.head[dst] = self.head[src]
        for p in self.pages[dst]:
            self.pool.incref(p)
        self._updates.extend((dst, j, p) for j, p in enumerate(self.table(dst)))

    def release(self, rid: Hashable) -> None:
        self._updates.extend((rid, self.logical_page(rid, i), -1)
                             for i in range(len(self.pages[rid])))
        for p in self.pages.pop(rid):
            self.pool.unref(p)
        del self.length[rid]
        del self.dropped[rid]
        del self.head[rid]

    def rewind(self, rid: Hashable, n: int) -> List[int]:
        """Drop the newest ``n`` rows; pages left without a row are released."""
        if not 0 <= n <= self.length[rid]:
            raise ValueError("cannot rewind past the start")
        P = self.page_size
        new_len = self.length[rid] - n
        d, h = self.dropped[rid], self.head[rid]
        if d > 0 and new_len < (h + d) * P:
            raise ValueError("cannot rewind into released pages")
        keep = -(-new_len // P) - d
        pages = self.pages[rid]
        out = []
        while len(pages) > keep:
            self._updates.append((rid, self.logical_page(rid, len(pages) - 1), -1))
            p = pages.pop()
            self.pool.unref(p)
            out.append(p)
        self.length[rid] = new_len
        return out

    # -- queries -----------------------------------------------------------------
    def used(self) -> int:
        return self.pool.used()

    def translate(self, rid: Hashable, row: int) -> Tuple[int, int]:
        """(physical page, offset) of a readable logical row."""
        P = self.page_size
        j, h, d = row // P, self.head[rid], self.dropped[rid]
        if not 0 <= row < self.length[rid] or h <= j < h + d:
            raise IndexError(f"row {row} of request {rid!r} is not readable")
        return self.pages[rid][j if j < h else j - d], row % P

    def logical_page(self, rid: Hashable, i: int) -> int:
        """Logical page index of the ``i``-th live page of a request."""
        return i if i < self.head[rid] else i + self.dropped[rid]

    def table(self, rid: Hashable) -> List[int]:
        """Block table indexed by logical page; -1 for released pages."""
        h, pages = self.head[rid], self.pages[rid]
        return list(pages[:h]) + [-1] * self.dropped[rid] + list(pages[h:])

    @staticmethod
    def pages_needed(cached_len: int, device_len: int, page_size: int) -> int:
        """Fresh pages to grow a request from ``cached_len`` to ``device_len`` rows."""
        return -(-device_len // page_size) - (-(-cached_len // page_size))

    # -- device operands ---------------------------------------------------------
    def block_tables(self, rids: Iterable[Hashable], stride: int) -> np.ndarray:
        rids = list(rids)
        out = np.full((len(rids), stride), -1, dtype=np.int32)
        for i, rid in enumerate(rids):
            t = self.table(rid)
            if len(t) > stride:
                raise ValueError(f"request {rid!r} needs {len(t)} table entries > {stride}")
            out[i, :len(t)] = t
        return out

    def slot_table(self, rids: Iterable[Hashable], stride: int, dummy_slot: int) -> np.ndarray:
        """Raw token-slot table: entry ``[i, r]`` is the flat slot of row ``r``.

        Rows that are not readable, and one extra dummy row at the end, hold
        ``dummy_slot``.
        """
        rids = list(rids)
        P = self.page_size
        out = np.full((len(rids) + 1, stride), dummy_slot, dtype=np.int64)
        for i, rid in enumerate(rids):
            L = self.length[rid]
            if L > stride:
                raise ValueError(f"request {rid!r} has {L} rows > {stride}")
            for j, p in enumerate(self.pages[rid]):
                r0 = self.logical_page(rid, j) * P
                r1 = min(r0 + P, L)
                out[i, r0:r1] = p * P + np.arange(r1 - r0)
        if out.max(initial=0) >= 2**31:
            raise ValueError("slot does not fit int32")
        return out.astype(np.int32)

    def plan_step(self, rids: Iterable[Hashable]) -> StepPlan:
        """Append one row to every request; returns slots and copy lists.

        All-or-nothing: if any append runs out of pages, the appends already
        made in this call are rewound and ``OutOfPages`` propagates.
        """
        rids = list(rids)
        plans: List[AppendPlan] = []
        try:
            for rid in rids:
                plans.append(self.append(rid))
        except OutOfPages:
            for p in reversed(plans):
                self._undo(p)
            raise
        copies = [p.copy for p in plans if p.copy is not None]
        return StepPlan(
            rids=rids,
            slots=np.array([p.slot for p in plans], dtype=np.int32),
            copy_src=np.array([c[0] for c in copies], dtype=np.int32),
            copy_dst=np.array([c[1] for c in copies], dtype=np.int32),
            context_lens=np.array([self.length[r] for r in rids], dtype=np.int32))

    def _undo(self, plan: AppendPlan) -> None:
        rid = plan.rid
        pages = self.pages[rid]
        self.length[rid] = plan.row
        j = plan.row // self.page_size
        if plan.new_page:
            self.pool.unref(pages.pop())
            self._updates.append((rid, j, -1))
        elif plan.copy is not None:
            src, dst = plan.copy
            self.pool.incref(src)
            pages[-1] = src
            self.pool.unref(dst)
            self._updates.append((rid, j, src))

    def take_table_updates(self, row_of: Dict[Hashable, int]):
        """The table changes since the last call, as int32 arrays (rows, logical
        pages, pages) for one scatter: the last change of each cell only, in the
        order the cells were first changed.  ``row_of`` gives each request's table
        row; changes of requests it does not name are dropped."""
        last: Dict[Tuple[int, int], int] = {}
        for rid, j, p in self._updates:
            r = row_of.get(rid)
            if r is not None:
                last[(r, j)] = p
        self._updates.clear()
        cells = list(last)
        return (np.array([c[0] for c in cells], dtype=np.int32),
                np.array([c[1] for c in cells], dtype=np.int32),
                np.array([last[c] for c in cells], dtype=np.int32))

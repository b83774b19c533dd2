"""Host block allocator: free list, reference counts, copy-on-write, window trim.

Plain host code.  It decides where each new K/V row goes and which pages must
be copied first; it never touches K/V data.  Its output is what the kernels
consume: int32 block tables (-1 where a page was released), raw token-slot
tables, the slot of every new row and the list of pages to copy.

The rules are those of the page table in the silicon-compiler chapter 15
(section "The model"), stated here as properties of a request's table:

* a request's table is indexed by logical page (row // page_size); a cell
  holds a physical page or -1 once the window released it;
* a new row whose logical page has no cell yet takes a fresh page; a new row
  that lands in a page other requests also hold (reference count above one)
  takes a fresh page that receives a whole-page copy of the shared one first,
  and the request's reference moves from the shared page to its copy (lazy
  copy-on-write); otherwise the row is written in place.  A failed allocation
  raises ``OutOfPages`` and changes nothing;
* trimming at ``keep_from`` releases every page all of whose slots lie before
  ``keep_from`` -- page j goes when ``(j + 1) * page_size <= keep_from`` -- so
  a page that still holds, or will receive, a needed row stays.  After a decode
  step at context ``L`` with window ``W`` the next step needs rows
  ``>= L + 1 - W``;
* with ``sinks`` rows kept at the start (the attention-sink exercise of that
  chapter, section "Exercises"), the first ``ceil(sinks / P)`` cells are never
  released; the released cells form a hole between them and the window;
* ``fork`` shares every page, a partial tail included (one more reference
  each); ``release`` drops the request's references;
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

Every change to a table cell (a page mapped, remapped by copy-on-write or
released) is also recorded as an update ``(request, logical page, physical
page or -1)``; ``take_table_updates`` hands them over as index lists for one
device scatter (``pa_update_tables``), the way the mini-sglang page writes new
table cells with one scatter instead of rebuilding tables on the host.

``unshared`` tells whether every page a set of requests holds has a single
reference: then no page is attended twice in their decode call, which the
decode entry point can use as its cache hint (``pa_decode_hinted``).
"""
from __future__ import annotations

from collections import deque
from collections.abc import Mapping
from dataclasses import dataclass
from typing import Callable, Dict, Hashable, Iterable, Iterator, List, Optional, Sequence, Tuple

import numpy as np


class OutOfPages(RuntimeError):
    """No free page is left in the pool."""


RELEASED = -1


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
    unshared: bool = False        # after the step, every page of the batch has one holder


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

    def take(self, p: int) -> None:
        """Hold page ``p`` once more; a free page leaves the free list."""
        if not 0 <= p < self.num_pages:
            raise IndexError(f"page {p} is outside the pool of {self.num_pages}")
        if self.ref[p] == 0:
            self._free.remove(p)
        self.ref[p] += 1

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


@dataclass
class _Request:
    """One request's table: ``cells[j]`` is the page of logical page j, or -1."""
    cells: List[int]
    rows: int          # rows written
    head: int          # leading cells kept for sink rows, never released by a trim
    floor: int         # cells [head, floor) were released by the window


class _View(Mapping):
    """Read-only per-request mapping computed from the request records."""

    def __init__(self, reqs: Dict[Hashable, _Request], get: Callable[[_Request], object]):
        self._reqs, self._get = reqs, get

    def __getitem__(self, rid):
        return self._get(self._reqs[rid])

    def __iter__(self) -> Iterator:
        return iter(self._reqs)

    def __len__(self) -> int:
        return len(self._reqs)


class PagedKVCache:
    """Per-request block tables over one ``BlockAllocator``."""

    def __init__(self, num_pages: int, page_size: int, policy: str = "lifo",
                 free_order: Optional[Sequence[int]] = None):
        if page_size <= 0:
            raise ValueError("page_size must be positive")
        self.page_size = page_size
        self.pool = BlockAllocator(num_pages, policy, free_order)
        self._reqs: Dict[Hashable, _Request] = {}
        self._updates: List[Tuple[Hashable, int, int]] = []   # (request, logical page, page)

    # -- read-only views ---------------------------------------------------------
    @property
    def pages(self) -> Mapping:
        """Live pages of each request, in logical order."""
        return _View(self._reqs, lambda r: [c for c in r.cells if c != RELEASED])

    @property
    def length(self) -> Mapping:
        """Rows written to each request."""
        return _View(self._reqs, lambda r: r.rows)

    @property
    def dropped(self) -> Mapping:
        """Pages each request released to the window."""
        return _View(self._reqs, lambda r: r.floor - r.head)

    @property
    def head(self) -> Mapping:
        """Leading pages each request keeps for its sink rows."""
        return _View(self._reqs, lambda r: r.head)

    # -- lifecycle -------------------------------------------------------------
    def new(self, rid: Hashable, sinks: int = 0) -> None:
        if rid in self._reqs:
            raise KeyError(f"request {rid!r} exists")
        if sinks < 0:
            raise ValueError("sinks must be >= 0")
        head = -(-sinks // self.page_size)
        self._reqs[rid] = _Request(cells=[], rows=0, head=head, floor=head)

    def adopt(self, rid: Hashable, table: Sequence[int], rows: int, sinks: int = 0) -> None:
        """Register a request whose table was built elsewhere (a restored cache, or a
        batch laid out by another host): ``table`` holds a page or -1 per logical page,
        ``rows`` rows are written.  Each page named takes one reference.  The -1 cells
        must lie after the sink pages and before the live window, as a trim leaves them."""
        if rid in self._reqs:
            raise KeyError(f"request {rid!r} exists")
        P = self.page_size
        n = -(-rows // P)
        cells = [int(c) for c in list(table)[:n]]
        if len(cells) < n:
            raise ValueError(f"a table of {len(cells)} cells cannot hold {rows} rows")
        head = -(-sinks // P)
        live = [j for j in range(min(head, n), n) if cells[j] != RELEASED]
        floor = live[0] if live else n
        if any(cells[j] == RELEASED for j in range(min(head, n))) or \
                any(cells[j] == RELEASED for j in range(floor, n)):
            raise ValueError("released cells must form one run after the sink pages")
        for c in cells:
            if c != RELEASED:
                self.pool.take(c)
        self._reqs[rid] = _Request(cells=cells, rows=rows, head=head, floor=max(floor, head))

    def _placement(self, r: _Request, ref_of: Callable[[int], int]) -> Tuple[str, int]:
        """How the next row of ``r`` is placed: ("open", -1) for a row with no page yet,
        ("cow", page) for a row landing in a page held elsewhere too, else ("in", page)."""
        j = r.rows // self.page_size
        if j == len(r.cells):
            return "open", RELEASED
        page = r.cells[j]
        return ("cow" if ref_of(page) > 1 else "in"), page

    def append(self, rid: Hashable) -> AppendPlan:
        """Place one new row at the end of request ``rid``."""
        r = self._reqs[rid]
        P = self.page_size
        row, j = r.rows, r.rows // P
        kind, page = self._placement(r, lambda p: self.pool.ref[p])
        copy = None
        if kind == "open":
            page = self.pool.alloc()
            r.cells.append(page)
            self._updates.append((rid, j, page))
        elif kind == "cow":
            fresh = self.pool.alloc()         # raises before anything changes
            self.pool.unref(page)
            copy = (page, fresh)
            r.cells[j] = page = fresh
            self._updates.append((rid, j, fresh))
        r.rows = row + 1
        return AppendPlan(rid, row, page, row % P, page * P + row % P, copy, kind == "open")

    def trim(self, rid: Hashable, keep_from: int) -> List[int]:
        """Release pages lying wholly before row ``keep_from``, sink pages excepted;
        returns them, oldest first."""
        r = self._reqs[rid]
        stop = min(keep_from // self.page_size, len(r.cells))
        out = []
        for j in range(r.floor, stop):
            out.append(r.cells[j])
            r.cells[j] = RELEASED
            self.pool.unref(out[-1])
            self._updates.append((rid, j, RELEASED))
        r.floor = max(r.floor, stop)
        return out

    def fork(self, src: Hashable, dst: Hashable) -> None:
        if dst in self._reqs:
            raise KeyError(f"request {dst!r} exists")
        s = self._reqs[src]
        self._reqs[dst] = _Request(cells=list(s.cells), rows=s.rows, head=s.head, floor=s.floor)
        for c in s.cells:
            if c != RELEASED:
                self.pool.incref(c)
        self._updates.extend((dst, j, c) for j, c in enumerate(s.cells))

    def release(self, rid: Hashable) -> None:
        r = self._reqs.pop(rid)
        for j, c in enumerate(r.cells):
            if c != RELEASED:
                self._updates.append((rid, j, RELEASED))
                self.pool.unref(c)

    def rewind(self, rid: Hashable, n: int) -> List[int]:
        """Drop the newest ``n`` rows; pages left without a row are released (newest
        first, which is the order returned)."""
        r = self._reqs[rid]
        if not 0 <= n <= r.rows:
            raise ValueError("cannot rewind past the start")
        rows = r.rows - n
        if r.floor > r.head and rows < r.floor * self.page_size:
            raise ValueError("cannot rewind into released pages")
        keep = -(-rows // self.page_size)
        out = []
        for j in range(len(r.cells) - 1, keep - 1, -1):
            self._updates.append((rid, j, RELEASED))
            out.append(r.cells[j])
            self.pool.unref(r.cells[j])
        del r.cells[keep:]
        r.rows = rows
        return out

    # -- queries -----------------------------------------------------------------
    def used(self) -> int:
        return self.pool.used()

    def translate(self, rid: Hashable, row: int) -> Tuple[int, int]:
        """(physical page, offset) of a readable logical row."""
        r = self._reqs[rid]
        j = row // self.page_size
        if not 0 <= row < r.rows or r.cells[j] == RELEASED:
            raise IndexError(f"row {row} of request {rid!r} is not readable")
        return r.cells[j], row % self.page_size

    def logical_page(self, rid: Hashable, i: int) -> int:
        """Logical page index of the ``i``-th live page of a request."""
        return [j for j, c in enumerate(self._reqs[rid].cells) if c != RELEASED][i]

    def table(self, rid: Hashable) -> List[int]:
        """Block table indexed by logical page; -1 for released pages."""
        return list(self._reqs[rid].cells)

    def unshared(self, rids: Iterable[Hashable]) -> bool:
        """True when every page these requests hold has one reference, so no page is
        read twice by their decode call."""
        return all(self.pool.ref[c] == 1 for rid in rids for c in self._reqs[rid].cells
                   if c != RELEASED)

    @staticmethod
    def pages_needed(cached_len: int, device_len: int, page_size: int) -> int:
        """Fresh pages to grow a request from ``cached_len`` to ``device_len`` rows."""
        return -(-device_len // page_size) - (-(-cached_len // page_size))

    # -- device operands ---------------------------------------------------------
    def block_tables(self, rids: Iterable[Hashable], stride: int) -> np.ndarray:
        rids = list(rids)
        out = np.full((len(rids), stride), RELEASED, dtype=np.int32)
        for i, rid in enumerate(rids):
            cells = self._reqs[rid].cells
            if len(cells) > stride:
                raise ValueError(f"request {rid!r} needs {len(cells)} table entries > {stride}")
            out[i, :len(cells)] = cells
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
            r = self._reqs[rid]
            if r.rows > stride:
                raise ValueError(f"request {rid!r} has {r.rows} rows > {stride}")
            for j, c in enumerate(r.cells):
                if c != RELEASED:
                    r0, r1 = j * P, min((j + 1) * P, r.rows)
                    out[i, r0:r1] = c * P + np.arange(r1 - r0)
        if out.max(initial=0) >= 2**31:
            raise ValueError("slot does not fit int32")
        return out.astype(np.int32)

    def plan_step(self, rids: Iterable[Hashable]) -> StepPlan:
        """Append one row to every request; returns slots and copy lists.

        All-or-nothing: the placements are decided first, counting the fresh pages
        they take (a copy-on-write in the batch lowers the count of the page it
        leaves for the requests after it); if the free list cannot supply them,
        ``OutOfPages`` is raised and nothing changes.
        """
        rids = list(rids)
        if len(set(rids)) != len(rids):
            raise ValueError("a step appends one row per request; a request is named twice")
        leaving: Dict[int, int] = {}
        fresh = 0
        for rid in rids:
            kind, page = self._placement(self._reqs[rid],
                                         lambda p: self.pool.ref[p] - leaving.get(p, 0))
            if kind == "cow":
                leaving[page] = leaving.get(page, 0) + 1
            fresh += kind != "in"
        if fresh > self.pool.free_count():
            raise OutOfPages(f"the step needs {fresh} fresh pages, "
                             f"{self.pool.free_count()} are free")
        plans = [self.append(rid) for rid in rids]
        copies = [p.copy for p in plans if p.copy is not None]
        return StepPlan(
            rids=rids,
            slots=np.array([p.slot for p in plans], dtype=np.int32),
            copy_src=np.array([c[0] for c in copies], dtype=np.int32),
            copy_dst=np.array([c[1] for c in copies], dtype=np.int32),
            context_lens=np.array([self._reqs[r].rows for r in rids], dtype=np.int32),
            unshared=self.unshared(rids))

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

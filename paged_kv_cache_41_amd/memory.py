"""Memory and fragmentation report of a paged K/V cache (host only).

Three measures from the pages, over the host allocator's state:

* Capacity and waste of contiguous reservation against paging: with
  contiguous reservation every request holds ``max_context`` rows; with pages
  it holds its rows rounded up to whole pages (the silicon-compiler chapter 15
  "A Paged KV Cache and Sliding-Window Attention", section "Running example B",
  part 1, with its memory table; the cookbook notebook "PagedAttention block
  allocator", section "Waste measurement", whose paged waste is bounded by
  ``1 / page_size``).
* Admission: requests taken in order until the pool cannot hold the next one
  (``admit``), which gives the chapter's "requests held" column.
* Fragmentation (the tiny-llm page "Paged KV Cache", section "What Paging
  Changes"): at a snapshot, the unused slots of the final live page of every
  request divided by all slots of the live pages; a run reports the snapshot
  where those unused slots peak.  Free pool capacity is not in the fraction; it
  is reported apart as live and free pages.

With shared pages (forks) each request counts the pages it holds, as each
request's cache would; ``pages_in_use`` counts physical pages once.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Hashable, Iterable, List, Optional

from .alloc import OutOfPages, PagedKVCache


def contiguous_waste(lengths: Iterable[int], max_context: int) -> float:
    """1 - rows used / rows reserved when every request reserves ``max_context`` rows."""
    lengths = list(lengths)
    return 1.0 - sum(lengths) / (max_context * len(lengths))


def paged_waste(lengths: Iterable[int], page_size: int) -> float:
    """1 - rows used / rows of the pages holding them, one request after another."""
    lengths = list(lengths)
    cache = PagedKVCache(sum(-(-L // page_size) for L in lengths) or 1, page_size)
    for i, L in enumerate(lengths):
        cache.new(i)
        for _ in range(L):
            cache.append(i)
    used = sum(cache.length.values())
    return 1.0 - used / (cache.used() * page_size)


@dataclass
class Admission:
    """Requests admitted in order until the next one does not fit."""
    scheme: str
    held: int
    rows_used: int
    rows_reserved: int

    @property
    def wasted(self) -> float:
        return 1.0 - self.rows_used / self.rows_reserved if self.rows_reserved else 0.0


def admit(lengths: Iterable[int], pool_rows: int, page_size: Optional[int] = None,
          max_context: Optional[int] = None) -> Admission:
    """Admit requests of ``lengths`` rows in order into ``pool_rows`` rows.

    Contiguous (``max_context`` given): each request reserves ``max_context``
    rows.  Paged (``page_size`` given): each request appends its rows through
    the allocator; the first one that runs out of pages is released and ends
    the admission.
    """
    lengths = list(lengths)
    if max_context is not None:
        n = min(len(lengths), pool_rows // max_context)
        return Admission("contiguous", n, sum(lengths[:n]), n * max_context)
    assert page_size is not None
    cache = PagedKVCache(pool_rows // page_size, page_size)
    n = used = 0
    for i, L in enumerate(lengths):
        cache.new(i)
        try:
            for _ in range(L):
                cache.append(i)
        except OutOfPages:
            cache.release(i)
            break
        n += 1
        used += L
    return Admission(f"paged{page_size}", n, used, cache.used() * page_size)


@dataclass
class Snapshot:
    requests: int
    live_page_slots: int       # page_size x pages held, summed over requests
    unused_last_page_slots: int
    pages_in_use: int          # physical pages, each counted once
    free_pages: int

    @property
    def fragmentation(self) -> float:
        return self.unused_last_page_slots / self.live_page_slots if self.live_page_slots else 0.0


def snapshot(cache: PagedKVCache, rids: Optional[Iterable[Hashable]] = None) -> Snapshot:
    """The cache's live and unused slots now (every request, or ``rids``)."""
    P = cache.page_size
    rids = list(cache.pages) if rids is None else list(rids)
    live = unused = 0
    for rid in rids:
        pages = cache.pages[rid]
        live += len(pages) * P
        if pages:
            L = cache.length[rid]
            # the final live page holds rows up to L - 1; its other slots are unused
            unused += (-L) % P
    return Snapshot(len(rids), live, unused, cache.used(), cache.pool.free_count())


class FragmentationTracker:
    """Keeps the snapshot with the most unused final-page slots."""

    def __init__(self, row_bytes: int = 0):
        self.row_bytes = row_bytes
        self.worst: Optional[Snapshot] = None
        self.snapshots = 0

    def observe(self, cache: PagedKVCache, rids=None) -> Snapshot:
        s = snapshot(cache, rids)
        self.snapshots += 1
        if self.worst is None or s.unused_last_page_slots > self.worst.unused_last_page_slots:
            self.worst = s
        return s

    def report(self) -> Dict[str, float]:
        w = self.worst or Snapshot(0, 0, 0, 0, 0)
        return {"snapshots": self.snapshots, "fragmentation": w.fragmentation,
                "unused_last_page_slots": w.unused_last_page_slots,
                "unused_bytes": w.unused_last_page_slots * self.row_bytes,
                "live_page_slots": w.live_page_slots, "pages_in_use": w.pages_in_use,
                "free_pages": w.free_pages}


def example_b_table(lengths: List[int], pool_rows: int = 8192, max_context: int = 2048,
                    pages=(1, 4, 16, 64, 256)) -> List[Admission]:
    """The chapter's memory table: contiguous reservation, then each page size."""
    return [admit(lengths, pool_rows, max_context=max_context)] + \
        [admit(lengths, pool_rows, page_size=p) for p in pages]


if __name__ == "__main__":
    import random
    r = random.Random(11)
    lens = [min(2048, max(16, int(r.lognormvariate(5.2, 0.9)))) for _ in range(400)]
    print("scheme      held  rows used  rows reserved  wasted")
    for a in example_b_table(lens):
        print(f"{a.scheme:10s} {a.held:5d} {a.rows_used:10d} {a.rows_reserved:14d}  {100 * a.wasted:5.1f}%")
    r = random.Random(0)
    lens = [max(4, int(r.lognormvariate(4.5, 0.8))) for _ in range(100)]
    pre, paged = contiguous_waste(lens, 4096), paged_waste(lens, 16)
    print(f"reserve 4096 each: {100 * pre:.1f}% wasted; pages of 16: {100 * paged:.1f}% wasted")

"""Bit-exact reference of the table update: per-step changes to block and slot tables.

The mini-sglang page (part 4, the section on writing the page table) fills a
request's new table cells with one scatter, ``table[row, position] = slot``,
from index lists built on the host, rather than one write per request.  Here
the same scatter keeps both table kinds in step with the allocator: each
update names a table row, a logical page ``j`` and the physical page now
behind it (``-1``: released).  The block table gets that page (or ``-1``) in
cell ``[row, j]``; the slot table gets, for the ``page_size`` positions
``j * P .. j * P + P - 1`` of that row, the flat slots ``page * P + k`` (the
page-to-token expansion of that section: a whole page of positions, spare
capacity included), or ``dummy_slot`` for a released page (the mini-sglang
dummy row's slot: real memory that is never allocated).

An update outside a table (row or column) is skipped for that table.  Two
updates of one cell in one call are a caller error.  Works on plain integer
arrays and returns new ones.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def update_tables(block_tables: Optional[np.ndarray], slot_table: Optional[np.ndarray],
                  rows, logical_pages, pages, page_size: int, dummy_slot: int):
    cells = list(zip((int(r) for r in rows), (int(j) for j in logical_pages)))
    if len(set(cells)) != len(cells):
        raise ValueError("two updates of one table cell")
    bt = None if block_tables is None else np.array(block_tables, copy=True)
    st = None if slot_table is None else np.array(slot_table, copy=True)
    for (r, j), p in zip(cells, (int(x) for x in pages)):
        if bt is not None and 0 <= r < bt.shape[0] and 0 <= j < bt.shape[1]:
            bt[r, j] = p if p >= 0 else -1
        if st is not None and 0 <= r < st.shape[0]:
            for k in range(page_size):
                pos = j * page_size + k
                if 0 <= pos < st.shape[1]:
                    st[r, pos] = p * page_size + k if p >= 0 else dummy_slot
    return bt, st

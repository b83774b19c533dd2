"""CPU oracle for paged decode attention, the K/V slot scatter and the page copy.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls this
package.  Only the tests, the smoke check of ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` use it.  It shares no code, table or helper with
the HIP path; it takes plain NumPy arrays.

What it computes, and from which passage:

* ``attention.decode`` -- gather every attended row through the block table
  into contiguous K/V (the dense-gather checkpoint of the tiny-llm page
  "Paged KV Cache", section "Correctness Checkpoint: Gather Pages for Dense
  Attention"; the row lookup of the silicon-compiler chapter 15, section "The
  model", ``PageTable.rows``) and run plain single-query softmax attention in
  float64 over the last ``min(L, W)`` rows (same chapter, the window rule of
  ``PagedChip.generate``).
* ``attention.prefill`` -- several query tokens per sequence (a prefill
  chunk or a verify step; the tiny-llm page, section "Prefill with Pages"):
  each query attends, causally and within the window counted from its own
  row, the rows a single-query step at its position would.
* ``kvstore.store_kv`` -- write each new row to its flat slot (the
  mini-sglang page, section on the KV buffer and its store call).
* ``kvstore.copy_pages`` -- whole-page copy for copy-on-write (silicon chapter
  15, section "The model", ``PageTable.append``).
* ``tables.update_tables`` -- the per-step scatter of table changes into block
  and slot tables (the mini-sglang page, section on writing the page table).
* ``shadow`` -- the page-table semantics as plain per-request row lists, and
  the closed-form page counts of the window rule (silicon chapter 15,
  sections "The problem", "Tests", check 3).

Every function is pinned by tests that do not reuse its formula: values the
pages print, closed forms, brute force on tiny inputs, library routines and
invariances (see ``tests/test_oracle_*.py``).  No function here is parity
unpinned.
"""
from . import attention, kvstore, numerics, shadow, tables

__all__ = ["attention", "kvstore", "numerics", "shadow", "tables"]

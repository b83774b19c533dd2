"""Decode attention over a paged K/V pool: gather, then dense float64 attention.

The computation, step by step, for one sequence ``s`` with context length
``L`` (which counts the token being decoded, whose K/V row is already stored
at logical row ``L - 1``):

1. Live range.  With a window ``W > 0`` the step attends the new token and at
   most ``W - 1`` earlier ones: rows ``[L - min(L, W), L)``; without a window
   rows ``[0, L)``.  (silicon-compiler chapter 15, section "The model",
   ``PagedChip.generate``: ``nc = min(L, W)``, ``lo = L - nc``.)
2. Address.  Logical row ``i`` lives in page ``table[i // P]`` at offset
   ``i % P``.  (llm-systems-cookbook notebook "PagedAttention block allocator",
   section "Sequence block table"; silicon chapter 15 ``PageTable.rows``,
   where released front pages are counted by ``dropped``; here the table is
   indexed by logical page and a released page reads -1.)  A live row that
   maps to no page is an error, as reading a released row is in ``rows``.
3. Dense attention per query head ``h``: kv head ``g = h // (Hq / Hkv)``,
   logits ``z_i = scale * <q_h, k_i,g>``, weights ``exp(z_i - max z)``, output
   ``sum_i w_i v_i,g / sum_i w_i``.  (The tiny-llm page keeps the dense
   attention equation as the checkpoint for paged storage, section "How This
   Maps to tiny-llm".)

``L == 0`` yields a zero output row.

Several query tokens per sequence (a prefill chunk, or the drafted tokens a
speculative step verifies; the tiny-llm page "Paged KV Cache", section
"Prefill with Pages", where a chunk's rows are stored into pages first):
the ``n`` queries of a sequence of ``L`` rows are its last ``n`` rows, query
``i`` sits at row ``p = L - n + i`` and attends exactly what a single-query
step at context ``p + 1`` attends (causal, and within the window counted from
its own row).  A query with ``p < 0`` (more queries than rows) gets zeros.

Attention sinks (silicon-compiler chapter 15, section "Exercises", exercise 3):
with ``S`` sink rows and a window ``W`` the step attends the first ``S`` rows
and the last ``W - S`` rows, so the context is still ``W`` rows once ``L``
exceeds ``W``; while ``L <= W`` every row is attended.  ``0 <= S < W`` keeps
the new token among the attended rows.
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np

from .numerics import to_f64


def live_rows(L: int, window: int) -> tuple[int, int]:
    """First and one-past-last attended logical row."""
    if window > 0:
        return L - min(L, window), L
    return 0, L


def attended_rows(L: int, window: int, sinks: int = 0) -> list:
    """Logical rows attended by a sequence of ``L`` rows, in increasing order."""
    if window <= 0 or sinks <= 0:
        lo, hi = live_rows(L, window)
        return list(range(lo, hi))
    if not sinks < window:
        raise ValueError(f"{sinks} sink rows need a window of more than {sinks} rows")
    lo, hi = live_rows(L, window - sinks)
    return sorted(set(range(min(sinks, L))) | set(range(lo, hi)))


def gather_rows(pool_bits: np.ndarray, table_row: np.ndarray, rows, dtype: str) -> np.ndarray:
    """Logical rows ``rows`` of one sequence through its block table, in float64."""
    num_pages, P = pool_bits.shape[0], pool_bits.shape[1]
    out = np.empty((len(rows),) + pool_bits.shape[2:], dtype=np.float64)
    for n, i in enumerate(rows):
        page = int(table_row[i // P])
        if not 0 <= page < num_pages:
            raise IndexError(f"row {i} maps to page {page}, outside the pool of {num_pages}")
        out[n] = to_f64(pool_bits[page, i % P], dtype)
    return out


def gather(pool_bits: np.ndarray, table_row: np.ndarray, lo: int, hi: int,
           dtype: str) -> np.ndarray:
    """Rows ``lo..hi-1`` of one sequence through its block table, in float64.

    ``pool_bits`` is ``[num_pages, page_size, kv_heads, head_dim]`` raw bits.
    Returns ``[hi - lo, kv_heads, head_dim]``.
    """
    num_pages, P = pool_bits.shape[0], pool_bits.shape[1]
    out = np.empty((hi - lo,) + pool_bits.shape[2:], dtype=np.float64)
    for n, i in enumerate(range(lo, hi)):
        page = int(table_row[i // P])
        if not 0 <= page < num_pages:
            raise IndexError(f"row {i} maps to page {page}, outside the pool of {num_pages}")
        out[n] = to_f64(pool_bits[page, i % P], dtype)
    return out


def kv_head_of(h: int, q_heads: int, kv_heads: int) -> int:
    """Consecutive query heads share one kv head."""
    return h // (q_heads // kv_heads)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query vector over rows ``K``, ``V`` (float64)."""
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def decode(q_bits: np.ndarray, k_pool_bits: np.ndarray, v_pool_bits: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray, page_size: int,
           window: int, scale: float, dtype: str,
           seqs: Optional[Iterable[int]] = None, sinks: int = 0) -> np.ndarray:
    """Float64 output ``[len(seqs), q_heads, head_dim]`` of one decode step.

    ``q_bits`` is ``[num_seqs, q_heads, head_dim]`` raw bits; ``block_tables``
    is ``[>= num_seqs, stride]`` integers; ``seqs`` selects sequences (all by
    default); ``sinks`` rows at the start are kept besides the window.
    """
    assert k_pool_bits.shape[1] == page_size and v_pool_bits.shape == k_pool_bits.shape
    num_seqs, q_heads, head_dim = q_bits.shape
    kv_heads = k_pool_bits.shape[2]
    assert q_heads % kv_heads == 0 and k_pool_bits.shape[3] == head_dim
    seqs = list(range(num_seqs)) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), q_heads, head_dim), dtype=np.float64)
    for n, s in enumerate(seqs):
        L = int(context_lens[s])
        if L < 0:
            raise ValueError(f"negative context length {L}")
        if L == 0:
            continue
        if sinks > 0 and window > 0:
            rows = attended_rows(L, window, sinks)
            K = gather_rows(k_pool_bits, block_tables[s], rows, dtype)
            V = gather_rows(v_pool_bits, block_tables[s], rows, dtype)
        else:
            lo, hi = live_rows(L, window)
            K = gather(k_pool_bits, block_tables[s], lo, hi, dtype)
            V = gather(v_pool_bits, block_tables[s], lo, hi, dtype)
        qs = to_f64(q_bits[s], dtype)
        for h in range(q_heads):
            g = kv_head_of(h, q_heads, kv_heads)
            out[n, h] = attend(qs[h], K[:, g, :], V[:, g, :], scale)
    return out


def query_position(L: int, n: int, i: int) -> int:
    """Row of the ``i``-th of the ``n`` query tokens of a sequence of ``L`` rows."""
    return L - n + i


def prefill(q_bits: np.ndarray, k_pool_bits: np.ndarray, v_pool_bits: np.ndarray,
            block_tables: np.ndarray, context_lens: np.ndarray, q_start: np.ndarray,
            page_size: int, window: int, scale: float, dtype: str,
            rows: Optional[Iterable[int]] = None) -> np.ndarray:
    """Float64 output ``[len(rows), q_heads, head_dim]`` for query rows ``rows``.

    ``q_bits`` is ``[num_q, q_heads, head_dim]`` raw bits; the query rows of
    sequence ``s`` are ``q_start[s] .. q_start[s + 1] - 1``; ``rows`` selects
    query rows (all by default).
    """
    num_q, q_heads, head_dim = q_bits.shape
    kv_heads = k_pool_bits.shape[2]
    assert q_heads % kv_heads == 0 and k_pool_bits.shape[3] == head_dim
    q_start = np.asarray(q_start, dtype=np.int64)
    B = len(q_start) - 1
    assert q_start[0] == 0 and q_start[B] == num_q and np.all(np.diff(q_start) >= 0)
    rows = list(range(num_q)) if rows is None else list(rows)
    out = np.zeros((len(rows), q_heads, head_dim), dtype=np.float64)
    for n_out, r in enumerate(rows):
        s = int(np.searchsorted(q_start, r, side="right")) - 1
        n = int(q_start[s + 1] - q_start[s])
        p = query_position(int(context_lens[s]), n, r - int(q_start[s]))
        if p < 0:
            continue
        lo, hi = live_rows(p + 1, window)
        K = gather(k_pool_bits, block_tables[s], lo, hi, dtype)
        V = gather(v_pool_bits, block_tables[s], lo, hi, dtype)
        qs = to_f64(q_bits[r], dtype)
        for h in range(q_heads):
            g = kv_head_of(h, q_heads, kv_heads)
            out[n_out, h] = attend(qs[h], K[:, g, :], V[:, g, :], scale)
    return out

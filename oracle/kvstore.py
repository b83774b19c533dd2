"""Bit-exact reference of the two data-movement operations of a decode step.

``store_kv``: each new row ``t`` goes to flat slot ``slot[t]`` of the pool
viewed as ``[num_pages * page_size, kv_heads, head_dim]`` (the mini-sglang
page, section on the KV buffer: the pool is flattened to token rows before
the store, and the store indexes its first axis with the slot list).  A
negative slot is skipped.  Two new rows for one slot are a caller error.

``copy_pages``: ``pool[dst[i]] = pool[src[i]]`` for every pair, whole pages,
K and V (silicon-compiler chapter 15, section "The model", the copy-on-write
branch of ``PageTable.append``, which copies the whole shared page before the
row is written).  Targets must be distinct and disjoint from the sources, so
the order of the pairs cannot matter.

Both work on raw element bits and return new arrays.
"""
from __future__ import annotations

import numpy as np


def store_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
             v_new: np.ndarray, slots: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    num_pages, page_size = k_pool.shape[0], k_pool.shape[1]
    used = [int(s) for s in slots if s >= 0]
    if len(set(used)) != len(used):
        raise ValueError("two new rows for one slot")
    kp, vp = k_pool.copy(), v_pool.copy()
    for t, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        if slot >= num_pages * page_size:
            raise IndexError(f"slot {slot} outside the pool")
        page, off = divmod(slot, page_size)
        kp[page, off] = k_new[t]
        vp[page, off] = v_new[t]
    return kp, vp


def copy_pages(k_pool: np.ndarray, v_pool: np.ndarray, src: np.ndarray,
               dst: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    src = [int(x) for x in src]
    dst = [int(x) for x in dst]
    if len(src) != len(dst):
        raise ValueError("source and target lists differ in length")
    if len(set(dst)) != len(dst) or set(src) & set(dst):
        raise ValueError("copy targets must be distinct and disjoint from the sources")
    n = k_pool.shape[0]
    if any(not 0 <= p < n for p in src + dst):
        raise IndexError("page outside the pool")
    kp, vp = k_pool.copy(), v_pool.copy()
    for s, d in zip(src, dst):
        kp[d] = k_pool[s]
        vp[d] = v_pool[s]
    return kp, vp

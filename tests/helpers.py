"""Test glue: torch tensors to raw-bit NumPy arrays, and the oracle's view of a step."""
from __future__ import annotations

import numpy as np
import torch

import oracle


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a float32 or bfloat16 tensor as a NumPy array."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


def ints(t) -> np.ndarray:
    return np.asarray(t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else t, dtype=np.int64)


def table_view(pool_bits: np.ndarray, table_page_size: int) -> np.ndarray:
    """The pool seen in pages of ``table_page_size`` rows (a reshape, no copy)."""
    n, P = pool_bits.shape[:2]
    return pool_bits.reshape(n * P // table_page_size, table_page_size, *pool_bits.shape[2:])


def expected_step(sc, seqs=None, k_pool_bits=None, v_pool_bits=None):
    """Oracle result of one step of scenario ``sc``: copy, then store, then decode.

    Returns (k_pool_bits, v_pool_bits, out_f64).  Pre-step pools may be passed
    in (already on the host) to avoid a second device-to-host copy.
    """
    dt = sc.spec.dtype
    kp = bits(sc.k_pool) if k_pool_bits is None else k_pool_bits
    vp = bits(sc.v_pool) if v_pool_bits is None else v_pool_bits
    kp, vp = oracle.kvstore.copy_pages(kp, vp, ints(sc.copy_src), ints(sc.copy_dst))
    kp, vp = oracle.kvstore.store_kv(kp, vp, bits(sc.k_new), bits(sc.v_new), ints(sc.slot_mapping))
    if sc.q_start is not None:
        # several query tokens per sequence; `seqs` then selects query rows
        out = oracle.attention.prefill(
            bits(sc.q), table_view(kp, sc.table_page_size), table_view(vp, sc.table_page_size),
            ints(sc.block_tables), ints(sc.context_lens), ints(sc.q_start),
            sc.table_page_size, sc.spec.window, sc.scale, dt, rows=seqs)
        return kp, vp, out
    out = oracle.attention.decode(
        bits(sc.q), table_view(kp, sc.table_page_size), table_view(vp, sc.table_page_size),
        ints(sc.block_tables), ints(sc.context_lens), sc.table_page_size, sc.spec.window,
        sc.scale, dt, seqs=seqs, sinks=getattr(sc.spec, "sinks", 0))
    return kp, vp, out


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()

"""Test glue: torch tensors to raw-bit NumPy arrays, the oracle's view of a step, and the
random shapes of several query tokens per sequence."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads


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


def random_multi_spec(seed):
    # random shapes for several query tokens per sequence: every path (streaming groups of
    # 1 or 2 blocks, the tile kernel, the per-row kernels) and the boundaries between them
    r = np.random.default_rng(1000 + seed)
    kvh = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 2, 3, 4, 8, 16]))
    d = int(r.choice([128, 128, 128, 64]))
    B = int(r.choice([1, 3, 8, 24, 40]))
    q_hi = int(r.choice([2, 5, 17, 40, 90, 150]))
    dt = str(r.choice(["bf16", "bf16", "f32"]))
    if seed >= 24:
        # shapes the tile kernel takes (long chunks over many tiles)
        kvh, g, d, dt = int(r.choice([4, 8])), int(r.choice([2, 4, 8, 16])), 128, "bf16"
        B, q_hi = 64, int(r.integers(100, 220))
    len_hi = int(r.integers(q_hi, q_hi + 500))
    return workloads.Spec(name=f"rmulti{seed}", dtype=dt,
                          num_seqs=B, q_heads=kvh * g, kv_heads=kvh, head_dim=d,
                          page_size=int(r.choice([1, 4, 16, 32])),
                          window=int(r.choice([0, 0, 1, 9, 33, 300])), len_lo=1, len_hi=len_hi,
                          q_lo=1, q_hi=q_hi, spare=str(r.choice(["canary", "nan"])),
                          pool_factor=1.5)

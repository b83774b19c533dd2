"""Torch-facing binding of the C-ABI entry points.

Argument marshalling only: shape, dtype, device and contiguity checks, then
raw device pointers and the current HIP stream go to libpa.so.  Every step of
the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.PA_F32, torch.bfloat16: _lib.PA_BF16}


def _code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16") from None


def _dev(*ts: torch.Tensor) -> torch.device:
    d = ts[0].device
    if d.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    for t in ts:
        if t.device != d:
            raise ValueError("tensors are on different devices")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return d


def _i32(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")


def _stream(device: torch.device, stream: Optional[torch.cuda.Stream]) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


LAYOUTS = ("token", "head")


def _pool_dims(k_pool: torch.Tensor, v_pool: torch.Tensor, layout: str = "token"):
    """(num_pages, page_size, kv_heads, head_dim) of the pools.  ``layout="token"``:
    ``[num_pages, page_size, kv_heads, head_dim]``; ``"head"`` (head-major):
    ``[num_pages, kv_heads, page_size, head_dim]``."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {LAYOUTS}")
    if k_pool.dim() != 4 or k_pool.shape != v_pool.shape or k_pool.dtype != v_pool.dtype:
        raise ValueError("pools must both be 4-D, of one shape and dtype")
    n, a, b, d = (int(x) for x in k_pool.shape)
    return (n, a, b, d) if layout == "token" else (n, b, a, d)


def _fmt(t: torch.Tensor, layout: str) -> int:
    """The dtype argument of a call on pools of this layout."""
    return _code(t) | (_lib.PA_HEAD_MAJOR if layout == "head" else 0)


def store_kv(k_pool, v_pool, k_new, v_new, slot_mapping, stream=None,
             layout: str = "token") -> None:
    """Write row t of k_new/v_new to flat slot slot_mapping[t] of the pools (in place)."""
    dev = _dev(k_pool, v_pool, k_new, v_new, slot_mapping)
    n, P, hkv, d = _pool_dims(k_pool, v_pool, layout)
    T = int(slot_mapping.numel())
    if k_new.shape != (T, hkv, d) or v_new.shape != (T, hkv, d):
        raise ValueError("new rows must be [num_tokens, kv_heads, head_dim]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise TypeError("new rows must have the pool dtype")
    _i32(slot_mapping, "slot_mapping")
    lib = _lib.load()
    _lib.check("pa_store_kv", lib.pa_store_kv(
        k_pool.data_ptr(), v_pool.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
        slot_mapping.data_ptr(), T, n, P, hkv, d, _fmt(k_pool, layout), _stream(dev, stream)))


def copy_pages(k_pool, v_pool, src_pages, dst_pages, stream=None,
               layout: str = "token") -> None:
    """pool[dst[i]] = pool[src[i]] for K and V, whole pages (in place)."""
    dev = _dev(k_pool, v_pool, src_pages, dst_pages)
    n, P, hkv, d = _pool_dims(k_pool, v_pool, layout)
    if src_pages.numel() != dst_pages.numel():
        raise ValueError("source and target lists differ in length")
    _i32(src_pages, "src_pages")
    _i32(dst_pages, "dst_pages")
    lib = _lib.load()
    _lib.check("pa_copy_pages", lib.pa_copy_pages(
        k_pool.data_ptr(), v_pool.data_ptr(), src_pages.data_ptr(), dst_pages.data_ptr(),
        int(src_pages.numel()), n, P, hkv, d, _fmt(k_pool, layout), _stream(dev, stream)))


def reset_workspace(workspace: torch.Tensor, stream=None) -> None:
    """Zero the counter header of a decode/prefill workspace (``pa_reset_workspace``),
    in stream order: needed before reusing a workspace whose last call did not complete
    (a freshly zero-filled workspace needs nothing)."""
    dev = _dev(workspace)
    lib = _lib.load()
    _lib.check("pa_reset_workspace", lib.pa_reset_workspace(
        workspace.data_ptr() if workspace.numel() else None,
        workspace.numel() * workspace.element_size(), _stream(dev, stream)))


def _decode_call(out, q, k_pool, v_pool, block_tables, context_lens, window, sinks, scale,
                 max_context_len, ws_ptr, ws_size, stream_handle, hints=0, layout="token"):
    n, P, hkv, d = _pool_dims(k_pool, v_pool, layout)
    B, hq, dq = (int(x) for x in q.shape)
    lib = _lib.load()
    size = ctypes.c_size_t(ws_size)
    head = (out.data_ptr() if out is not None else None, q.data_ptr(), k_pool.data_ptr(),
            v_pool.data_ptr(), block_tables.data_ptr(), int(block_tables.shape[1]),
            context_lens.data_ptr(), B, hq, hkv, d, n, P, int(window))
    tail = (int(max_context_len), float(scale), _fmt(q, layout), ws_ptr, ctypes.byref(size),
            stream_handle)
    if hints:
        _lib.check("pa_decode_hinted",
                   lib.pa_decode_hinted(*head, int(sinks), int(hints), *tail))
    elif sinks:
        _lib.check("pa_decode_sinks", lib.pa_decode_sinks(*head, int(sinks), *tail))
    else:
        _lib.check("pa_decode", lib.pa_decode(*head, *tail))
    return size.value


def decode_workspace_bytes(q, k_pool, v_pool, block_tables, context_lens, *, window=0,
                           sinks=0, max_context_len=0, layout: str = "token") -> int:
    """Bytes of device workspace ``decode`` needs for these operands."""
    return _decode_call(None, q, k_pool, v_pool, block_tables, context_lens, window, sinks,
                        1.0, max_context_len, None, 0, None, layout=layout)


def decode(q, k_pool, v_pool, block_tables, context_lens, *, window: int = 0,
           sinks: int = 0, scale: Optional[float] = None, max_context_len: int = 0,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           stream=None, unshared_pages: bool = False, layout: str = "token") -> torch.Tensor:
    """Single-query paged attention; returns fp32 ``[num_seqs, q_heads, head_dim]``.

    ``layout="head"`` takes head-major pools ``[num_pages, kv_heads, page_size,
    head_dim]`` (``PA_HEAD_MAJOR``); the result is bit-identical to the same call on
    token-major pools holding the same rows.

    A raw token-slot table is passed as ``block_tables`` together with pools
    viewed in pages of one row (``pool.view(-1, 1, kv_heads, head_dim)``).
    ``sinks > 0`` (below ``window``) also attends the first ``sinks`` rows of
    every sequence, through ``pa_decode_sinks``; 0 calls ``pa_decode``.
    ``unshared_pages=True`` promises that no physical page is attended by two
    sequences of the batch and calls ``pa_decode_hinted``, which reads V rows with
    the non-temporal cache hint; the result is the same bit for bit.
    A ``workspace`` passed in must be zero-filled before its first use (or reset
    with ``reset_workspace``); each completed call leaves it ready for the next,
    whatever its shape.  Without one (or with one too small) a zeroed workspace is
    allocated for this call.
    """
    dev = _dev(q, k_pool, v_pool, block_tables, context_lens)
    n, P, hkv, d = _pool_dims(k_pool, v_pool, layout)
    if q.dim() != 3 or q.shape[2] != d or q.dtype != k_pool.dtype:
        raise ValueError("q must be [num_seqs, q_heads, head_dim] in the pool dtype")
    B = int(q.shape[0])
    if block_tables.dim() != 2 or block_tables.shape[0] < B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [>= num_seqs, stride], context_lens [num_seqs]")
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty(B, q.shape[1], d, dtype=torch.float32, device=dev)
    elif out.shape != (B, q.shape[1], d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [num_seqs, q_heads, head_dim]")
    need = _decode_call(None, q, k_pool, v_pool, block_tables, context_lens, window, sinks,
                        scale, max_context_len, None, 0, None, layout=layout)
    # (an empty tensor's pointer is NULL, which the library reads as a size query: even
    # when the call needs no workspace it gets a byte of its own)
    if workspace is None or workspace.numel() == 0 or \
            workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    _decode_call(out, q, k_pool, v_pool, block_tables, context_lens, window, sinks, scale,
                 max_context_len, workspace.data_ptr(),
                 workspace.numel() * workspace.element_size(), _stream(dev, stream),
                 _lib.PA_HINT_UNSHARED if unshared_pages else 0, layout=layout)
    return out


def decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, *, out: torch.Tensor,
                   window: int = 0, sinks: int = 0, scale: Optional[float] = None,
                   max_context_len: int = 0, stream=None, unshared_pages: bool = False,
                   layout: str = "token") -> torch.Tensor:
    """``decode`` through ``pa_decode_noalloc``: no workspace, nothing allocated (the
    caller passes ``out``).  The library's one scratch buffer per GPU serves every such
    call, so calls that overlap on one GPU race."""
    dev = _dev(q, k_pool, v_pool, block_tables, context_lens, out)
    n, P, hkv, d = _pool_dims(k_pool, v_pool, layout)
    B, hq = int(q.shape[0]), int(q.shape[1])
    if q.dim() != 3 or q.shape[2] != d or q.dtype != k_pool.dtype:
        raise ValueError("q must be [num_seqs, q_heads, head_dim] in the pool dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] < B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [>= num_seqs, stride], context_lens [num_seqs]")
    if out.shape != (B, hq, d) or out.dtype != torch.float32:
        raise ValueError("out must be a contiguous fp32 [num_seqs, q_heads, head_dim]")
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    if scale is None:
        scale = d ** -0.5
    lib = _lib.load()
    _lib.check("pa_decode_noalloc", lib.pa_decode_noalloc(
        out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
        block_tables.data_ptr(), int(block_tables.shape[1]), context_lens.data_ptr(), B, hq, hkv,
        d, n, P, int(window), int(sinks), _lib.PA_HINT_UNSHARED if unshared_pages else 0,
        int(max_context_len), float(scale), _fmt(q, layout), _stream(dev, stream)))
    return out


def _prefill_call(out, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len,
                  window, scale, max_context_len, ws_ptr, ws_size, stream_handle,
                  layout="token", hints=0):
    n, P, hkv, d = _pool_dims(k_pool, v_pool, layout)
    num_q, hq, _ = (int(x) for x in q.shape)
    B = int(context_lens.shape[0])
    lib = _lib.load()
    size = ctypes.c_size_t(ws_size)
    head = (out.data_ptr() if out is not None else None, q.data_ptr(), q_start.data_ptr(),
            k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(),
            int(block_tables.shape[1]), context_lens.data_ptr(), B, num_q, int(max_q_len), hq,
            hkv, d, n, P, int(window))
    tail = (int(max_context_len), float(scale), _fmt(q, layout), ws_ptr, ctypes.byref(size),
            stream_handle)
    if hints:
        _lib.check("pa_prefill_hinted", lib.pa_prefill_hinted(*head, int(hints), *tail))
    else:
        _lib.check("pa_prefill", lib.pa_prefill(*head, *tail))
    return size.value


def prefill_workspace_bytes(q, q_start, k_pool, v_pool, block_tables, context_lens, *,
                            max_q_len: int, window: int = 0, scale: Optional[float] = None,
                            max_context_len: int = 0, layout: str = "token") -> int:
    """Bytes of device workspace ``prefill`` needs for these operands (and scale: the
    kernel that serves long chunks needs none, and takes positive scales only)."""
    if scale is None:
        scale = int(q.shape[-1]) ** -0.5
    return _prefill_call(None, q, q_start, k_pool, v_pool, block_tables, context_lens,
                         max_q_len, window, scale, max_context_len, None, 0, None,
                         layout=layout)


def prefill(q, q_start, k_pool, v_pool, block_tables, context_lens, *, max_q_len: int,
            window: int = 0, scale: Optional[float] = None, max_context_len: int = 0,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            stream=None, layout: str = "token", unshared_pages: bool = False) -> torch.Tensor:
    """Several query tokens per sequence (``pa_prefill``); returns fp32 ``[num_q, q_heads, head_dim]``.

    ``q`` is ``[num_q, q_heads, head_dim]``; the query rows of sequence ``s`` are
    ``q_start[s] .. q_start[s+1]-1`` (int32 ``[num_seqs + 1]``, at most
    ``max_q_len`` per sequence) and are its last rows.  Workspace rules,
    ``layout`` and ``unshared_pages`` (``pa_prefill_hinted``: same result bit for bit)
    as for ``decode``.
    """
    dev = _dev(q, q_start, k_pool, v_pool, block_tables, context_lens)
    n, P, hkv, d = _pool_dims(k_pool, v_pool, layout)
    if q.dim() != 3 or q.shape[2] != d or q.dtype != k_pool.dtype:
        raise ValueError("q must be [num_q, q_heads, head_dim] in the pool dtype")
    B = int(context_lens.shape[0])
    if context_lens.dim() != 1 or q_start.shape != (B + 1,):
        raise ValueError("context_lens must be [num_seqs] and q_start [num_seqs + 1]")
    if block_tables.dim() != 2 or block_tables.shape[0] < B:
        raise ValueError("block_tables must be [>= num_seqs, stride]")
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    _i32(q_start, "q_start")
    if scale is None:
        scale = d ** -0.5
    num_q = int(q.shape[0])
    if out is None:
        out = torch.empty(num_q, q.shape[1], d, dtype=torch.float32, device=dev)
    elif out.shape != (num_q, q.shape[1], d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [num_q, q_heads, head_dim]")
    need = _prefill_call(None, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len,
                         window, scale, max_context_len, None, 0, None, layout=layout)
    # (an empty tensor's pointer is NULL, which the library reads as a size query: even
    # when the call needs no workspace it gets a byte of its own)
    if workspace is None or workspace.numel() == 0 or \
            workspace.numel() * workspace.element_size() < need:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    _prefill_call(out, q, q_start, k_pool, v_pool, block_tables, context_lens, max_q_len, window,
                  scale, max_context_len, workspace.data_ptr(),
                  workspace.numel() * workspace.element_size(), _stream(dev, stream),
                  layout=layout, hints=_lib.PA_HINT_UNSHARED if unshared_pages else 0)
    return out


def update_tables(rows, logical_pages, pages, *, page_size: int,
                  block_tables: Optional[torch.Tensor] = None,
                  slot_table: Optional[torch.Tensor] = None, dummy_slot: int = 0,
                  stream=None) -> None:
    """Scatter one step's table changes (``pa_update_tables``) into the tables, in place.

    ``rows``, ``logical_pages``, ``pages``: int32 ``[n]`` on the device (for instance
    ``PagedKVCache.take_table_updates`` moved there); ``pages[i] < 0`` releases the cell.
    """
    tabs = [t for t in (block_tables, slot_table) if t is not None]
    dev = _dev(rows, logical_pages, pages, *tabs)
    for name, t in (("rows", rows), ("logical_pages", logical_pages), ("pages", pages)):
        _i32(t, name)
    n = int(rows.numel())
    if logical_pages.numel() != n or pages.numel() != n:
        raise ValueError("index lists differ in length")
    for name, t in (("block_tables", block_tables), ("slot_table", slot_table)):
        if t is not None:
            _i32(t, name)
            if t.dim() != 2:
                raise ValueError(f"{name} must be 2-D")
    bt = block_tables
    st = slot_table
    lib = _lib.load()
    _lib.check("pa_update_tables", lib.pa_update_tables(
        bt.data_ptr() if bt is not None else None, int(bt.shape[1]) if bt is not None else 0,
        int(bt.shape[0]) if bt is not None else 0,
        st.data_ptr() if st is not None else None, int(st.shape[1]) if st is not None else 0,
        int(st.shape[0]) if st is not None else 0, int(dummy_slot), rows.data_ptr(),
        logical_pages.data_ptr(), pages.data_ptr(), n, int(page_size), _stream(dev, stream)))

"""Scenario builder: seeded, synthetic decode steps over a paged K/V pool.

A scenario is the state of a batch just before one decode step, plus the
operands of that step:

* a physical pool ``[pool_pages, page_size, kv_heads, head_dim]`` per K and V
  (the buffer layout of the mini-sglang page, section on the KV buffer,
  with the layer axis taken out);
* per-sequence block tables (int32, ``-1`` where no page is mapped), or, in
  raw-slot mode, a token-slot table with one extra dummy row and one extra
  dummy page (the mini-sglang page, sections on the page table and on the
  dummy request);
* context lengths ``L`` that count the token being decoded, the query, the
  one new K/V row per sequence and the slot it goes to, and, for the
  shared-prefix case, the list of pages to copy before the write.

Placement: the pages a scenario needs are taken from a seeded permutation of
``range(pool_pages)`` in (shared prefix, then sequence by sequence, then the
copy targets) order.  Rows that are mapped but hold no data (the slots of the
new row before the write, slots past ``L`` in the last page, rows of the first
live page that lie before the window) hold large finite canaries, or NaN with
``spare="nan"``; pages that no table maps hold NaN.  A kernel that attends a
masked row therefore gives a gross error (canaries) or NaN, and one that reads
an unmapped page gives NaN.

Random values are float32 N(0, 1) drawn with a seeded ``torch.Generator`` on
the requested device and rounded to the pool dtype (round to nearest even);
integers (lengths, permutations) come from a seeded NumPy PCG64 generator.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np
import torch

K_CANARY = 64.0      # exact in bf16 and fp32
V_CANARY = 8192.0    # exact in bf16 and fp32

CONFIG_NAMES = ("tiny_f32", "gqa_b64", "window_b32", "prefix_b256", "slot_b256")


@dataclass(frozen=True)
class Spec:
    name: str
    dtype: str = "bf16"            # "f32" or "bf16"
    num_seqs: int = 4
    q_heads: int = 2
    kv_heads: int = 2
    head_dim: int = 16
    page_size: int = 16
    window: int = 0                # 0: attend the whole context
    sinks: int = 0                 # rows at the start kept besides the window (0 <= sinks < window)
    q_lo: int = 1                  # query tokens per sequence, uniform in [q_lo, q_hi] and at
    q_hi: int = 1                  # most L: a prefill chunk or a verify step when above 1
    lens: Optional[tuple] = None   # explicit context lengths (include the new token)
    len_dist: str = "uniform"      # "uniform" | "lognormal" (when lens is None)
    len_lo: int = 1                # uniform: low bound; lognormal: median
    len_hi: int = 64               # uniform: high bound; lognormal: cap
    sigma: float = 1.0
    pool_pages: int = 0            # fixed pool size; 0: ceil(pool_factor * needed)
    pool_factor: float = 1.25
    bt_stride: int = 0             # block-table width; 0: pages of the longest context
    prefix_len: int = 0            # rows of a prefix shared by every sequence
    suffix_lo: int = 0             # private rows after the prefix, uniform [lo, hi]
    suffix_hi: int = 0
    sibling_cow: bool = False      # tail page also held by a sibling: copy before the write
    slot_table: bool = False       # raw token-slot table, page-size-1 addressing
    slot_stride: int = 0           # width of the slot table; 0: align32(longest context)
    scale: float = 0.0             # 0: fp32(1/sqrt(head_dim))
    spare: str = "canary"          # rows of mapped pages that hold no data: "canary" or "nan"


def _align32(x: int) -> int:
    return (x + 31) // 32 * 32


def config_spec(index: int) -> Spec:
    """The five named workloads, indexed 1..5."""
    if index == 1:
        return Spec(name="tiny_f32", dtype="f32", num_seqs=4, q_heads=2, kv_heads=2,
                    head_dim=16, page_size=4, lens=(5, 17, 32, 40), pool_pages=64,
                    bt_stride=10)
    if index == 2:
        return Spec(name="gqa_b64", dtype="bf16", num_seqs=64, q_heads=32, kv_heads=8,
                    head_dim=128, page_size=16, len_dist="uniform", len_lo=1, len_hi=4096,
                    pool_factor=1.25, bt_stride=4096 // 16)
    if index == 3:
        return Spec(name="window_b32", dtype="bf16", num_seqs=32, q_heads=32, kv_heads=8,
                    head_dim=128, page_size=16, window=1024, len_dist="uniform",
                    len_lo=2048, len_hi=32768, pool_factor=1.25, bt_stride=32768 // 16)
    if index == 4:
        return Spec(name="prefix_b256", dtype="bf16", num_seqs=256, q_heads=64, kv_heads=8,
                    head_dim=128, page_size=16, prefix_len=2048, suffix_lo=0, suffix_hi=512,
                    sibling_cow=True, pool_factor=1.25, bt_stride=-(-(2048 + 512 + 1) // 16))
    if index == 5:
        return Spec(name="slot_b256", dtype="bf16", num_seqs=256, q_heads=64, kv_heads=8,
                    head_dim=128, page_size=16, len_dist="lognormal", len_lo=2048,
                    len_hi=32768, sigma=1.0, pool_factor=1.25, slot_table=True,
                    slot_stride=_align32(32768))
    raise ValueError(f"no config {index}")


def random_spec(seed: int, **over) -> Spec:
    """A small random shape for parity sweeps (page sizes, windows, GQA ratios)."""
    r = np.random.default_rng(seed)
    kvh = int(r.choice([1, 2, 4]))
    g = int(r.choice([1, 2, 4, 8]))
    base = dict(name=f"rand{seed}", dtype=str(r.choice(["f32", "bf16"])),
                num_seqs=int(r.integers(1, 7)), q_heads=kvh * g, kv_heads=kvh,
                head_dim=int(r.choice([16, 32, 64, 128])),
                page_size=int(r.choice([1, 2, 4, 16])),
                window=int(r.choice([0, 0, 1, 2, 3, 5, 16, 17])),
                len_dist="uniform", len_lo=int(r.integers(0, 3)), len_hi=int(r.integers(3, 90)),
                pool_factor=1.5)
    base.update(over)
    return Spec(**base)


@dataclass
class Scenario:
    spec: Spec
    seed: int
    device: str
    lens: np.ndarray                 # int64 [B], context length incl. the new token
    lo: np.ndarray                   # int64 [B], L less the rows attended (with no sinks: the first attended row)
    pool_pages: int                  # physical pages, incl. the dummy page in slot mode
    k_pool: torch.Tensor             # [pool_pages, page_size, kv_heads, head_dim]
    v_pool: torch.Tensor
    block_tables: torch.Tensor       # int32 [rows, stride]; slot mode: token slots
    table_page_size: int             # page size the table is written in (1 in slot mode)
    context_lens: torch.Tensor       # int32 [B]
    q: torch.Tensor                  # [B, q_heads, head_dim]
    k_new: torch.Tensor              # [B, kv_heads, head_dim]
    v_new: torch.Tensor
    slot_mapping: torch.Tensor       # int32 [B]; -1 for an empty sequence
    copy_src: torch.Tensor           # int32 [C]
    copy_dst: torch.Tensor
    scale: float
    max_context_len: int
    # the unpaged attended rows of every sequence in row order (last one = the new row), CPU,
    # if kept
    k_src: Optional[List[torch.Tensor]] = None
    v_src: Optional[List[torch.Tensor]] = None
    shared_pages: int = 0            # pages of the shared prefix (mapped by every sequence)
    # several query tokens per sequence: q, k_new, v_new and slot_mapping have one row per
    # query token; those of sequence s are rows q_start[s] .. q_start[s+1]-1 (int32 [B+1])
    q_start: Optional[torch.Tensor] = None
    nq: Optional[np.ndarray] = None  # int64 [B], query tokens per sequence

    @property
    def table_num_pages(self) -> int:
        """Pool size in units of ``table_page_size`` rows."""
        return self.pool_pages * self.spec.page_size // self.table_page_size

    @property
    def torch_dtype(self):
        return torch.float32 if self.spec.dtype == "f32" else torch.bfloat16


def _draw_lens(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    if spec.lens is not None:
        lens = np.asarray(spec.lens, dtype=np.int64)
        assert len(lens) == spec.num_seqs
        return lens
    if spec.prefix_len:
        s = rng.integers(spec.suffix_lo, spec.suffix_hi + 1, size=spec.num_seqs)
        return spec.prefix_len + s + 1
    if spec.len_dist == "uniform":
        return rng.integers(spec.len_lo, spec.len_hi + 1, size=spec.num_seqs).astype(np.int64)
    if spec.len_dist == "lognormal":
        z = rng.normal(math.log(spec.len_lo), spec.sigma, size=spec.num_seqs)
        return np.clip(np.exp(z).astype(np.int64), 1, spec.len_hi)
    raise ValueError(spec.len_dist)


def spare_is_canary(spec: Spec) -> bool:
    if spec.spare not in ("canary", "nan"):
        raise ValueError(spec.spare)
    return spec.spare == "canary"


def build(spec: Spec, seed: int, device: str = "cpu", keep_source: bool = False) -> Scenario:
    """Build the scenario of ``spec`` with ``seed`` on ``device``."""
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    B, Hkv, D, P, W = spec.num_seqs, spec.kv_heads, spec.head_dim, spec.page_size, spec.window
    assert spec.q_heads % Hkv == 0
    lens = _draw_lens(spec, rng)
    assert (lens >= 0).all()
    multi = spec.q_hi > 1
    nq = np.minimum(lens, 1)
    if multi:
        # several query tokens per sequence: its last nq rows are new, stored by the step
        assert not spec.prefix_len and not spec.sinks and 1 <= spec.q_lo <= spec.q_hi
        nq = np.minimum(rng.integers(spec.q_lo, spec.q_hi + 1, size=B), lens)
    if spec.prefix_len:
        assert W == 0 and spec.prefix_len % P == 0 and (lens > spec.prefix_len).all()
    # first row attended by the first query (row L - nq)
    lo = np.maximum(lens - nq + 1 - W, 0) if W > 0 else np.zeros_like(lens)
    S = spec.sinks
    if S:
        assert 0 < S < W and not spec.prefix_len and not spec.sibling_cow

    def attended(L):
        # the first S rows and the last W - S once the window cuts, else [lo, L)
        if S and L > W:
            return list(range(S)) + list(range(L - W + S, L))
        return list(range(max(L - W, 0) if W > 0 else 0, L))

    # logical pages that must be mapped: those holding a row in [lo, L)
    first = lo // P
    last = np.where(lens > 0, (lens - 1) // P, first - 1)
    n_shared = spec.prefix_len // P
    cow = np.zeros(B, dtype=bool)
    if spec.sibling_cow:
        # the tail page holding rows before the new one is also held by a sibling;
        # the new row lands inside it exactly when (L-1) is not a page start
        cow = ((lens - 1) % P != 0) & ((lens - 1) // P >= n_shared)
    private = np.maximum(last - np.maximum(first, n_shared) + 1, 0)
    page_sets = None
    if S:
        # with sinks the mapped pages are those of the attended rows (a hole between)
        page_sets = [sorted({r // P for r in attended(int(L))}) for L in lens]
        private = np.array([len(ps) for ps in page_sets], dtype=np.int64)
        lo = np.array([int(L) - len(attended(int(L))) for L in lens], dtype=lens.dtype)
    needed = n_shared + int(private.sum()) + int(cow.sum())
    pool_pages = spec.pool_pages or int(math.ceil(spec.pool_factor * max(needed, 1)))
    assert pool_pages >= needed, "pool too small for the scenario"
    perm = rng.permutation(pool_pages)
    take = iter(perm.tolist())

    shared = [next(take) for _ in range(n_shared)]
    seq_pages = []                     # per seq: dict logical page -> physical (pre-step)
    for s in range(B):
        if page_sets is not None:
            seq_pages.append({j: next(take) for j in page_sets[s]})
            continue
        m = {j: shared[j] for j in range(first[s], min(last[s] + 1, n_shared))}
        for j in range(max(first[s], n_shared), last[s] + 1):
            m[j] = next(take)
        seq_pages.append(m)
    copies = []                        # (src, dst) per copy-on-write sequence
    post_pages = [dict(m) for m in seq_pages]
    for s in range(B):
        if cow[s]:
            j = int((lens[s] - 1) // P)
            dst = next(take)
            copies.append((seq_pages[s][j], dst))
            post_pages[s][j] = dst

    total_pages = pool_pages + (1 if spec.slot_table else 0)
    dummy_page = pool_pages            # slot mode: a real page no table entry ever names
    nan = float("nan")
    k_pool = torch.full((total_pages, P, Hkv, D), nan, dtype=tdt, device=device)
    v_pool = torch.full((total_pages, P, Hkv, D), nan, dtype=tdt, device=device)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32).to(tdt)

    # every mapped page first gets canaries (or stays NaN), then the rows that hold data
    mapped = sorted({p for m in seq_pages for p in m.values()})
    if mapped and spare_is_canary(spec):
        idx = torch.tensor(mapped, device=device, dtype=torch.long)
        k_pool[idx] = K_CANARY
        v_pool[idx] = V_CANARY
    if spec.slot_table:
        k_pool[dummy_page] = K_CANARY
        v_pool[dummy_page] = V_CANARY

    prefix_k = randn(spec.prefix_len, Hkv, D) if spec.prefix_len else None
    prefix_v = randn(spec.prefix_len, Hkv, D) if spec.prefix_len else None
    if spec.prefix_len:
        r = torch.arange(spec.prefix_len, device=device)
        pg = torch.tensor(shared, device=device, dtype=torch.long)[r // P]
        k_pool[pg, r % P] = prefix_k
        v_pool[pg, r % P] = prefix_v

    k_src, v_src = ([], []) if keep_source else (None, None)
    if multi:
        num_q = int(nq.sum())
        q_start = np.concatenate([[0], np.cumsum(nq)]).astype(np.int64)
        k_new = torch.zeros(num_q, Hkv, D, dtype=tdt, device=device)
        v_new = torch.zeros(num_q, Hkv, D, dtype=tdt, device=device)
        slots = np.full(num_q, -1, dtype=np.int64)
        for s in range(B):
            L, l0, n = int(lens[s]), int(lo[s]), int(nq[s])
            kr = randn(L - l0, Hkv, D)
            vr = randn(L - l0, Hkv, D)
            if L - n > l0:                        # rows before the chunk go into the pool
                r = torch.arange(l0, L - n)
                pg = torch.tensor([seq_pages[s][int(j)] for j in (r // P).tolist()],
                                  device=device, dtype=torch.long)
                off = (r % P).to(device)
                k_pool[pg, off] = kr[:L - n - l0]
                v_pool[pg, off] = vr[:L - n - l0]
            q0 = int(q_start[s])
            k_new[q0:q0 + n] = kr[L - n - l0:]
            v_new[q0:q0 + n] = vr[L - n - l0:]
            for i in range(n):
                t = L - n + i
                slots[q0 + i] = post_pages[s][t // P] * P + t % P
            if keep_source:
                k_src.append(kr.cpu())
                v_src.append(vr.cpu())
        q = randn(num_q, spec.q_heads, D)
    else:
        k_new = torch.zeros(B, Hkv, D, dtype=tdt, device=device)
        v_new = torch.zeros(B, Hkv, D, dtype=tdt, device=device)
        slots = np.full(B, -1, dtype=np.int64)
    for s in range(B if not multi else 0):
        L, l0 = int(lens[s]), int(lo[s])
        if L == 0:
            if keep_source:
                k_src.append(torch.zeros(0, Hkv, D, dtype=tdt))
                v_src.append(torch.zeros(0, Hkv, D, dtype=tdt))
            continue
        if S:
            # data only in the attended rows (sinks, then the window); the new row last
            rows = attended(L)
            kr = randn(len(rows), Hkv, D)
            vr = randn(len(rows), Hkv, D)
            if len(rows) > 1:
                r = torch.tensor(rows[:-1])
                pg = torch.tensor([seq_pages[s][int(j)] for j in (r // P).tolist()],
                                  device=device, dtype=torch.long)
                off = (r % P).to(device)
                k_pool[pg, off] = kr[:-1]
                v_pool[pg, off] = vr[:-1]
            k_new[s] = kr[-1]
            v_new[s] = vr[-1]
            slots[s] = post_pages[s][(L - 1) // P] * P + (L - 1) % P
            if keep_source:
                k_src.append(kr.cpu())
                v_src.append(vr.cpu())
            continue
        own0 = max(l0, spec.prefix_len)          # first private row that carries data
        kr = randn(L - own0, Hkv, D)
        vr = randn(L - own0, Hkv, D)
        if L - 1 > own0:                          # rows before the new one go into the pool
            r = torch.arange(own0, L - 1)
            pg = torch.tensor([seq_pages[s][int(j)] for j in (r // P).tolist()],
                              device=device, dtype=torch.long)
            off = (r % P).to(device)
            k_pool[pg, off] = kr[:-1]
            v_pool[pg, off] = vr[:-1]
        k_new[s] = kr[-1]
        v_new[s] = vr[-1]
        slots[s] = post_pages[s][(L - 1) // P] * P + (L - 1) % P
        if keep_source:
            if spec.prefix_len:
                k_src.append(torch.cat([prefix_k[l0:], kr]).cpu())
                v_src.append(torch.cat([prefix_v[l0:], vr]).cpu())
            else:
                k_src.append(kr.cpu())
                v_src.append(vr.cpu())
    if not multi:
        q = randn(B, spec.q_heads, D)

    if spec.slot_table:
        stride = spec.slot_stride or _align32(int(lens.max()))
        dummy_slot = dummy_page * P
        table = np.full((B + 1, stride), dummy_slot, dtype=np.int64)
        for s in range(B):
            for j, ph in post_pages[s].items():
                r0, r1 = j * P, min((j + 1) * P, int(lens[s]))
                table[s, r0:r1] = ph * P + np.arange(r1 - r0)
        table_page_size = 1
    else:
        stride = spec.bt_stride or max(int(last.max()) + 1, 1)
        table = np.full((B, stride), -1, dtype=np.int64)
        for s in range(B):
            for j, ph in post_pages[s].items():
                table[s, j] = ph
        table_page_size = P
    assert (table[:B, :] < 2**31).all()

    scale = spec.scale or float(np.float32(1.0 / math.sqrt(D)))
    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32), device=device)
    return Scenario(
        spec=spec, seed=seed, device=device, lens=lens, lo=lo, pool_pages=total_pages,
        k_pool=k_pool, v_pool=v_pool, block_tables=i32(table), table_page_size=table_page_size,
        context_lens=i32(lens), q=q, k_new=k_new, v_new=v_new, slot_mapping=i32(slots),
        copy_src=i32([c[0] for c in copies]), copy_dst=i32([c[1] for c in copies]),
        scale=scale, max_context_len=int(lens.max()) if B else 0,
        k_src=k_src, v_src=v_src, shared_pages=n_shared,
        q_start=i32(q_start) if multi else None, nq=nq)


def make_config(index: int, seed: Optional[int] = None, device: str = "cpu",
                keep_source: bool = False, **over) -> Scenario:
    """Scenario of the named workload ``index`` (1..5); default seed 41000 + index."""
    spec = config_spec(index)
    if over:
        spec = replace(spec, **over)
    return build(spec, 41000 + index if seed is None else seed, device, keep_source)

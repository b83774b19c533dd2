"""HIP path against the CPU oracle, through the C ABI, on the same seeded inputs.

Scatter and copy must match bit for bit over the whole pool (NaN poison
included); attention within max abs error 2e-3 (bf16 inputs) or 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import bits, expected_step, ints, random_multi_spec

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_41_amd import _lib
    _lib.load()


def ops():
    from paged_kv_cache_41_amd import ops as _ops
    return _ops


def decode_views(sc):
    if sc.table_page_size == sc.spec.page_size:
        return sc.k_pool, sc.v_pool
    hkv, d = sc.spec.kv_heads, sc.spec.head_dim
    return sc.k_pool.view(-1, 1, hkv, d), sc.v_pool.view(-1, 1, hkv, d)


def gpu_step(sc):
    """copy -> store -> decode on the device; returns the pre-step pools (host bits) and out."""
    kp0, vp0 = bits(sc.k_pool), bits(sc.v_pool)
    o = ops()
    o.copy_pages(sc.k_pool, sc.v_pool, sc.copy_src, sc.copy_dst)
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    kv, vv = decode_views(sc)
    if sc.q_start is not None:
        out = o.prefill(sc.q, sc.q_start, kv, vv, sc.block_tables, sc.context_lens,
                        max_q_len=max(int(sc.nq.max()), 1), window=sc.spec.window,
                        scale=sc.scale, max_context_len=sc.max_context_len)
    else:
        out = o.decode(sc.q, kv, vv, sc.block_tables, sc.context_lens, window=sc.spec.window,
                       sinks=sc.spec.sinks, scale=sc.scale, max_context_len=sc.max_context_len)
    torch.cuda.synchronize()
    return kp0, vp0, out


def check_step(sc, seqs=None):
    print(f"case {sc.spec.name} seed {sc.seed}", flush=True)
    kp0, vp0, out = gpu_step(sc)
    kp, vp, ref = expected_step(sc, seqs=seqs, k_pool_bits=kp0, v_pool_bits=vp0)
    assert np.array_equal(bits(sc.k_pool), kp), "K pool differs from the oracle after copy+store"
    assert np.array_equal(bits(sc.v_pool), vp), "V pool differs from the oracle after copy+store"
    got = out.cpu().double().numpy()
    if seqs is not None:
        got_s = got[list(seqs)]
    else:
        got_s = got
    err = float(np.max(np.abs(got_s - ref))) if ref.size else 0.0
    assert np.isfinite(got).all(), "non-finite output"
    assert err <= TOL[sc.spec.dtype], f"{sc.spec.name}: max abs error {err:.3g}"
    return out, err


@pytest.mark.parametrize("index", [1, 2, 3])
def test_config_full(index):
    sc = workloads.make_config(index, device="cuda")
    check_step(sc)


@pytest.mark.parametrize("q_len", [4, 128, 512])
def test_config_prefill_chunks_sampled(q_len):
    # the workloads `bench.py --q-len N` times, at full size, in the same launch: the
    # 4-token verify streams, the 128- and 512-token chunks take the tile kernel with its
    # longest-first order; sampled query rows, the first and last of the call included
    base = workloads.config_spec(2)
    sc = workloads.make_config(2, device="cuda", q_lo=q_len, q_hi=q_len,
                               name=f"{base.name}_q{q_len}")
    assert int(sc.nq.max()) == q_len
    rng = np.random.default_rng(q_len)
    rows = sorted(set(rng.choice(len(sc.q), 64, replace=False).tolist()) | {0, len(sc.q) - 1})
    check_step(sc, seqs=rows)


def test_config_window_sinks_full():
    # `bench.py --config 3 --sinks 4`: every sequence, every row
    base = workloads.config_spec(3)
    sc = workloads.make_config(3, device="cuda", sinks=4, name=f"{base.name}_sinks4")
    check_step(sc)


@pytest.mark.parametrize("cfg,sinks", [(2, 0), (3, 0), (3, 4), (5, 0), ("page4", 0)])
def test_unshared_hint_is_bit_identical(cfg, sinks):
    """pa_decode_hinted with PA_HINT_UNSHARED changes only the cache policy of the V
    loads: its output equals the plain call's bit for bit (which the config tests pin to
    the oracle), on the batch-64 and window workloads, with and without sinks, on the raw
    slot table (pages of one row) and on pages of 4 rows."""
    o = ops()
    if cfg == "page4":
        sc = workloads.build(workloads.Spec(name="hint_p4", num_seqs=32, q_heads=32,
                                            kv_heads=8, head_dim=128, page_size=4, len_lo=1,
                                            len_hi=900, spare="nan"), 71, device="cuda")
    else:
        sc = workloads.make_config(cfg, device="cuda", sinks=sinks,
                                   name=f"{workloads.config_spec(cfg).name}_s{sinks}")
    s = sc.spec
    print(f"case {s.name} seed {sc.seed}", flush=True)
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    kv, vv = decode_views(sc)
    outs = []
    for hint in (False, True, True):
        outs.append(o.decode(sc.q, kv, vv, sc.block_tables, sc.context_lens,
                               window=s.window, sinks=s.sinks, scale=sc.scale,
                               max_context_len=sc.max_context_len, unshared_pages=hint))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("cfg,q_len", [(2, 4), (3, 4), (5, 4), (2, 128)])
def test_prefill_hint_is_bit_identical(cfg, q_len):
    """pa_prefill_hinted with PA_HINT_UNSHARED gives pa_prefill's output bit for bit: the
    streaming path with one block per group (batch-64), the aligned window split, groups
    of two blocks over a raw slot table, and the tile kernel for long chunks (which
    ignores the hint)."""
    o = ops()
    base = workloads.config_spec(cfg)
    sc = workloads.make_config(cfg, device="cuda", q_lo=q_len, q_hi=q_len,
                               name=f"{base.name}_q{q_len}")
    s = sc.spec
    print(f"case {s.name} seed {sc.seed}", flush=True)
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    kv, vv = decode_views(sc)
    outs = []
    for hint in (False, True, True):
        outs.append(o.prefill(sc.q, sc.q_start, kv, vv, sc.block_tables, sc.context_lens,
                              max_q_len=q_len, window=s.window, scale=sc.scale,
                              max_context_len=sc.max_context_len, unshared_pages=hint))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_config_prefix_full():
    # every sequence of the prefix-shared workload: 243 copy-on-write copies, the store,
    # then decode over the 128 shared prefix pages and each private suffix
    sc = workloads.make_config(4, device="cuda")
    assert len(sc.copy_src) > 200
    check_step(sc)


def test_config_slot_table_full():
    # every sequence of the raw slot-table workload (page-size-1 addressing, lognormal
    # lengths up to 32768)
    sc = workloads.make_config(5, device="cuda")
    check_step(sc)


# (sequences, kv heads, window, sinks, context lengths low and high, empty sequences[,
# query tokens low and high])
ALIGNED_CASES = {
    # every segment 64 or 65 tiles, one per workgroup
    "one_segment_per_workgroup": (64, 4, 1024, 0, 1024, 3000, 0),
    # a few empty sequences: some workgroups get no tiles and only join the barrier
    "empty_workgroups": (64, 4, 1024, 0, 1024, 3000, 3),
    # 2048 segments of 16 or 17 tiles, eight per workgroup
    "eight_segments_per_workgroup": (256, 8, 256, 0, 300, 900, 0),
    # segments of 2 or 3 tiles: wavefronts with no tile between the pieces of a segment
    "short_segments": (64, 4, 32, 0, 40, 200, 0),
    # sink rows: a tile of their own ahead of every window
    "sinks": (64, 4, 1024, 4, 1100, 3000, 0),
    # contexts mostly inside the window: segments too uneven, the flat split is kept
    "uneven_keeps_flat_split": (64, 4, 1024, 0, 16, 2000, 0),
    # verify steps (one block of 16 / G = 4 query tokens per sequence): the same split for
    # segments of query blocks
    "verify_q4": (64, 4, 1024, 0, 1100, 3000, 0, 4, 4),
    "verify_q1_to_4": (64, 8, 512, 0, 600, 2000, 0, 1, 4),
    "verify_uneven_keeps_flat_split": (64, 4, 1024, 0, 16, 2000, 0, 4, 4),
}


@pytest.mark.parametrize("case", sorted(ALIGNED_CASES))
def test_window_segments_aligned_to_workgroups(case):
    """With a window, the host sizes the grid so that each workgroup can take whole
    segments (a sequence's kv head, or with several query tokens a block of them); when
    they are about equal the kernel does so and combines the pieces of a cut segment in
    LDS, else it keeps the equal flat split.  Either way the result is the oracle's."""
    B, hkv, window, sinks, lo, hi, empty, *q = ALIGNED_CASES[case]
    q_lo, q_hi = q if q else (1, 1)
    lens = np.random.default_rng(40 + B + window + sinks + lo).integers(lo, hi, size=B)
    lens[:empty] = 0
    spec = workloads.Spec(name=f"window_aligned_{case}", dtype="bf16", num_seqs=B,
                          q_heads=4 * hkv, kv_heads=hkv, head_dim=128, page_size=16,
                          window=window, sinks=sinks, lens=tuple(int(x) for x in lens),
                          q_lo=q_lo, q_hi=q_hi, pool_factor=1.25, spare="nan")
    sc = workloads.build(spec, 44 + empty, device="cuda")
    # the flat split leaves partials of cut segments past the counter header; the aligned
    # one keeps them in LDS and writes nothing there
    ws = torch.zeros(_need(sc), dtype=torch.uint8, device="cuda")
    ws[4096:] = 0x5A
    _run_on_workspace(sc, ws)
    untouched = bool((ws[4096:] == 0x5A).all())
    assert untouched == ("keeps_flat_split" not in case), case


@pytest.mark.parametrize("window", [0, 40])
def test_batch_above_streaming_limit(window):
    # more sequences than the streaming path takes: the chunked matrix-core path
    spec = workloads.Spec(name=f"b2100_w{window}", dtype="bf16", num_seqs=2100, q_heads=16,
                          kv_heads=4, head_dim=128, page_size=16, window=window, len_lo=1,
                          len_hi=300, pool_factor=1.25)
    sc = workloads.build(spec, 13, device="cuda")
    rng = np.random.default_rng(2)
    seqs = sorted(set(rng.choice(2100, 40, replace=False).tolist()) |
                  {0, 2099, int(np.argmax(sc.lens)), int(np.argmin(sc.lens))})
    check_step(sc, seqs=seqs)


# Attention sinks: the first S rows plus the last W - S.  The pools map only the pages of
# those rows (the table reads -1 between them), and rows of mapped pages that are not
# attended hold canaries or NaN, so a row read or weighted by mistake shows.
_GQA = dict(dtype="bf16", q_heads=32, kv_heads=8, head_dim=128)
SINKS = {
    "stream_p16_s4": dict(_GQA, num_seqs=64, page_size=16, window=256, sinks=4, len_lo=1,
                          len_hi=1200),
    "stream_p16_s40_nan": dict(_GQA, num_seqs=48, page_size=16, window=100, sinks=40,
                               len_lo=1, len_hi=700, spare="nan"),
    "stream_p16_s16": dict(_GQA, num_seqs=40, page_size=16, window=48, sinks=16, len_lo=1,
                           len_hi=300),
    "stream_p4_s10_w12": dict(_GQA, num_seqs=40, page_size=4, window=12, sinks=10, len_lo=1,
                              len_hi=90, spare="nan"),
    "stream_p8_s3": dict(_GQA, num_seqs=30, page_size=8, window=77, sinks=3, len_lo=1,
                         len_hi=400),
    "stream_slots_s5": dict(_GQA, num_seqs=24, page_size=16, window=64, sinks=5, len_lo=1,
                            len_hi=500, slot_table=True),
    "stream_g1_s2": dict(dtype="bf16", q_heads=8, kv_heads=8, head_dim=128, num_seqs=16,
                         page_size=32, window=40, sinks=2, len_lo=1, len_hi=200),
    "f32_generic_s3": dict(dtype="f32", q_heads=8, kv_heads=2, head_dim=64, num_seqs=20,
                           page_size=4, window=30, sinks=3, len_lo=1, len_hi=150, spare="nan"),
    "bf16_d32_s7": dict(dtype="bf16", q_heads=4, kv_heads=1, head_dim=32, num_seqs=20,
                        page_size=2, window=20, sinks=7, len_lo=1, len_hi=100),
}


@pytest.mark.parametrize("name", sorted(SINKS))
def test_sinks(name):
    sc = workloads.build(workloads.Spec(name=f"sinks_{name}", pool_factor=1.25, **SINKS[name]),
                         31, device="cuda")
    assert (sc.lens > sc.spec.window).any() and (sc.lens <= sc.spec.window).any()
    check_step(sc)


# Pages under 16 rows: the one-token streaming path takes tiles of 4 or 2 kv heads (as
# many as keep group x heads within 16 score columns and divide kv_heads), or of one head
# where no such set exists.  Every sequence against the oracle.
HEAD_SETS = {
    "hs4_p1_nan": dict(_GQA, num_seqs=48, page_size=1, len_lo=1, len_hi=700, spare="nan"),
    "hs4_p4_window_sinks": dict(_GQA, num_seqs=40, page_size=4, window=100, sinks=5, len_lo=1,
                                len_hi=600, spare="nan"),
    "hs4_g1_p4": dict(dtype="bf16", q_heads=8, kv_heads=8, head_dim=128, num_seqs=24,
                      page_size=4, len_lo=1, len_hi=500, spare="nan"),
    "hs2_g8_p8": dict(dtype="bf16", q_heads=64, kv_heads=8, head_dim=128, num_seqs=32,
                      page_size=8, len_lo=1, len_hi=900, spare="nan"),
    "hs2_kv6_p2": dict(dtype="bf16", q_heads=12, kv_heads=6, head_dim=128, num_seqs=20,
                       page_size=2, len_lo=1, len_hi=400, spare="nan"),
    "hs2_g8_slots_window": dict(dtype="bf16", q_heads=64, kv_heads=8, head_dim=128,
                                num_seqs=24, page_size=16, slot_table=True, window=300,
                                len_lo=1, len_hi=1500),
    "hs1_kv3_p4": dict(dtype="bf16", q_heads=12, kv_heads=3, head_dim=128, num_seqs=20,
                       page_size=4, len_lo=1, len_hi=400, spare="nan"),
}


@pytest.mark.parametrize("name", sorted(HEAD_SETS))
def test_head_sets_small_pages(name):
    sc = workloads.build(workloads.Spec(name=name, **HEAD_SETS[name]), 33, device="cuda")
    check_step(sc)


def test_sinks_batch_above_streaming_limit():
    # the chunked matrix-core path: sink chunks, then window chunks
    spec = workloads.Spec(name="sinks_b2100", dtype="bf16", num_seqs=2100, q_heads=16,
                          kv_heads=4, head_dim=128, page_size=16, window=200, sinks=24,
                          len_lo=1, len_hi=700, pool_factor=1.25, spare="nan")
    sc = workloads.build(spec, 17, device="cuda")
    rng = np.random.default_rng(3)
    seqs = sorted(set(rng.choice(2100, 40, replace=False).tolist()) |
                  {0, 2099, int(np.argmax(sc.lens)), int(np.argmin(sc.lens))})
    check_step(sc, seqs=seqs)


def test_sinks_equal_window_rows_differ_from_plain_window():
    # same pool, all rows stored: sinks change the result exactly where L > W
    spec = workloads.Spec(name="sinks_vs_window", **_GQA, num_seqs=32, page_size=16,
                          len_lo=1, len_hi=600, pool_factor=1.25)
    sc = workloads.build(spec, 5, device="cuda")
    o = ops()
    o.copy_pages(sc.k_pool, sc.v_pool, sc.copy_src, sc.copy_dst)
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    args = (sc.q, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens)
    W, S = 160, 8
    a = o.decode(*args, window=W, scale=sc.scale).cpu().double().numpy()
    b = o.decode(*args, window=W, sinks=S, scale=sc.scale).cpu().double().numpy()
    kp, vp = bits(sc.k_pool), bits(sc.v_pool)
    ref = oracle.attention.decode(bits(sc.q), kp, vp, ints(sc.block_tables), ints(sc.context_lens),
                                  16, W, sc.scale, "bf16", sinks=S)
    assert float(np.max(np.abs(b - ref))) <= TOL["bf16"]
    cut = sc.lens > W
    assert cut.any() and (~cut).any()
    # uncut sequences attend the same rows; the partition of the batch into ranges differs
    # between the two calls (more tiles with sinks), so only the rounding order may differ
    assert float(np.max(np.abs(a[~cut] - b[~cut]))) <= 1e-5
    assert (np.max(np.abs(a[cut] - b[cut]), axis=(1, 2)) > 1e-3).all()


# Several query tokens per sequence (prefill chunks, verify steps): the chunk's rows are
# stored by the step, then every query attends causally within its window.
MULTI = {
    "verify_g4_p16": dict(_GQA, num_seqs=48, page_size=16, len_lo=1, len_hi=700, q_lo=1,
                          q_hi=8, spare="nan"),
    "verify_g4_p16_w64": dict(_GQA, num_seqs=48, page_size=16, window=64, len_lo=1,
                              len_hi=700, q_lo=2, q_hi=8),
    "chunk_g4_p16": dict(_GQA, num_seqs=6, page_size=16, len_lo=40, len_hi=400, q_lo=20,
                         q_hi=90, spare="nan"),
    "chunk_g4_p16_w40": dict(_GQA, num_seqs=6, page_size=16, window=40, len_lo=40,
                             len_hi=400, q_lo=20, q_hi=90),
    "chunk_g1_p8": dict(dtype="bf16", q_heads=8, kv_heads=8, head_dim=128, num_seqs=5,
                        page_size=8, len_lo=1, len_hi=200, q_lo=1, q_hi=40),
    "verify_g2_p4_w9": dict(dtype="bf16", q_heads=8, kv_heads=4, head_dim=128, num_seqs=20,
                            page_size=4, window=9, len_lo=1, len_hi=120, q_lo=1, q_hi=6,
                            spare="nan"),
    "verify_g8_slots": dict(dtype="bf16", q_heads=64, kv_heads=8, head_dim=128, num_seqs=16,
                            page_size=16, len_lo=1, len_hi=500, q_lo=1, q_hi=5,
                            slot_table=True),
    "verify_g16_p32_w30": dict(dtype="bf16", q_heads=16, kv_heads=1, head_dim=128,
                               num_seqs=12, page_size=32, window=30, len_lo=1, len_hi=300,
                               q_lo=1, q_hi=4),
    # other paths: every query row as a row of its own
    "rows_f32_d64": dict(dtype="f32", q_heads=8, kv_heads=2, head_dim=64, num_seqs=8,
                         page_size=4, window=25, len_lo=1, len_hi=150, q_lo=1, q_hi=12,
                         spare="nan"),
    "rows_bf16_g3": dict(dtype="bf16", q_heads=12, kv_heads=4, head_dim=128, num_seqs=10,
                         page_size=16, len_lo=1, len_hi=400, q_lo=1, q_hi=10),
    "rows_bf16_d32": dict(dtype="bf16", q_heads=4, kv_heads=2, head_dim=32, num_seqs=10,
                          page_size=2, window=11, len_lo=1, len_hi=90, q_lo=1, q_hi=9),
}


# Long chunks over enough (sequence, kv head, 128-column) tiles: the tile kernel with K/V
# staged through LDS.
MULTI_TILE = {
    "tile_g4_p16": dict(_GQA, num_seqs=16, page_size=16, len_lo=130, len_hi=700, q_lo=60,
                        q_hi=130, spare="nan"),
    "tile_g4_p16_w100": dict(_GQA, num_seqs=16, page_size=16, window=100, len_lo=130,
                             len_hi=700, q_lo=60, q_hi=130),
    "tile_g4_p4_w37": dict(_GQA, num_seqs=16, page_size=4, window=37, len_lo=100, len_hi=500,
                           q_lo=70, q_hi=130, spare="nan"),
    "tile_g1_p8": dict(dtype="bf16", q_heads=8, kv_heads=8, head_dim=128, num_seqs=48,
                       page_size=8, len_lo=100, len_hi=400, q_lo=65, q_hi=140),
    "tile_g16_p32": dict(dtype="bf16", q_heads=32, kv_heads=2, head_dim=128, num_seqs=24,
                         page_size=32, len_lo=40, len_hi=300, q_lo=10, q_hi=130),
    "tile_g8_slots": dict(dtype="bf16", q_heads=64, kv_heads=8, head_dim=128, num_seqs=8,
                          page_size=16, len_lo=40, len_hi=400, q_lo=20, q_hi=140,
                          slot_table=True),
}


@pytest.mark.parametrize("name", sorted(MULTI_TILE))
def test_prefill_tile(name):
    sc = workloads.build(workloads.Spec(name=f"prefill_{name}", pool_factor=1.25,
                                        **MULTI_TILE[name]), 47, device="cuda")
    s = sc.spec
    G = s.q_heads // s.kv_heads
    tiles = s.num_seqs * s.kv_heads * -(-int(sc.nq.max()) // (128 // G))
    assert tiles >= 512 and int(sc.nq.max()) * G >= 48    # the tile path's conditions
    check_step(sc)


def _tile_shape(sc):
    s = sc.spec
    G = s.q_heads // s.kv_heads
    return (s.num_seqs * s.kv_heads * -(-int(sc.nq.max()) // (128 // G)) >= 512 and
            int(sc.nq.max()) * G >= 48)


def _prefill_ws(sc, scale):
    return ops().prefill_workspace_bytes(sc.q, sc.q_start, sc.k_pool, sc.v_pool,
                                         sc.block_tables, sc.context_lens,
                                         max_q_len=max(int(sc.nq.max()), 1),
                                         window=sc.spec.window, scale=scale,
                                         max_context_len=sc.max_context_len)


def test_prefill_tile_shape_negative_scale():
    # The tile kernel takes the block max of unscaled scores, so it serves positive
    # scales only; a negative one on the same long chunks goes to the streaming kernel
    # (which needs a workspace, the tile kernel none).
    kw = dict(MULTI_TILE["tile_g4_p16_w100"])
    sc = workloads.build(workloads.Spec(name="prefill_tile_negscale", pool_factor=1.25,
                                        scale=-0.0625, **kw), 53, device="cuda")
    assert _tile_shape(sc) and sc.scale < 0
    assert _prefill_ws(sc, 0.0625) == 0 and _prefill_ws(sc, sc.scale) > 0
    check_step(sc)


def test_empty_workspace_tensor_still_computes():
    # the tile kernel needs no workspace; an empty tensor (NULL pointer) must not turn
    # the call into a size query that leaves the output unwritten
    sc = workloads.build(workloads.Spec(name="prefill_tile_emptyws", pool_factor=1.25,
                                        **MULTI_TILE["tile_g4_p16"]), 61, device="cuda")
    assert _tile_shape(sc) and _prefill_ws(sc, sc.scale) == 0
    o = ops()
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    mq = int(sc.nq.max())
    kw = dict(max_q_len=mq, window=sc.spec.window, scale=sc.scale,
              max_context_len=sc.max_context_len)
    ref = o.prefill(sc.q, sc.q_start, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens,
                    **kw)
    out = torch.full_like(ref, float("nan"))
    empty = torch.zeros(0, dtype=torch.uint8, device="cuda")
    o.prefill(sc.q, sc.q_start, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens,
              out=out, workspace=empty, **kw)
    assert torch.equal(out, ref)


def test_prefill_tile_many_sequences():
    # more sequences than the tile kernel ranks (256): its work stays in index order
    spec = workloads.Spec(name="prefill_tile_b300", **_GQA, num_seqs=300, page_size=16,
                          len_lo=40, len_hi=300, q_lo=33, q_hi=40, pool_factor=1.25)
    sc = workloads.build(spec, 59, device="cuda")
    assert _tile_shape(sc) and sc.spec.num_seqs > 256
    assert _prefill_ws(sc, sc.scale) == 0
    rng = np.random.default_rng(5)
    rows = sorted(set(rng.choice(len(sc.q), 240, replace=False).tolist()) | {0, len(sc.q) - 1})
    check_step(sc, seqs=rows)


@pytest.mark.parametrize("name", sorted(MULTI))
def test_prefill(name):
    sc = workloads.build(workloads.Spec(name=f"prefill_{name}", pool_factor=1.25,
                                        **MULTI[name]), 37, device="cuda")
    assert int(sc.nq.max()) > 1
    check_step(sc)


def test_prefill_many_blocks_rows_path():
    # 64 sequences of up to 200 query tokens: more blocks than the streaming path takes,
    # so every query row runs as a row of its own on the chunked matrix-core kernel
    spec = workloads.Spec(name="prefill_b64_q200", **_GQA, num_seqs=64, page_size=16,
                          len_lo=150, len_hi=600, q_lo=150, q_hi=200, pool_factor=1.25)
    sc = workloads.build(spec, 41, device="cuda")
    rng = np.random.default_rng(4)
    rows = sorted(set(rng.choice(len(sc.q), 60, replace=False).tolist()) | {0, len(sc.q) - 1})
    check_step(sc, seqs=rows)


def test_prefill_more_queries_than_rows():
    # contexts shortened below the chunk length: queries before row 0 give zero rows
    spec = workloads.Spec(name="prefill_short", **_GQA, num_seqs=24, page_size=16, len_lo=1,
                          len_hi=120, q_lo=4, q_hi=24, pool_factor=1.25)
    sc = workloads.build(spec, 43, device="cuda")
    o = ops()
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    ctx = sc.context_lens.clone()
    ctx[::2] = torch.as_tensor(sc.nq[::2] // 2, device="cuda", dtype=torch.int32)
    assert int(sc.nq.max()) <= 32 and len(sc.q) >= 170
    for path in ("stream", "tile"):
        # the bound on query tokens picks the path: the shape's own bound (at most 32
        # tokens: 24 x 8 tiles, fewer than the tile kernel takes) streams; 170 makes
        # 24 x 8 x 6 tiles of 32 tokens, enough for the tile kernel
        mq = {"stream": max(int(sc.nq.max()), 1), "tile": 170}[path]
        out = o.prefill(sc.q, sc.q_start, sc.k_pool, sc.v_pool, sc.block_tables, ctx,
                        max_q_len=mq, scale=sc.scale).cpu().double().numpy()
        ref = oracle.attention.prefill(bits(sc.q), bits(sc.k_pool), bits(sc.v_pool),
                                       ints(sc.block_tables), ints(ctx), ints(sc.q_start), 16,
                                       0, sc.scale, "bf16")
        assert (ref == 0).all(axis=(1, 2)).any(), "no query before row 0"
        assert float(np.max(np.abs(out - ref))) <= TOL["bf16"], path


def test_prefill_single_token_equals_decode():
    # one query per sequence: pa_prefill and pa_decode attend the same rows
    sc = workloads.make_config(2, device="cuda")
    o = ops()
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    B = sc.spec.num_seqs
    qs = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    a = o.decode(sc.q, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens, scale=sc.scale)
    b = o.prefill(sc.q, qs, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens,
                  max_q_len=1, scale=sc.scale)
    assert float((a - b).abs().max()) <= 1e-5


@pytest.mark.parametrize("seed", range(60))
def test_random_small(seed):
    sc = workloads.build(workloads.random_spec(seed), seed, device="cuda")
    check_step(sc)


@pytest.mark.parametrize("seed", range(36))
def test_random_prefill(seed):
    spec = random_multi_spec(seed)
    sc = workloads.build(spec, 2000 + seed, device="cuda")
    if len(sc.q) > 1500:
        rng = np.random.default_rng(seed)
        rows = sorted(set(rng.choice(len(sc.q), 200, replace=False).tolist()) | {0, len(sc.q) - 1})
        check_step(sc, seqs=rows)
    else:
        check_step(sc)


EDGE = {
    "group16": dict(q_heads=16, kv_heads=1, head_dim=128, dtype="bf16"),
    "d256_bf16": dict(q_heads=4, kv_heads=2, head_dim=256, dtype="bf16"),
    "d256_f32": dict(q_heads=4, kv_heads=2, head_dim=256, dtype="f32"),
    "d16_bf16": dict(q_heads=6, kv_heads=3, head_dim=16, dtype="bf16"),
    "d64_g8": dict(q_heads=16, kv_heads=2, head_dim=64, dtype="bf16"),
    "window1": dict(q_heads=8, kv_heads=2, head_dim=128, window=1, len_lo=1, len_hi=300),
    "window_page_minus1": dict(q_heads=8, kv_heads=2, head_dim=128, window=15, len_lo=1, len_hi=300),
    "window_page_plus1": dict(q_heads=8, kv_heads=2, head_dim=128, window=17, len_lo=1, len_hi=300),
    "page1": dict(q_heads=8, kv_heads=2, head_dim=128, page_size=1, len_lo=0, len_hi=700),
    "page2_g4": dict(q_heads=8, kv_heads=2, head_dim=128, page_size=2, len_lo=0, len_hi=300),
    "long_multichunk": dict(num_seqs=3, q_heads=8, kv_heads=2, head_dim=128, len_lo=3000, len_hi=9000),
    "long_window": dict(num_seqs=3, q_heads=8, kv_heads=2, head_dim=128, window=2000, len_lo=2500, len_hi=9000),
    "empty_and_one": dict(num_seqs=4, q_heads=8, kv_heads=2, head_dim=128, lens=(0, 1, 0, 2)),
    "page3_generic": dict(q_heads=8, kv_heads=2, head_dim=128, page_size=3, len_lo=1, len_hi=400),
    "page32": dict(q_heads=12, kv_heads=4, head_dim=128, page_size=32, len_lo=1, len_hi=900),
    "page64_window": dict(q_heads=8, kv_heads=8, head_dim=128, page_size=64, window=100, len_lo=1, len_hi=900),
    "group3": dict(q_heads=6, kv_heads=2, head_dim=128, len_lo=1, len_hi=500),
    "group12_long": dict(num_seqs=3, q_heads=24, kv_heads=2, head_dim=128, len_lo=1500, len_hi=6000),
    # rows of mapped pages that hold no data are NaN: masked rows must never reach a product
    "nan_spare_p16": dict(q_heads=8, kv_heads=2, head_dim=128, len_lo=1, len_hi=300, spare="nan"),
    "nan_spare_window": dict(q_heads=8, kv_heads=2, head_dim=128, window=37, len_lo=1, len_hi=400, spare="nan"),
    "nan_spare_p1": dict(q_heads=8, kv_heads=2, head_dim=128, page_size=1, len_lo=0, len_hi=300, spare="nan"),
    "nan_spare_p64": dict(q_heads=16, kv_heads=4, head_dim=128, page_size=64, window=70, len_lo=1, len_hi=700, spare="nan"),
    "nan_spare_generic_f32": dict(q_heads=4, kv_heads=2, head_dim=64, dtype="f32", page_size=4, window=5, len_lo=1, len_hi=90, spare="nan"),
    "all_empty": dict(num_seqs=3, q_heads=8, kv_heads=2, head_dim=128, lens=(0, 0, 0)),
    # one sequence across the whole grid: every segment is cut into dozens of pieces
    "one_seq_20k": dict(num_seqs=1, q_heads=32, kv_heads=8, head_dim=128, lens=(20000,)),
    "one_seq_20k_g16": dict(num_seqs=1, q_heads=16, kv_heads=1, head_dim=128, lens=(20000,)),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge(name):
    base = dict(name=name, dtype="bf16", num_seqs=5, page_size=16, pool_factor=1.5)
    base.update(EDGE[name])
    sc = workloads.build(workloads.Spec(**base), 1234, device="cuda")
    check_step(sc)


def test_full_table_context():
    # the longest context the table can address: every entry used
    spec = workloads.Spec(name="full_table", dtype="bf16", num_seqs=2, q_heads=8, kv_heads=2,
                          head_dim=128, page_size=16, lens=(4096, 4095), bt_stride=256,
                          pool_factor=1.0)
    sc = workloads.build(spec, 5, device="cuda")
    check_step(sc)


def test_short_contexts_under_large_bound():
    # contexts far below max_context_len: the grid is sized for the bound, so most
    # wavefronts find no work and the ranges of the others hold a tile or two, cutting
    # segments into many pieces; the workspace was used before by a call of another shape
    spec = workloads.Spec(name="short_under_bound", dtype="bf16", num_seqs=6, q_heads=32,
                          kv_heads=8, head_dim=128, page_size=16, len_lo=1, len_hi=70,
                          bt_stride=256, pool_factor=1.5)
    sc = workloads.build(spec, 9, device="cuda")
    print(f"case {spec.name}", flush=True)
    o = ops()
    kp0, vp0 = bits(sc.k_pool), bits(sc.v_pool)
    o.copy_pages(sc.k_pool, sc.v_pool, sc.copy_src, sc.copy_dst)
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    bound = 256 * 16
    other = workloads.make_config(2, device="cuda", num_seqs=8)
    need = max(o.decode_workspace_bytes(sc.q, sc.k_pool, sc.v_pool, sc.block_tables,
                                        sc.context_lens, max_context_len=bound),
               o.decode_workspace_bytes(other.q, other.k_pool, other.v_pool, other.block_tables,
                                        other.context_lens,
                                        max_context_len=other.max_context_len))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    o.decode(other.q, other.k_pool, other.v_pool, other.block_tables, other.context_lens,
             max_context_len=other.max_context_len, workspace=ws)
    out = o.decode(sc.q, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens,
                   scale=sc.scale, max_context_len=bound, workspace=ws)
    torch.cuda.synchronize()
    _, _, ref = expected_step(sc, k_pool_bits=kp0, v_pool_bits=vp0)
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    assert float(np.max(np.abs(got - ref))) <= TOL["bf16"]


def _run_on_workspace(sc, ws, max_context_len=None):
    """copy -> store -> attention of ``sc`` with the caller's workspace and an output
    filled with NaN first (a row the call fails to write shows), checked against the
    oracle; then the workspace's counter header must read zero again."""
    o = ops()
    print(f"case {sc.spec.name} seed {sc.seed} max_context_len {max_context_len}", flush=True)
    kp0, vp0 = bits(sc.k_pool), bits(sc.v_pool)
    o.copy_pages(sc.k_pool, sc.v_pool, sc.copy_src, sc.copy_dst)
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    kv, vv = decode_views(sc)
    s = sc.spec
    out = torch.full((len(sc.q), s.q_heads, s.head_dim), float("nan"), device="cuda")
    bound = max_context_len or sc.max_context_len
    if sc.q_start is not None:
        o.prefill(sc.q, sc.q_start, kv, vv, sc.block_tables, sc.context_lens,
                  max_q_len=max(int(sc.nq.max()), 1), window=s.window, scale=sc.scale,
                  max_context_len=bound, out=out, workspace=ws)
    else:
        o.decode(sc.q, kv, vv, sc.block_tables, sc.context_lens, window=s.window,
                 sinks=s.sinks, scale=sc.scale, max_context_len=bound, out=out, workspace=ws)
    torch.cuda.synchronize()
    _, _, ref = expected_step(sc, k_pool_bits=kp0, v_pool_bits=vp0)
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all(), f"{s.name}: a row was not written"
    assert float(np.max(np.abs(got - ref))) <= TOL[s.dtype], s.name
    header = ws[:4096].cpu()
    assert int(header.count_nonzero()) == 0, f"{s.name}: counters left raised"
    return out


def _need(sc, max_context_len=None):
    o = ops()
    kv, vv = decode_views(sc)
    s = sc.spec
    bound = max_context_len or sc.max_context_len
    if sc.q_start is not None:
        return o.prefill_workspace_bytes(sc.q, sc.q_start, kv, vv, sc.block_tables,
                                         sc.context_lens, max_q_len=max(int(sc.nq.max()), 1),
                                         window=s.window, scale=sc.scale, max_context_len=bound)
    return o.decode_workspace_bytes(sc.q, kv, vv, sc.block_tables, sc.context_lens,
                                    window=s.window, sinks=s.sinks, max_context_len=bound)


def test_workspace_shared_by_every_path():
    """One workspace, zero-filled once, serves calls of every path and shape in turn:
    the per-row fp32 decode and prefill paths (partials right after the counter
    header), streaming decode with few wavefronts then many (small batch, then the
    batch-64 workload with a growing max_context_len), and streaming verify steps.
    Every call is checked against the oracle with a NaN-filled output, and leaves the
    counter header at zero."""
    tiny = workloads.make_config(1, device="cuda")
    small = workloads.make_config(2, device="cuda", num_seqs=5, name="gqa_b5")
    full = workloads.make_config(2, device="cuda")
    rows_multi = workloads.build(workloads.Spec(
        name="f32_prefill_rows", dtype="f32", num_seqs=6, q_heads=8, kv_heads=2,
        head_dim=64, page_size=4, len_lo=1, len_hi=80, q_lo=1, q_hi=6, pool_factor=1.5),
        5, device="cuda")
    verify = workloads.make_config(2, device="cuda", num_seqs=16, q_lo=4, q_hi=4,
                                   name="gqa_b16_q4")
    window = workloads.make_config(3, device="cuda", num_seqs=6, name="window_b6")
    # bounds at or above every context: the small batch takes more wavefronts with the
    # table's full 4096 rows than with its own longest context
    plan = [(tiny, None), (small, None), (small, 256 * 16), (full, None), (full, 256 * 16),
            (rows_multi, None), (verify, None), (small, None), (window, None), (tiny, None),
            (full, None)]
    need = max(_need(sc, mc) for sc, mc in plan)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = {}
    for sc, mc in plan:
        out = _run_on_workspace(sc, ws, mc)
        key = (sc.spec.name, mc)
        if key in outs:
            assert torch.equal(out, outs[key]), f"{key}: a repeated call differs"
        outs[key] = out


def test_workspace_reset_recovers_raised_counters():
    """A workspace whose counters were left raised (as after a call that did not
    complete) is usable again after pa_reset_workspace."""
    sc = workloads.make_config(2, device="cuda")
    ws = torch.zeros(_need(sc), dtype=torch.uint8, device="cuda")
    first = _run_on_workspace(sc, ws)
    ws[:4096] = 0x5A          # every counter raised
    ops().reset_workspace(ws)
    assert int(ws[:4096].count_nonzero()) == 0
    assert torch.equal(_run_on_workspace(sc, ws), first)


def test_deterministic_and_placement_invariant():
    spec = workloads.config_spec(2)
    sc = workloads.build(spec, 77, device="cuda")
    o = ops()
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    run = lambda kp, vp, bt: o.decode(sc.q, kp, vp, bt, sc.context_lens, scale=sc.scale,
                                      max_context_len=sc.max_context_len).clone()
    a = run(sc.k_pool, sc.v_pool, sc.block_tables)
    b = run(sc.k_pool, sc.v_pool, sc.block_tables)
    assert torch.equal(a, b), "two runs differ"
    perm = torch.randperm(sc.k_pool.shape[0], generator=torch.Generator().manual_seed(3)).cuda()
    kq = torch.empty_like(sc.k_pool)
    vq = torch.empty_like(sc.v_pool)
    kq[perm] = sc.k_pool
    vq[perm] = sc.v_pool
    bt = torch.where(sc.block_tables >= 0, perm[sc.block_tables.clamp(min=0).long()].int(),
                     sc.block_tables)
    c = run(kq, vq, bt)
    assert torch.equal(a, c), "physical placement changed the output"


def test_block_table_equals_slot_table():
    # the same pool read through a page table (P = 16) and through a raw slot table (P = 1)
    spec = workloads.Spec(name="bt_vs_slots", dtype="bf16", num_seqs=8, q_heads=32, kv_heads=8,
                          head_dim=128, page_size=16, len_lo=1, len_hi=2000, pool_factor=1.25)
    sc = workloads.build(spec, 21, device="cuda")
    o = ops()
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    bt = sc.block_tables.long()
    rows = torch.arange(bt.shape[1] * 16, device="cuda")
    slots = torch.where(bt[:, rows // 16] >= 0, bt[:, rows // 16] * 16 + rows % 16, 0).int()
    a = o.decode(sc.q, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens, scale=sc.scale)
    b = o.decode(sc.q, sc.k_pool.view(-1, 1, 8, 128), sc.v_pool.view(-1, 1, 8, 128),
                 slots.contiguous(), sc.context_lens, scale=sc.scale)
    torch.cuda.synchronize()
    # The two calls split the work differently (the slot table's pages of one row take
    # tiles of four kv heads), so their probabilities are rounded against different running
    # maxima: P keeps about 16 significant bits (a bf16 high part and a bf16 remainder), so
    # outputs of magnitude under 1 may differ by a few 1e-6.
    assert float((a - b).abs().max()) <= 1e-5


@pytest.mark.parametrize("q_len", [1, 64])
def test_pools_above_4gib(q_len):
    """Pools of more than 2^32 bytes, read with 64-bit offsets: the pages of a scenario are
    moved to the top of 4.3 GB pools (table entries shifted with them), so every K/V row
    lies past 4 GiB; decode (streaming kernel) and 64-token chunks (tile kernel) match the
    oracle of the scenario as built."""
    o = ops()
    spec = workloads.Spec(name=f"pool_4g_q{q_len}", dtype="bf16", num_seqs=32, q_heads=32,
                          kv_heads=8, head_dim=128, page_size=16, len_lo=64, len_hi=700,
                          q_lo=q_len, q_hi=q_len, spare="nan")
    sc = workloads.build(spec, 78, device="cuda")
    print(f"case {spec.name} seed {sc.seed}", flush=True)
    kp0, vp0 = bits(sc.k_pool), bits(sc.v_pool)
    _, _, ref = expected_step(sc, k_pool_bits=kp0, v_pool_bits=vp0)
    o.copy_pages(sc.k_pool, sc.v_pool, sc.copy_src, sc.copy_dst)
    o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    page_bytes = 16 * 8 * 128 * 2
    n = (1 << 32) // page_bytes + sc.pool_pages + 64
    base = n - sc.pool_pages
    big_k = torch.zeros((n, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    big_v = torch.zeros_like(big_k)
    big_k[base:] = sc.k_pool
    big_v[base:] = sc.v_pool
    bt = torch.where(sc.block_tables >= 0, sc.block_tables + base, sc.block_tables)
    assert base * page_bytes >= (1 << 32)
    if sc.q_start is not None:
        out = o.prefill(sc.q, sc.q_start, big_k, big_v, bt, sc.context_lens, max_q_len=q_len,
                        scale=sc.scale, max_context_len=sc.max_context_len)
    else:
        out = o.decode(sc.q, big_k, big_v, bt, sc.context_lens, scale=sc.scale,
                       max_context_len=sc.max_context_len)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    del big_k, big_v
    torch.cuda.empty_cache()
    err = float(np.max(np.abs(got - ref)))
    assert np.isfinite(got).all()
    assert err <= TOL["bf16"], f"max abs error {err:.3g}"


def test_decode_loop_with_allocator():
    """Several decode steps driven by the host allocator: forks, copy-on-write,
    window trims; pools stay bit-identical to the oracle's, outputs within tolerance."""
    from paged_kv_cache_41_amd.alloc import PagedKVCache
    o = ops()
    P, Hkv, Hq, D, W, N = 16, 2, 8, 128, 40, 96
    rng = np.random.default_rng(4)
    cache = PagedKVCache(N, P, free_order=rng.permutation(N).tolist())
    kpool = torch.full((N, P, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vpool = torch.full_like(kpool, float("nan"))
    kh, vh = bits(kpool), bits(vpool)
    rids = [0, 1, 2]
    for r in rids:
        cache.new(r)
    gen = torch.Generator(device="cuda").manual_seed(9)
    stride = 8
    worst = 0.0
    for step in range(70):
        if step == 20:
            cache.fork(1, 3); rids.append(3)
        if step == 37:
            cache.fork(0, 4); rids.append(4)
        plan = cache.plan_step(rids)
        B = len(rids)
        kn = torch.randn(B, Hkv, D, generator=gen, device="cuda").to(torch.bfloat16)
        vn = torch.randn(B, Hkv, D, generator=gen, device="cuda").to(torch.bfloat16)
        q = torch.randn(B, Hq, D, generator=gen, device="cuda").to(torch.bfloat16)
        bt_np = np.stack([np.array(cache.table(r)[:stride] + [-1] * (stride - len(cache.table(r)[:stride])))
                          for r in rids]).astype(np.int32)
        # a request longer than the table never occurs: W keeps the live pages few
        cs, cd = (torch.as_tensor(plan.copy_src, device="cuda"),
                  torch.as_tensor(plan.copy_dst, device="cuda"))
        slots = torch.as_tensor(plan.slots, device="cuda")
        ctx = torch.as_tensor(plan.context_lens, device="cuda")
        bt = torch.as_tensor(bt_np, device="cuda")
        o.copy_pages(kpool, vpool, cs, cd)
        o.store_kv(kpool, vpool, kn, vn, slots)
        out = o.decode(q, kpool, vpool, bt, ctx, window=W, scale=D ** -0.5)
        torch.cuda.synchronize()
        kh, vh = oracle.kvstore.copy_pages(kh, vh, plan.copy_src, plan.copy_dst)
        kh, vh = oracle.kvstore.store_kv(kh, vh, bits(kn), bits(vn), plan.slots)
        assert np.array_equal(bits(kpool), kh) and np.array_equal(bits(vpool), vh), f"step {step}"
        ref = oracle.attention.decode(bits(q), kh, vh, bt_np, plan.context_lens, P, W,
                                      D ** -0.5, "bf16")
        err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
        worst = max(worst, err)
        assert err <= TOL["bf16"], f"step {step}: {err}"
        for r, L in zip(rids, plan.context_lens):
            cache.trim(r, int(L) + 1 - W)
    assert worst > 0


def test_update_tables_scatter():
    """pa_update_tables against the oracle scatter, bit for bit: mapped, released and
    out-of-table cells, pages of 1, 4 and 16 rows."""
    o = ops()
    rng = np.random.default_rng(12)
    for P in (1, 4, 16):
        rows_n, stride = 37, 24
        cells = rng.choice(rows_n * (stride + 2), 300, replace=False)
        rows = (cells // (stride + 2)).astype(np.int32)
        js = (cells % (stride + 2)).astype(np.int32)           # some past the block table
        rows[::17] = rows_n + 3 + np.arange(len(rows[::17]))      # some outside both tables
        pages = rng.integers(-1, 5000, size=300).astype(np.int32)
        bt0 = rng.integers(-1, 5000, size=(rows_n, stride)).astype(np.int32)
        st0 = rng.integers(0, 5000, size=(rows_n, stride * P - 5)).astype(np.int32)
        bt_ref, st_ref = oracle.tables.update_tables(bt0, st0, rows, js, pages, P, 77777)
        bt = torch.as_tensor(bt0, device="cuda")
        st = torch.as_tensor(st0, device="cuda")
        dv = lambda a: torch.as_tensor(a, device="cuda")
        o.update_tables(dv(rows), dv(js), dv(pages), page_size=P, block_tables=bt,
                        slot_table=st, dummy_slot=77777)
        torch.cuda.synchronize()
        assert np.array_equal(bt.cpu().numpy(), bt_ref), P
        assert np.array_equal(st.cpu().numpy(), st_ref), P


def test_decode_loop_device_tables():
    """A decode loop whose block and slot tables live on the device and change only by
    scattering the allocator's updates each step (forks, copy-on-write, sink pages, window
    trims, a release and a new request in its row): the tables equal the allocator's, and
    decode through either table matches the oracle."""
    from paged_kv_cache_41_amd.alloc import PagedKVCache
    o = ops()
    P, Hkv, Hq, D, W, S, N = 16, 2, 8, 128, 40, 4, 96
    rng = np.random.default_rng(6)
    cache = PagedKVCache(N, P, free_order=rng.permutation(N).tolist())
    # page N is the dummy page of the slot table: real memory no request is given
    kpool = torch.full((N + 1, P, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vpool = torch.full_like(kpool, float("nan"))
    kpool[N] = 0
    vpool[N] = 0
    kh, vh = bits(kpool), bits(vpool)
    ROWS, BTS, STS, DUMMY = 6, 8, 128, N * P
    bt = torch.full((ROWS, BTS), -1, dtype=torch.int32, device="cuda")
    st = torch.full((ROWS, STS), DUMMY, dtype=torch.int32, device="cuda")
    row_of = {}
    for r in (0, 1, 2):
        cache.new(r, sinks=S)
        row_of[r] = r
    gen = torch.Generator(device="cuda").manual_seed(3)
    dv = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32), device="cuda")
    for step in range(80):
        if step == 20:
            cache.fork(1, 3); row_of[3] = 3
        if step == 45:
            cache.release(0)
        if step == 50:
            cache.new(5, sinks=S); row_of[5] = 0               # reuses the released row
        rids = sorted(r for r in row_of if r in cache.pages)
        if step == 45:
            rids = [r for r in rids if r != 0]
        plan = cache.plan_step(rids)
        rows, js, pages = cache.take_table_updates(row_of)
        if step == 45:
            del row_of[0]
        o.update_tables(dv(rows), dv(js), dv(pages), page_size=P, block_tables=bt,
                        slot_table=st, dummy_slot=DUMMY)
        B = len(rids)
        kn = torch.randn(B, Hkv, D, generator=gen, device="cuda").to(torch.bfloat16)
        vn = torch.randn(B, Hkv, D, generator=gen, device="cuda").to(torch.bfloat16)
        q = torch.randn(B, Hq, D, generator=gen, device="cuda").to(torch.bfloat16)
        o.copy_pages(kpool, vpool, dv(plan.copy_src), dv(plan.copy_dst))
        o.store_kv(kpool, vpool, kn, vn, dv(plan.slots))
        sel = dv([row_of[r] for r in rids]).long()
        btb, stb = bt[sel].contiguous(), st[sel].contiguous()
        ref_bt = cache.block_tables(rids, BTS)
        ref_st = cache.slot_table(rids, STS, dummy_slot=DUMMY)
        ctx = plan.context_lens
        got_bt, got_st = btb.cpu().numpy(), stb.cpu().numpy()
        assert np.array_equal(got_bt, ref_bt), f"step {step}"
        for i, L in enumerate(ctx):
            assert np.array_equal(got_st[i, :L], ref_st[i, :L]), f"step {step} row {i}"
        ctxd = dv(ctx)
        out1 = o.decode(q, kpool, vpool, btb, ctxd, window=W, sinks=S, scale=D ** -0.5)
        flat_k, flat_v = kpool.view(-1, 1, Hkv, D), vpool.view(-1, 1, Hkv, D)
        out2 = o.decode(q, flat_k, flat_v, stb, ctxd, window=W, sinks=S, scale=D ** -0.5)
        torch.cuda.synchronize()
        kh, vh = oracle.kvstore.copy_pages(kh, vh, plan.copy_src, plan.copy_dst)
        kh, vh = oracle.kvstore.store_kv(kh, vh, bits(kn), bits(vn), plan.slots)
        ref = oracle.attention.decode(bits(q), kh, vh, ref_bt, ctx, P, W, D ** -0.5, "bf16",
                                      sinks=S)
        for out in (out1, out2):
            err = float(np.max(np.abs(out.cpu().double().numpy() - ref)))
            assert err <= TOL["bf16"], f"step {step}: {err}"
        for r, L in zip(rids, ctx):
            cache.trim(r, int(L) + 1 - (W - S))
    assert 5 in cache.pages and cache.length[5] == 30


def test_batch_at_streaming_limit():
    # exactly as many sequences as the streaming path takes
    spec = workloads.Spec(name="b2048", dtype="bf16", num_seqs=2048, q_heads=8, kv_heads=2,
                          head_dim=128, page_size=16, len_lo=0, len_hi=64, pool_factor=1.25)
    sc = workloads.build(spec, 19, device="cuda")
    rng = np.random.default_rng(5)
    seqs = sorted(set(rng.choice(2048, 40, replace=False).tolist()) | {0, 2047})
    check_step(sc, seqs=seqs)


def test_graph_replays_match_eager():
    """The step (table scatter, copy, store, decode; and a verify step through pa_prefill)
    captured in a HIP graph and replayed several times, with eager work and
    synchronizations in between: every replay equals the eager result bit for bit.  The
    workspaces are zero-filled once before capture; the calls put their counters back to
    zero themselves, so no memset is recorded."""
    o = ops()
    sc = workloads.make_config(2, device="cuda")
    s = sc.spec
    B = s.num_seqs
    ws = torch.zeros(o.decode_workspace_bytes(sc.q, sc.k_pool, sc.v_pool, sc.block_tables,
                                              sc.context_lens, max_context_len=sc.max_context_len),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(B, s.q_heads, s.head_dim, device="cuda")
    # a table update that rewrites each sequence's last page with itself (same values)
    rows = torch.arange(B, dtype=torch.int32, device="cuda")
    js = torch.as_tensor(((np.maximum(sc.lens, 1) - 1) // 16).astype(np.int32), device="cuda")
    pages = sc.block_tables[rows.long(), js.long()].contiguous()
    k0, v0 = sc.k_pool.clone(), sc.v_pool.clone()
    qv = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    outv = torch.empty_like(out)
    wsv = torch.zeros(max(o.prefill_workspace_bytes(sc.q, qv, sc.k_pool, sc.v_pool,
                                                    sc.block_tables, sc.context_lens,
                                                    max_q_len=1), 1),
                      dtype=torch.uint8, device="cuda")

    def step():
        o.update_tables(rows, js, pages, page_size=16, block_tables=sc.block_tables)
        o.copy_pages(sc.k_pool, sc.v_pool, sc.copy_src, sc.copy_dst)
        o.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
        o.decode(sc.q, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens, scale=sc.scale,
                 max_context_len=sc.max_context_len, out=out, workspace=ws)
        o.prefill(sc.q, qv, sc.k_pool, sc.v_pool, sc.block_tables, sc.context_lens, max_q_len=1,
                  scale=sc.scale, out=outv, workspace=wsv)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()                                   # eager, on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    want, wantv = out.clone(), outv.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step()
    for i in range(4):
        out.fill_(float("nan"))
        outv.fill_(float("nan"))
        sc.k_pool.copy_(k0)                      # eager work between the replays
        sc.v_pool.copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {i}: decode differs from the eager call"
        assert torch.equal(outv, wantv), f"replay {i}: verify step differs from the eager call"
    assert not torch.isnan(want).any()
    assert (ws[:4096] == 0).all(), "the arrival counters must be back at zero"

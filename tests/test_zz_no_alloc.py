"""pa_decode_noalloc (the entry point for callers that cannot allocate) against
pa_decode_hinted, through the C ABI: two calls in a row, the second smaller, on the
library's static scratch buffer."""
import numpy as np
import pytest
import torch

import workloads
from helpers import bits, expected_step

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _views(sc):
    if sc.table_page_size == sc.spec.page_size:
        return sc.k_pool, sc.v_pool
    hkv, d = sc.spec.kv_heads, sc.spec.head_dim
    return sc.k_pool.view(-1, 1, hkv, d), sc.v_pool.view(-1, 1, hkv, d)


def _both(sc, unshared):
    """The no-allocation call and the workspace call on the same stored step."""
    from paged_kv_cache_41_amd import ops
    s = sc.spec
    print(f"case {s.name} seed {sc.seed}", flush=True)
    kp0, vp0 = bits(sc.k_pool), bits(sc.v_pool)
    ops.copy_pages(sc.k_pool, sc.v_pool, sc.copy_src, sc.copy_dst)
    ops.store_kv(sc.k_pool, sc.v_pool, sc.k_new, sc.v_new, sc.slot_mapping)
    kv, vv = _views(sc)
    kw = dict(window=s.window, sinks=s.sinks, scale=sc.scale, max_context_len=sc.max_context_len,
              unshared_pages=unshared)
    out = torch.full((len(sc.q), s.q_heads, s.head_dim), float("nan"), device="cuda")
    ops.decode_noalloc(sc.q, kv, vv, sc.block_tables, sc.context_lens, out=out, **kw)
    ref_call = ops.decode(sc.q, kv, vv, sc.block_tables, sc.context_lens, **kw)
    torch.cuda.synchronize()
    _, _, ref = expected_step(sc, k_pool_bits=kp0, v_pool_bits=vp0)
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    assert torch.equal(out, ref_call), f"{s.name}: differs from pa_decode_hinted"
    assert float(np.max(np.abs(got - ref))) <= TOL[s.dtype], s.name


def test_noalloc_matches_workspace_call_large_then_small():
    # the batch-64 workload (1024 wavefronts, partials far into the buffer), then a
    # batch of 5 with fewer wavefronts on the same buffer
    _both(workloads.make_config(2, device="cuda"), True)
    _both(workloads.make_config(2, device="cuda", num_seqs=5, name="gqa_b5"), False)


def test_noalloc_head_sets_on_small_pages():
    # pages of one row (a raw slot table, G = 8: tiles of two kv heads, 16-column
    # partials), then pages of 4 rows at G = 4 (four heads per tile), on the same buffer
    _both(workloads.make_config(5, device="cuda", num_seqs=48, len_hi=6000,
                                name="slot_b48"), True)
    _both(workloads.build(workloads.Spec(name="p4_b16", dtype="bf16", num_seqs=16, q_heads=32,
                                         kv_heads=8, head_dim=128, page_size=4, len_lo=1,
                                         len_hi=900, spare="nan"), 35, device="cuda"), False)


def test_noalloc_other_paths_and_sinks():
    # the window workload with sinks (streaming), then the per-row fp32 path (its
    # partials start after the counter header), then the streaming path again
    _both(workloads.make_config(3, device="cuda", sinks=4, num_seqs=8, name="window_b8_s4"), True)
    _both(workloads.make_config(1, device="cuda"), False)
    _both(workloads.make_config(2, device="cuda", num_seqs=3, name="gqa_b3"), False)


def test_noalloc_rejects_calls_beyond_the_buffer():
    from paged_kv_cache_41_amd import _lib, ops
    # per-row path (more than 2048 sequences) with long contexts: far more partials than
    # the buffer holds; rejected before anything is launched
    B, hq, hkv, d = 3000, 32, 8, 128
    q = torch.zeros(B, hq, d, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(4, 16, hkv, d, dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros(B, 2048, dtype=torch.int32, device="cuda")
    ctx = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.zeros(B, hq, d, device="cuda")
    with pytest.raises(_lib.PAError) as e:
        ops.decode_noalloc(q, pool, pool, bt, ctx, out=out, max_context_len=32768)
    assert e.value.status == _lib.PA_ESCRATCH

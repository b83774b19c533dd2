"""The seeded scenarios have the shapes and structure the five workloads name."""
import math

import numpy as np
import torch

import workloads
from oracle.shadow import window_bound


def test_tiny_f32():
    sc = workloads.make_config(1)
    assert list(sc.lens) == [5, 17, 32, 40]
    assert sc.pool_pages == 64 and tuple(sc.block_tables.shape) == (4, 10)
    assert sc.k_pool.dtype == torch.float32 and sc.scale == 0.25
    bt = sc.block_tables.numpy()
    mapped = bt[bt >= 0]
    assert len(mapped) == 25 and len(set(mapped.tolist())) == 25
    # the new rows land at page offsets 0, 0, 3, 3
    assert [int(s) % 4 for s in sc.slot_mapping] == [0, 0, 3, 3]


def test_unmapped_pages_are_nan_and_spare_rows_are_canaries():
    sc = workloads.make_config(1)
    bt = sc.block_tables.numpy()
    mapped = set(bt[bt >= 0].tolist())
    for p in range(sc.pool_pages):
        page = sc.k_pool[p]
        if p in mapped:
            assert torch.isfinite(page).all()
        else:
            assert torch.isnan(page).all()
    # the slot of each new row holds a canary before the store
    flat = sc.k_pool.reshape(-1, 2, 16)
    for s in sc.slot_mapping.tolist():
        assert (flat[s] == workloads.K_CANARY).all()


def test_gqa_b64_shape():
    sc = workloads.make_config(2)
    assert sc.spec.q_heads == 32 and sc.spec.kv_heads == 8 and sc.spec.head_dim == 128
    assert tuple(sc.block_tables.shape) == (64, 256)
    assert sc.lens.min() >= 1 and sc.lens.max() <= 4096
    needed = int(sum(-(-int(L) // 16) for L in sc.lens))
    assert sc.pool_pages == math.ceil(1.25 * needed)
    assert abs(sc.scale - 1 / math.sqrt(128)) < 1e-8
    assert len(sc.copy_src) == 0


def test_window_b32_footprint():
    sc = workloads.make_config(3)
    bt = sc.block_tables.numpy()
    assert bt.shape == (32, 2048)
    assert sc.lens.min() >= 2048 and sc.lens.max() <= 32768
    bound = window_bound(1024, 16)
    for s, L in enumerate(sc.lens):
        live = np.nonzero(bt[s] >= 0)[0]
        assert 1 <= len(live) <= bound
        assert live[0] == (L - 1024) // 16 and live[-1] == (L - 1) // 16
        assert (bt[s, :live[0]] == -1).all()


def test_prefix_b256_sharing_and_copies():
    sc = workloads.make_config(4)
    bt = sc.block_tables.numpy()
    assert bt.shape == (256, 161)
    assert (bt[:, :128] == bt[0, :128]).all() and (bt[0, :128] >= 0).all()
    assert ((sc.lens - 2049 >= 0) & (sc.lens - 2049 <= 512)).all()
    need_copy = (sc.lens - 1) % 16 != 0
    assert len(sc.copy_src) == int(need_copy.sum())
    assert len(set(sc.copy_dst.tolist())) == len(sc.copy_dst)
    assert not set(sc.copy_dst.tolist()) & set(sc.copy_src.tolist())
    # after the step every table maps the copy, never the shared tail page
    assert set(sc.copy_dst.tolist()) <= set(bt[need_copy].ravel().tolist())
    assert not set(sc.copy_src.tolist()) & set(bt.ravel().tolist())


def test_slot_table_layout():
    sc = workloads.make_config(5, num_seqs=16)
    st = sc.block_tables.numpy()
    assert st.shape == (17, 32768) and sc.table_page_size == 1
    dummy = (sc.pool_pages - 1) * 16
    assert (st[16] == dummy).all()
    for s, L in enumerate(sc.lens):
        assert 1 <= L <= 32768
        row = st[s, :L]
        assert (row < dummy).all() and (row[::16] % 16 == 0).all()
        assert (st[s, L:] == dummy).all()
    assert sc.table_num_pages == sc.pool_pages * 16


def test_seeded_and_reproducible():
    a = workloads.make_config(2, num_seqs=8)
    b = workloads.make_config(2, num_seqs=8)
    assert torch.equal(a.block_tables, b.block_tables)
    assert torch.equal(a.k_pool.view(torch.int16), b.k_pool.view(torch.int16))
    c = workloads.make_config(2, seed=5, num_seqs=8)
    assert not torch.equal(a.block_tables, c.block_tables)

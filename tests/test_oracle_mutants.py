"""Plant one-line mistakes in the oracle (on the CPU) and check that a pin catches each.

This is the mutation method of the silicon-compiler chapter 15 (section
"Mutation tests") applied to the oracle: a pin set that lets a plausible
mistake through is not pinning anything.
"""
import numpy as np
import pytest

import oracle
import pins
from oracle import attention as A
from oracle import kvstore as S
from oracle import shadow as SH
from oracle import tables as TB

_live, _gather, _head, _attend = A.live_rows, A.gather, A.kv_head_of, A.attend
_rows, _gather_rows = A.attended_rows, A.gather_rows
_qpos = A.query_position
_upd = TB.update_tables
_store, _copy = S.store_kv, S.copy_pages
_exact, _exact_s = SH.pages_exact, SH.pages_exact_sinks
_wbound, _sbound = SH.window_bound, SH.sink_bound


def _gather_shift_page(pool, table_row, lo, hi, dtype):
    # the page lookup ignores the logical page index offset by one
    return _gather(pool, np.concatenate([table_row[1:], table_row[:1]]), lo, hi, dtype)


def _gather_bad_offset(pool, table_row, lo, hi, dtype):
    P = pool.shape[1]
    out = _gather(pool, table_row, lo, hi, dtype)
    if P > 1 and hi - lo > 1:
        out = out.copy()
        out[1:] = out[:-1].copy()       # every row read one slot early
    return out


def _attend_no_norm(q, K, V, scale):
    z = scale * (K @ q)
    w = np.exp(z - z.max())
    return w @ V


def _attend_keys(q, K, V, scale):
    return _attend(q, K, K, scale)


def _attend_no_scale(q, K, V, scale):
    return _attend(q, K, V, 1.0)


def _store_off_by_one(k, v, kn, vn, slots):
    return _store(k, v, kn, vn, np.where(np.asarray(slots) >= 0, np.asarray(slots) + 1, -1) % (k.shape[0] * k.shape[1]))


def _store_k_into_v(k, v, kn, vn, slots):
    return _store(k, v, kn, kn, slots)


def _copy_empty(k, v, src, dst):
    return k.copy(), v.copy()


def _copy_keys_only(k, v, src, dst):
    k2, _ = _copy(k, v, src, dst)
    return k2, v.copy()


def _sinks_window_too_long(L, W, S=0):
    # the window part keeps W rows instead of W - S
    if W <= 0 or S <= 0:
        return _rows(L, W, S)
    return sorted(set(range(min(S, L))) | set(range(*_live(L, W))))


def _gather_rows_first_dup(pool, table_row, rows, dtype):
    # the first kept row read twice, the second never
    rows = list(rows)
    if len(rows) > 1:
        rows[1] = rows[0]
    return _gather_rows(pool, table_row, rows, dtype)


def _upd_release_as_page0(bt, st, rows, js, pages, P, dummy):
    return _upd(bt, st, rows, js, [max(int(p), 0) for p in pages], P, dummy)


def _upd_slot_page_size_one(bt, st, rows, js, pages, P, dummy):
    # the slot table written as if pages held one row
    return _upd(bt, None, rows, js, pages, P, dummy)[0], _upd(None, st, rows, js, pages, 1, dummy)[1]


def _upd_next_page(bt, st, rows, js, pages, P, dummy):
    return _upd(bt, st, rows, [int(j) + 1 for j in js], pages, P, dummy)


MUTANTS = {
    "gather starts one row late": (A, "live_rows", lambda L, W: (min(_live(L, W)[0] + 1, L), L)),
    "window keeps W+1 rows": (A, "live_rows", lambda L, W: _live(L, W + 1 if W > 0 else 0)),
    "window ignored": (A, "live_rows", lambda L, W: (0, L)),
    "last row dropped": (A, "live_rows", lambda L, W: (_live(L, W)[0], max(L - 1, _live(L, W)[0]))),
    "page lookup off by one": (A, "gather", _gather_shift_page),
    "row offset off by one": (A, "gather", _gather_bad_offset),
    "GQA heads interleaved": (A, "kv_head_of", lambda h, hq, hkv: h % hkv),
    "softmax not normalised": (A, "attend", _attend_no_norm),
    "keys where values belong": (A, "attend", _attend_keys),
    "scale dropped": (A, "attend", _attend_no_scale),
    "store one slot late": (S, "store_kv", _store_off_by_one),
    "store writes K into V": (S, "store_kv", _store_k_into_v),
    "copy-on-write copy is empty": (S, "copy_pages", _copy_empty),
    "copy forgets V": (S, "copy_pages", _copy_keys_only),
    "sinks ignored": (A, "attended_rows", lambda L, W, S=0: _rows(L, W, 0)),
    "sinks keep one row too many": (A, "attended_rows", lambda L, W, S=0: _rows(L, W, S + 1 if 0 < S < W - 1 else S)),
    "window beside the sinks too long": (A, "attended_rows", _sinks_window_too_long),
    "sink gather reads one row twice": (A, "gather_rows", _gather_rows_first_dup),
    "queries placed at the chunk start": (A, "query_position", lambda L, n, i: i),
    "queries one row late": (A, "query_position", lambda L, n, i: _qpos(L, n, i) + 1),
    "queries one row early": (A, "query_position", lambda L, n, i: _qpos(L, n, i) - 1),
    "every query at the chunk end": (A, "query_position", lambda L, n, i: L - 1),
    "released cell written as page 0": (TB, "update_tables", _upd_release_as_page0),
    "slot table written with pages of one row": (TB, "update_tables", _upd_slot_page_size_one),
    "update lands one page late": (TB, "update_tables", _upd_next_page),
    "window count rounds keep_from up": (SH, "pages_exact", lambda rows, kf, P: max(-(-rows // P) - -(-kf // P), 0) if rows > 0 else 0),
    "sink pages trimmed with the window": (SH, "pages_exact_sinks", lambda rows, kf, head, P: _exact(rows, kf, P)),
    "sink count releases one page more": (SH, "pages_exact_sinks", lambda rows, kf, head, P: max(_exact_s(rows, kf, head, P) - (1 if kf // P > head else 0), 0)),
    "window bound without the partly filled page": (SH, "window_bound", lambda W, P: _wbound(W, P) - 1),
    "sink bound without the partly filled page": (SH, "sink_bound", lambda W, S, P: _sbound(W, S, P) - 1),
    "sink bound counts the sinks inside the window": (SH, "sink_bound", lambda W, S, P: -(-S // P) + _wbound(W, P)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_caught(name, monkeypatch):
    mod, attr, fn = MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            problems = pin()
        except Exception as e:          # a crash is a catch too
            problems = [repr(e)]
        if problems:
            caught.append(pin.__name__)
    assert caught, f"mutant '{name}' survived every pin"


def test_unbroken_oracle_passes():
    assert all(pin() == [] for pin in pins.ALL_PINS)

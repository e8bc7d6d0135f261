"""Pins of the oracle's KV rollback (CPU only): hand-computed slot and page
lists for the worked examples and page-boundary cases."""
import numpy as np
import pytest


def _table(B, pages_per_req, seed=0):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(B * pages_per_req).astype(np.int32)
    return perm.reshape(B, pages_per_req)


def test_fig1_shape_rollback(orc):
    """TRT-MTP Fig. 1 shape: K=5, j=3 (A, B, C accepted after root G).  The
    root and three drafts stay; D and E (positions L+4, L+5) are rolled back."""
    K, L = 5, 100
    t = _table(1, 3, 1)
    rb = orc.kv_rollback(t, np.array([3], np.int32), np.array([L], np.int32), K)
    assert rb["seq_lens"][0] == L + 4
    expect = [t[0, p // 64] * 64 + p % 64 for p in (104, 105)]
    assert list(rb["rb_slots"][: rb["rb_offsets"][1]]) == expect
    assert list(rb["freed_offsets"]) == [0, 0]


def test_page_boundary_freeing(orc):
    """Positions 60..65 straddle logical pages 0 and 1 (page size 64)."""
    K, L = 5, 60
    t = _table(4, 2, 2)
    acc = np.array([3, 4, 5, 0], np.int32)
    rb = orc.kv_rollback(t, acc, np.full(4, L, np.int32), K)
    # new_len = 64, 65, 66, 61
    assert list(rb["seq_lens"]) == [64, 65, 66, 61]
    # request 0 keeps 60..63 -> logical page 1 holds nothing kept -> freed
    # request 1 keeps 64 -> page 1 stays; request 2 keeps all; request 3 keeps 60
    assert list(rb["freed_offsets"]) == [0, 1, 1, 1, 2]
    assert rb["freed"][0] == t[0, 1] and rb["freed"][1] == t[3, 1]
    slots = rb["rb_slots"]
    off = rb["rb_offsets"]
    assert list(off) == [0, 2, 3, 3, 8]
    assert list(slots[0:2]) == [t[0, 1] * 64 + 0, t[0, 1] * 64 + 1]
    assert list(slots[2:3]) == [t[1, 1] * 64 + 1]
    assert list(slots[3:8]) == [t[3, 0] * 64 + 61, t[3, 0] * 64 + 62, t[3, 0] * 64 + 63,
                                t[3, 1] * 64 + 0, t[3, 1] * 64 + 1]


def test_invalid_accept_count_rolls_back_whole_step(orc):
    K, L = 3, 10
    t = _table(2, 1, 3)
    rb = orc.kv_rollback(t, np.array([-1, 7], np.int32), np.full(2, L, np.int32), K)
    assert rb["n_bad"] == 2
    assert list(rb["seq_lens"]) == [L, L]
    assert list(rb["rb_offsets"]) == [0, 4, 8]
    assert list(rb["rb_slots"][:4]) == [t[0, 0] * 64 + p for p in range(10, 14)]


def test_all_accepted_rolls_back_nothing(orc):
    K = 4
    t = _table(3, 2, 4)
    rb = orc.kv_rollback(t, np.full(3, K, np.int32), np.array([0, 59, 63], np.int32), K)
    assert list(rb["seq_lens"]) == [5, 64, 68]
    assert list(rb["rb_offsets"]) == [0, 0, 0, 0]
    assert list(rb["freed_offsets"]) == [0, 0, 0, 0]


def test_poison_zeroes_only_rejected_slots(orc):
    K, L, H, d = 3, 62, 2, 4
    t = _table(1, 2, 5)
    kc = np.ones((2, H, 64, d), np.float32)
    vc = np.ones((2, H, 64, d), np.float32)
    rb = orc.kv_rollback(t, np.array([1], np.int32), np.array([L], np.int32), K, poison=True,
                         k_cache=kc, v_cache=vc, n_kv_heads=H, d_k=d, d_v=d)
    zero = {(t[0, p // 64], p % 64) for p in (64, 65)}
    for pg in range(2):
        for off in range(64):
            z = (pg, off) in zero
            assert (kc[pg, :, off] == 0).all() == z
            assert (vc[pg, :, off] == 0).all() == z
    assert rb["seq_lens"][0] == 64

"""Checks of the shared input generator (CPU only)."""
import numpy as np

import sdsynth


def test_philox_known_answers():
    """Known-answer vectors published with the Random123 library for
    philox4x32-10 (Salmon et al., SC'11)."""
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF),
         (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, expect in cases:
        got = sdsynth.philox4x32_10(np.array(ctr, np.uint32), key)
        assert tuple(int(x) for x in got) == expect


def test_uniforms_range_and_streams():
    a = sdsynth.philox_uniforms(7, 64, 9, sdsynth.STREAM_ACCEPT)
    b = sdsynth.philox_uniforms(7, 64, 9, sdsynth.STREAM_SAMPLE)
    assert a.dtype == np.float32 and (a >= 0).all() and (a < 1).all()
    assert not np.array_equal(a, b)
    assert np.array_equal(a, sdsynth.philox_uniforms(7, 64, 9, sdsynth.STREAM_ACCEPT))
    assert abs(float(a.mean()) - 0.5) < 0.05


def test_truncated_geometric_distribution():
    B, K, p = 40000, 3, 0.4
    j = sdsynth.truncated_geometric(11, B, K, p)
    freq = np.bincount(j, minlength=K + 1) / B
    expect = [p * (1 - p) ** k for k in range(K)] + [(1 - p) ** K]
    assert np.allclose(freq, expect, atol=0.01)


def test_greedy_drafts_realise_prefix():
    rng = np.random.default_rng(0)
    B, K, V = 200, 4, 50
    tt = rng.integers(0, V, (B, K + 1))
    d = sdsynth.greedy_drafts(tt, K, V, seed=3)
    j = sdsynth.truncated_geometric(3, B, K, 0.4)
    for b in range(B):
        n = 0
        while n < K and d[b, n] == tt[b, n]:
            n += 1
        assert n == j[b]
        assert ((d[b] >= 0) & (d[b] < V)).all()


def test_paged_layout_is_a_permutation():
    seq = np.array([5, 200, 64, 1000], np.int32)
    table, total = sdsynth.paged_layout(seq, 5, 64, 0, seed=9)
    used = table[table >= 0]
    assert len(used) == total and len(set(used.tolist())) == total
    for b, L in enumerate(seq):
        assert (table[b] >= 0).sum() == (L + 5 + 63) // 64

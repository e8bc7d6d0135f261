"""Pins of the oracle's verify attention, append and LM head (CPU only)."""
import math

import numpy as np
import pytest


def _identity_pages(B, Q, L, ps=64, extra=0):
    need = (L + Q + extra + ps - 1) // ps
    table = np.arange(B * need, dtype=np.int32).reshape(B, need)
    return table, B * need


def _gqa_cache(num_pages, Hkv, ps, d, fill=0.0):
    return np.full((num_pages, Hkv, ps, d), fill, np.float32)


def test_single_key_returns_its_value(orc):
    """L = 0 and K = 0: the only key is the query's own, so o = v."""
    rng = np.random.default_rng(0)
    B, Q, H, d = 2, 1, 3, 8
    seq = np.zeros(B, np.int32)
    table, P = _identity_pages(B, Q, 0)
    kc, vc = _gqa_cache(P, H, 64, d), _gqa_cache(P, H, 64, d)
    q = rng.standard_normal((B, Q, H, d)).astype(np.float32)
    kn = rng.standard_normal((B, Q, H, d)).astype(np.float32)
    vn = rng.standard_normal((B, Q, H, d)).astype(np.float32)
    orc.kv_append(seq, table, P, kn, vn, kc, vc)
    o = orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=H, d_v=d)
    assert np.array_equal(o, vn.astype(np.float64))


def test_two_keys_closed_form(orc):
    """Scores 0 and ln 3 (scale 1): weights 1/4 and 3/4."""
    d = 4
    q = np.zeros((1, 1, 1, d), np.float32)
    q[..., 0] = 1.0
    seq = np.array([1], np.int32)
    table, P = _identity_pages(1, 1, 1)
    kc, vc = _gqa_cache(P, 1, 64, d), _gqa_cache(P, 1, 64, d)
    v1 = np.array([1.0, 2.0, -4.0, 0.5], np.float32)
    v2 = np.array([5.0, -2.0, 8.0, 0.25], np.float32)
    vc[0, 0, 0] = v1
    kn = np.zeros((1, 1, 1, d), np.float32)
    kn[..., 0] = np.float32(math.log(3.0))
    vn = v2.reshape(1, 1, 1, d)
    orc.kv_append(seq, table, P, kn, vn, kc, vc)
    o = orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=1, d_v=d, scale=1.0)
    w2 = 3.0 * math.exp(float(np.float32(math.log(3.0))) - math.log(3.0))
    expect = (v1.astype(np.float64) + w2 * v2.astype(np.float64)) / (1.0 + w2)
    np.testing.assert_allclose(o[0, 0, 0], expect, rtol=1e-14, atol=1e-14)


def test_equal_keys_give_mean_of_values(orc):
    rng = np.random.default_rng(1)
    B, Q, H, d, L = 1, 3, 2, 16, 70
    seq = np.array([L], np.int32)
    table, P = _identity_pages(B, Q, L)
    kc = _gqa_cache(P, H, 64, d)
    key = rng.standard_normal(d).astype(np.float32)
    kc[:] = key
    vc = rng.standard_normal((P, H, 64, d)).astype(np.float32)
    kn = np.broadcast_to(key, (B, Q, H, d)).copy()
    vn = rng.standard_normal((B, Q, H, d)).astype(np.float32)
    q = rng.standard_normal((B, Q, H, d)).astype(np.float32)
    orc.kv_append(seq, table, P, kn, vn, kc, vc)
    o = orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=H, d_v=d)
    for i in range(Q):
        n = L + i + 1
        vals = np.stack([vc[p // 64, :, p % 64] for p in range(n)]).astype(np.float64)
        np.testing.assert_allclose(o[0, i], vals.mean(0), rtol=1e-12, atol=1e-12)


def test_causal_mask_includes_diagonal_excludes_future(orc):
    """Query i sees key L+i (its own) but not L+i+1: perturbing key L+i+1
    changes only outputs of queries > i; perturbing key L+i changes query i."""
    rng = np.random.default_rng(2)
    B, Q, H, d, L = 1, 4, 1, 8, 5
    seq = np.array([L], np.int32)
    table, P = _identity_pages(B, Q, L)
    base_k = rng.standard_normal((P, H, 64, d)).astype(np.float32)
    base_v = rng.standard_normal((P, H, 64, d)).astype(np.float32)
    q = rng.standard_normal((B, Q, H, d)).astype(np.float32)
    kn = rng.standard_normal((B, Q, H, d)).astype(np.float32)
    vn = rng.standard_normal((B, Q, H, d)).astype(np.float32)

    def run(kn_, vn_):
        kc, vc = base_k.copy(), base_v.copy()
        orc.kv_append(seq, table, P, kn_, vn_, kc, vc)
        return orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=H, d_v=d)

    o0 = run(kn, vn)
    for t in range(Q):
        vn2 = vn.copy()
        vn2[0, t] += 100.0
        o1 = run(kn, vn2)
        for i in range(Q):
            changed = not np.array_equal(o0[0, i], o1[0, i])
            assert changed == (i >= t), (t, i)


def test_page_permutation_invariance(orc):
    rng = np.random.default_rng(4)
    B, Q, Hq, Hkv, d = 3, 3, 4, 2, 16
    seq = np.array([130, 7, 64], np.int32)
    need = (seq + Q + 63) // 64
    P = int(need.sum())
    t1 = np.full((B, need.max()), -1, np.int32)
    t2 = np.full((B, need.max()), -1, np.int32)
    perm = rng.permutation(P).astype(np.int32)
    off = 0
    for b in range(B):
        t1[b, : need[b]] = np.arange(off, off + need[b])
        t2[b, : need[b]] = perm[off: off + need[b]]
        off += need[b]
    logical_k = [rng.standard_normal((need[b] * 64, Hkv, d)).astype(np.float32) for b in range(B)]
    logical_v = [rng.standard_normal((need[b] * 64, Hkv, d)).astype(np.float32) for b in range(B)]

    def fill(table):
        kc = np.zeros((P, Hkv, 64, d), np.float32)
        vc = np.zeros((P, Hkv, 64, d), np.float32)
        for b in range(B):
            for p in range(need[b] * 64):
                kc[table[b, p // 64], :, p % 64] = logical_k[b][p]
                vc[table[b, p // 64], :, p % 64] = logical_v[b][p]
        return kc, vc

    q = rng.standard_normal((B, Q, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((B, Q, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((B, Q, Hkv, d)).astype(np.float32)
    outs = []
    for t in (t1, t2):
        kc, vc = fill(t)
        orc.kv_append(seq, t, P, kn, vn, kc, vc)
        outs.append(orc.verify_attn(q, kc, vc, t, seq, P, n_kv_heads=Hkv, d_v=d))
    assert np.array_equal(outs[0], outs[1])


def test_gqa_head_mapping(orc):
    """Hq=6, Hkv=2: query heads 0-2 read kv head 0, heads 3-5 kv head 1.
    Constant values per kv head make the output that constant."""
    rng = np.random.default_rng(6)
    B, Q, Hq, Hkv, d, L = 1, 2, 6, 2, 8, 40
    seq = np.array([L], np.int32)
    table, P = _identity_pages(B, Q, L)
    kc = rng.standard_normal((P, Hkv, 64, d)).astype(np.float32)
    vc = np.zeros((P, Hkv, 64, d), np.float32)
    vc[:, 0] = 1.5
    vc[:, 1] = -2.5
    kn = rng.standard_normal((B, Q, Hkv, d)).astype(np.float32)
    vn = np.zeros((B, Q, Hkv, d), np.float32)
    vn[:, :, 0] = 1.5
    vn[:, :, 1] = -2.5
    q = rng.standard_normal((B, Q, Hq, d)).astype(np.float32)
    orc.kv_append(seq, table, P, kn, vn, kc, vc)
    o = orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=Hkv, d_v=d)
    np.testing.assert_allclose(o[0, :, :3], 1.5, rtol=1e-14)
    np.testing.assert_allclose(o[0, :, 3:], -2.5, rtol=1e-14)


def test_mla_latent_split(orc):
    """MLA: keys are the whole latent row, values its first d_v entries.
    With all scores equal, the output is the mean of the first d_v entries,
    and the trailing (key-only) entries never reach the output."""
    rng = np.random.default_rng(7)
    B, Q, Hq, dqk, dv, L = 1, 2, 3, 12, 8, 20
    seq = np.array([L], np.int32)
    table, P = _identity_pages(B, Q, L)
    lat = rng.standard_normal((P, 64, dqk)).astype(np.float32)
    q = np.zeros((B, Q, Hq, dqk), np.float32)  # zero query: uniform weights
    kn = rng.standard_normal((B, Q, dqk)).astype(np.float32)
    orc.kv_append(seq, table, P, kn, None, lat, None, mla=True)
    o = orc.verify_attn(q, lat, None, table, seq, P, n_kv_heads=1, d_v=dv, mla=True)
    for i in range(Q):
        n = L + i + 1
        rows = np.stack([lat[p // 64, p % 64] for p in range(n)]).astype(np.float64)
        for h in range(Hq):
            np.testing.assert_allclose(o[0, i, h], rows[:, :dv].mean(0), rtol=1e-12)
    # Scores use all d_qk entries: a query on the last (key-only) coordinate
    # changes the weights.
    q2 = np.zeros_like(q)
    q2[..., dqk - 1] = 3.0
    o2 = orc.verify_attn(q2, lat, None, table, seq, P, n_kv_heads=1, d_v=dv, mla=True)
    assert not np.allclose(o2, o)


def test_attention_selection_matches_full(orc):
    rng = np.random.default_rng(8)
    B, Q, Hq, Hkv, d = 2, 3, 4, 2, 8
    seq = np.array([10, 70], np.int32)
    table, P = _identity_pages(B, Q, int(seq.max()))
    kc = rng.standard_normal((P, Hkv, 64, d)).astype(np.float32)
    vc = rng.standard_normal((P, Hkv, 64, d)).astype(np.float32)
    q = rng.standard_normal((B, Q, Hq, d)).astype(np.float32)
    full = orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=Hkv, d_v=d)
    sel = np.array([[1, 2, 3], [0, 0, 1], [1, 0, 0]], np.int32)
    part = orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=Hkv, d_v=d, sel=sel)
    for r, (b, i, h) in enumerate(sel):
        assert np.array_equal(part[r], full[b, i, h])


def test_lm_head_unit_rows_transpose(orc):
    """H = unit rows e_m: logits[m][v] = W[v][m] (catches a transposed operand)."""
    rng = np.random.default_rng(9)
    M, hidden, V = 5, 7, 11
    H = np.zeros((M, hidden), np.float32)
    for m in range(M):
        H[m, m] = 1.0
    W = rng.standard_normal((V, hidden)).astype(np.float32)
    out = orc.lm_head(H, W)
    assert np.array_equal(out, W[:, :M].T.astype(np.float64))


def test_lm_head_rank_one_closed_form(orc):
    """H[m][k] = m+1, W[v][k] = v - 3 for all k: logits = hidden (m+1)(v-3)."""
    M, hidden, V = 4, 96, 9
    H = np.tile(np.arange(1, M + 1, dtype=np.float32)[:, None], (1, hidden))
    W = np.tile((np.arange(V, dtype=np.float32) - 3)[:, None], (1, hidden))
    out = orc.lm_head(H, W)
    expect = hidden * np.outer(np.arange(1, M + 1), np.arange(V) - 3).astype(np.float64)
    assert np.array_equal(out, expect)
    out_rows = orc.lm_head(H, W, rows=[3, 0])
    assert np.array_equal(out_rows, expect[[3, 0]])


def test_lm_head_bf16_inputs(orc):
    """bf16 bit patterns are read exactly: 1.5 * 2.5 summed 64 times."""
    one_five = np.uint16(0x3FC0)   # 1.5
    two_five = np.uint16(0x4020)   # 2.5
    H = np.full((1, 64), one_five, np.uint16)
    W = np.full((2, 64), two_five, np.uint16)
    out = orc.lm_head(H, W)
    assert np.array_equal(out, np.full((1, 2), 64 * 3.75))


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80), (1.0 + 2 ** -8, 0x3F80),            # tie -> even (1.0)
    (1.0 + 3 * 2 ** -8, 0x3F82),                       # tie -> even (1 + 2^-6)
    (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),                # above the tie -> up
    (-2.0 - 2 ** -7, -1), (3.0e38, 0x7F62), (4.0e38, 0x7F80),
    (2 ** -133, 0x0001), (2 ** -134, 0x0000), (0.0, 0x0000),
])
def test_round_bf16(orc, x, bits):
    got = int(orc.round_bf16(np.array([x]))[0])
    if bits == -1:
        # -2 - 2^-7: spacing in [2, 4) is 2^-6, so this is a tie between
        # -2 (mantissa 0, even) and -2 - 2^-6 -> -2.
        assert got == 0xC000
    else:
        assert got == bits, hex(got)

"""Pins of the oracle's FP8 (OCP E4M3, "fn" variant) KV-cache support (CPU only).

The format itself is not on the pages (they name FP8 attention only as prior
art, [TRT-MTP] "支持 MTP 的注意力機制"); its values are fixed by the OCP 8-bit
floating-point specification, and torch ships an independent implementation
of it (torch.float8_e4m3fn) that the decode and the in-range encode are
checked against.  The scaled attention is pinned by exact identities with the
bf16-cache attention, which the other oracle tests pin.
"""
import math

import numpy as np
import pytest
import torch


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_on_every_code(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = orc.e4m3_decode(codes), _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_decode_named_values(orc):
    v = orc.e4m3_decode(np.array([0x7E, 0x08, 0x01, 0x07, 0x38, 0x00, 0x80, 0xFE, 0x40], np.uint8))
    assert v[0] == 448.0                       # largest finite: 1.75 * 2^8
    assert v[1] == 2.0 ** -6                   # smallest normal
    assert v[2] == 2.0 ** -9                   # smallest subnormal
    assert v[3] == 7 * 2.0 ** -9               # largest subnormal
    assert v[4] == 1.0
    assert v[5] == 0.0 and not math.copysign(1, v[5]) < 0
    assert v[6] == 0.0 and math.copysign(1, v[6]) < 0
    assert v[7] == -448.0
    assert v[8] == 2.0


def test_encode_round_trips_every_finite_code(orc):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes)


def _finite_magnitudes(orc):
    return orc.e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448, increasing


def test_encode_matches_torch_at_midpoints_and_near_them(orc):
    """Every midpoint between neighbouring magnitudes (ties to even), the
    float32 neighbours on either side of it, and both signs."""
    m = _finite_magnitudes(orc)
    assert np.all(np.diff(m) > 0)
    mid = ((m[:-1] + m[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (m[:-1] + m[1:]) / 2)  # exact in f32
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    x = np.concatenate([mid, up, dn, m.astype(np.float32)])
    x = np.concatenate([x, -x])
    assert np.array_equal(orc.e4m3_encode(x.astype(np.float64)), _torch_encode(x))
    # ties go to the even code: 1 + 1/16 lies between 0x38 (1.0) and 0x39
    # (1.125) -> 0x38; 1 + 3/16 between 0x39 and 0x3A (1.25) -> 0x3A
    assert orc.e4m3_encode(np.array([1.0625, 1.1875]))[0] == 0x38
    assert orc.e4m3_encode(np.array([1.0625, 1.1875]))[1] == 0x3A


def test_encode_matches_torch_on_random_in_range_values(orc):
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = np.clip(x, -448, 448).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(x.astype(np.float64)), _torch_encode(x))


def test_encode_saturates_and_maps_nan(orc):
    x = np.array([448.0, 448.5, 464.0, 479.9, 480.0, 1e6, np.inf, -500.0, -np.inf, np.nan,
                  -0.0, 0.0, 2.0 ** -10, 2.0 ** -10 * 1.0001, 3 * 2.0 ** -10])
    c = orc.e4m3_encode(x)
    assert c.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F,
                          0x80, 0x00,
                          0x00,   # half the smallest subnormal: tie -> even code 0
                          0x01,   # just above it: rounds up to 2^-9
                          0x02]   # 1.5 * 2^-9: tie between codes 1 and 2 -> 2


def _pages(B, Q, L, ps=64):
    need = (L + Q + ps - 1) // ps
    return np.arange(B * need, dtype=np.int32).reshape(B, need)[:, ::-1].copy(), B * need


def test_quantizing_append_stores_codes_of_value_over_scale(orc):
    """Append into an E4M3 cache equals the elementwise encode of the same
    append into an f64 cache, divided by the kv head's scale."""
    rng = np.random.default_rng(3)
    B, Q, Hkv, d = 3, 4, 3, 16
    seq = np.array([5, 64, 130], np.int32)
    table, P = _pages(B, Q, int(seq.max()))
    kn = (rng.standard_normal((B, Q, Hkv, d)) * 4).astype(np.float32)
    vn = (rng.standard_normal((B, Q, Hkv, d)) * 0.3).astype(np.float32)
    ks = np.array([0.5, 0.01, 3.0], np.float32)
    vs = np.array([0.002, 1.0, 0.25], np.float32)
    k8 = np.full((P, Hkv, 64, d), 0xAA, np.uint8)
    v8 = np.full((P, Hkv, 64, d), 0xAA, np.uint8)
    kf = np.full((P, Hkv, 64, d), np.nan, np.float64)
    vf = np.full((P, Hkv, 64, d), np.nan, np.float64)
    orc.kv_append(seq, table, P, kn, vn, k8, v8, k_scale=ks, v_scale=vs)
    orc.kv_append(seq, table, P, kn.astype(np.float64), vn.astype(np.float64), kf, vf)
    written = ~np.isnan(kf)
    assert np.array_equal(written, ~np.isnan(vf))
    assert np.all(k8[~written] == 0xAA) and np.all(v8[~written] == 0xAA)
    ek = orc.e4m3_encode(kf / ks.astype(np.float64).reshape(1, -1, 1, 1))
    ev = orc.e4m3_encode(vf / vs.astype(np.float64).reshape(1, -1, 1, 1))
    assert np.array_equal(k8[written], ek[written])
    assert np.array_equal(v8[written], ev[written])


def _case(orc, seed, B=2, Q=3, Hq=6, Hkv=3, d=16, L=(70, 9)):
    rng = np.random.default_rng(seed)
    seq = np.array(L[:B], np.int32)
    table, P = _pages(B, Q, int(seq.max()))
    vals_k = rng.standard_normal((P, Hkv, 64, d)) * 2
    vals_v = rng.standard_normal((P, Hkv, 64, d))
    k8 = orc.e4m3_encode(vals_k)
    v8 = orc.e4m3_encode(vals_v)
    q = orc.round_bf16(rng.standard_normal((B, Q, Hq, d)))
    return seq, table, P, q, k8, v8


def test_attention_with_unit_scales_equals_bf16_cache_attention(orc):
    """Every E4M3 value is a bf16 value, so with scales 1 the FP8 attention
    equals the bf16 attention over the decoded cache, bit for bit."""
    seq, table, P, q, k8, v8 = _case(orc, 5)
    Hkv, d = k8.shape[1], k8.shape[3]
    one = np.ones(Hkv, np.float32)
    o8 = orc.verify_attn(q, k8, v8, table, seq, P, n_kv_heads=Hkv, d_v=d, k_scale=one,
                         v_scale=one)
    kb = orc.round_bf16(orc.e4m3_decode(k8))
    vb = orc.round_bf16(orc.e4m3_decode(v8))
    assert np.array_equal(orc.bf16_to_f64(kb), orc.e4m3_decode(k8))
    ob = orc.verify_attn(q, kb, vb, table, seq, P, n_kv_heads=Hkv, d_v=d)
    assert np.array_equal(o8, ob)


def test_attention_power_of_two_head_scales_are_exact(orc):
    """k_scale[h] = 2^a_h, v_scale[h] = 2^c_h: equals the bf16 attention over
    the decoded cache with kv head h's keys times 2^a_h and values times
    2^c_h (exact in bf16), bit for bit.  Distinct per-head exponents catch a
    wrong head index or swapped K/V scales."""
    seq, table, P, q, k8, v8 = _case(orc, 6)
    Hkv, d = k8.shape[1], k8.shape[3]
    ks = np.array([0.25, 2.0, 8.0], np.float32)
    vs = np.array([4.0, 0.5, 0.125], np.float32)
    o8 = orc.verify_attn(q, k8, v8, table, seq, P, n_kv_heads=Hkv, d_v=d, k_scale=ks,
                         v_scale=vs)
    kd = orc.e4m3_decode(k8) * ks.astype(np.float64).reshape(1, -1, 1, 1)
    vd = orc.e4m3_decode(v8) * vs.astype(np.float64).reshape(1, -1, 1, 1)
    kb, vb = orc.round_bf16(kd), orc.round_bf16(vd)
    assert np.array_equal(orc.bf16_to_f64(kb), kd) and np.array_equal(orc.bf16_to_f64(vb), vd)
    ob = orc.verify_attn(q, kb, vb, table, seq, P, n_kv_heads=Hkv, d_v=d)
    assert np.array_equal(o8, ob)
    # and the result differs from the one with the scales swapped between heads
    o_sw = orc.verify_attn(q, k8, v8, table, seq, P, n_kv_heads=Hkv, d_v=d,
                           k_scale=ks[::-1].copy(), v_scale=vs)
    assert not np.allclose(o_sw, o8)


def test_attention_value_scale_is_linear(orc):
    """The output is linear in the value scale: v_scale = c gives c times the
    output of v_scale = 1 (up to fp64 rounding)."""
    seq, table, P, q, k8, v8 = _case(orc, 7)
    Hkv, d = k8.shape[1], k8.shape[3]
    ks = np.array([0.3, 0.07, 1.7], np.float32)
    c = np.array([0.0123, 3.3, 0.71], np.float32)
    o1 = orc.verify_attn(q, k8, v8, table, seq, P, n_kv_heads=Hkv, d_v=d, k_scale=ks,
                         v_scale=np.ones(Hkv, np.float32))
    oc = orc.verify_attn(q, k8, v8, table, seq, P, n_kv_heads=Hkv, d_v=d, k_scale=ks,
                         v_scale=c)
    G = q.shape[2] // Hkv
    per_head = np.repeat(c.astype(np.float64), G).reshape(1, 1, -1, 1)
    np.testing.assert_allclose(oc, o1 * per_head, rtol=1e-13, atol=1e-300)


def test_fp8_attention_rejects_mla(orc):
    seq, table, P, q, k8, v8 = _case(orc, 8)
    with pytest.raises(ValueError):
        orc.verify_attn(q, k8, None, table, seq, P, n_kv_heads=1, d_v=8, mla=True,
                        k_scale=np.ones(1, np.float32), v_scale=np.ones(1, np.float32))

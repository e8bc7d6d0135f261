"""GPU parity of the FP8 (E4M3) KV-cache verify attention, append and rollback
poisoning against the fp64 oracle.  Tolerances: see tests/parity.py
(attention rows within 2e-3 of the row's largest magnitude; cache bytes and
rollback outputs bit-exact)."""

import numpy as np
import pytest
import torch

import oracle
import sdsynth
import speculative_decoding_sd_amd as sdv
from parity import DEV, bits, host, check_attention

pytestmark = pytest.mark.gpu


def _case(B, K, Hq, Hkv, D, lens, seed, extra=0):
    cfg = sdsynth.Config(name="case", batch=B, K=K, n_q_heads=Hq, n_kv_heads=Hkv, d_qk=D,
                         d_v=D, mla=False, hidden=Hq * D, vocab=8, dtype="bf16", seq_len=None,
                         kv_cache="e4m3")
    return sdsynth.make_workload(cfg, seed, device="cpu", seq_lens=np.array(lens),
                                 extra_tokens=extra, with_lm_head=False)


def _run_gpu(wl, append=True, max_seq_len=None):
    t = wl.tensors
    q, kc, vc = t["q"].to(DEV), t["k_cache"].to(DEV), t["v_cache"].to(DEV)
    ks, vs = t["k_scale"].to(DEV), t["v_scale"].to(DEV)
    kn = t["k_new"].to(DEV) if append else None
    vn = t["v_new"].to(DEV) if append else None
    pt = torch.tensor(wl.page_table, device=DEV)
    sl = torch.tensor(wl.seq_lens, device=DEV)
    B, Q, Hq, D = q.shape
    out = torch.full((B, Q, Hq, D), -5.0, dtype=torch.float32, device=DEV)
    lowp = torch.empty((B * Q, Hq * D), dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    d = sdv.attn_desc(q=q, k_cache=kc, v_cache=vc, page_table=pt, seq_lens=sl, out=out,
                      n_kv_heads=wl.cfg.n_kv_heads, num_pages=wl.num_pages,
                      max_seq_len=int(max_seq_len or wl.seq_lens.max()), k_new=kn, v_new=vn,
                      out_lowp=lowp, dev_error=err, k_scale=ks, v_scale=vs)
    assert d.kv_format == sdv.SD_KV_E4M3
    sdv.verify_attn(d)
    torch.cuda.synchronize()
    return out, lowp, kc, vc, int(err.item())


def _oracle(wl, sel=None, append=True):
    t = wl.tensors
    kc, vc = t["k_cache"].numpy().copy(), t["v_cache"].numpy().copy()
    ks, vs = t["k_scale"].numpy(), t["v_scale"].numpy()
    if append:
        oracle.kv_append(wl.seq_lens, wl.page_table, wl.num_pages, host(t["k_new"]),
                         host(t["v_new"]), kc, vc, k_scale=ks, v_scale=vs)
    ref = oracle.verify_attn(host(t["q"]), kc, vc, wl.page_table, wl.seq_lens, wl.num_pages,
                             n_kv_heads=wl.cfg.n_kv_heads, d_v=wl.cfg.d_v, sel=sel,
                             k_scale=ks, v_scale=vs)
    return ref, kc, vc


@pytest.mark.parametrize("B,K,Hq,Hkv,D,lens", [
    (3, 5, 16, 4, 128, [0, 61, 1300]),      # 24 rows/kv head; L=0; page-straddling append
    (2, 7, 10, 2, 64, [5, 700]),            # 40 rows/kv head (two row blocks), head dim 64
    (2, 7, 40, 8, 128, [3000, 1000]),       # long-context head layout: 40 rows, 16-row blocks
    (2, 10, 6, 2, 128, [0, 200]),           # 33 rows (fewest in 16-row blocks); L = 0
    (3, 7, 12, 2, 128, [17, 64, 2049]),     # 48 rows (most in 16-row blocks)
    (4, 4, 32, 8, 128, [512, 4097, 777, 64]),  # serving head layout, ragged
    (1, 0, 4, 1, 64, [33]),                 # K = 0: plain single-token decode
    (3, 3, 8, 1, 64, [95, 1, 2000]),        # one kv head, 32 rows, tails of 1..31 keys
    (2, 15, 8, 2, 64, [33, 1500]),          # 64 rows per kv head: the largest supported
])
def test_attention_gqa_e4m3(B, K, Hq, Hkv, D, lens):
    wl = _case(B, K, Hq, Hkv, D, lens, seed=20 + B + K)
    out, lowp, kc, vc, err = _run_gpu(wl)
    ref, kc_ref, vc_ref = _oracle(wl)
    assert err == 0
    check_attention(out.cpu().numpy(), ref, where=f"e4m3 {B},{K},{Hq},{Hkv},{D}")
    assert np.array_equal(kc.cpu().numpy(), kc_ref) and np.array_equal(vc.cpu().numpy(), vc_ref)
    exp_lowp = oracle.round_bf16(out.cpu().numpy().astype(np.float64)).reshape(B * (K + 1), -1)
    assert np.array_equal(bits(lowp), exp_lowp)


def test_attention_e4m3_long_chunks_sampled():
    """Long requests (1024-key chunks, segments of several chunks per wave)."""
    B, K, Hq, Hkv, D = 8, 7, 40, 8, 128
    lens = [30000, 29001, 26000, 28111, 30031, 25555, 29999, 27000]
    wl = _case(B, K, Hq, Hkv, D, lens, seed=78)
    out, _, _, _, err = _run_gpu(wl)
    rng = np.random.default_rng(1)
    sel = np.stack([rng.integers(0, B, 48), rng.integers(0, K + 1, 48), rng.integers(0, Hq, 48)], 1)
    ref, _, _ = _oracle(wl, sel=sel)
    o = out.cpu().numpy()
    assert err == 0
    check_attention(np.stack([o[b, i, h] for b, i, h in sel]), ref, where="e4m3 long chunks")


def test_attention_e4m3_preappended_and_errors():
    """k_new = NULL over a cache that already holds the step; a request with a
    bad page entry is flagged and gets NaN rows beside a valid one."""
    wl = _case(2, 3, 8, 2, 128, [100, 300], seed=9)
    ref, kc_ref, vc_ref = _oracle(wl)
    wl.tensors["k_cache"] = torch.from_numpy(kc_ref)
    wl.tensors["v_cache"] = torch.from_numpy(vc_ref)
    out, _, _, _, err = _run_gpu(wl, append=False)
    assert err == 0
    check_attention(out.cpu().numpy(), ref, where="e4m3 pre-appended")
    wl.page_table[1, 2] = wl.num_pages + 1
    out, _, _, _, err = _run_gpu(wl, append=False)
    assert err & sdv.SD_DERR_PAGE
    o = out.cpu().numpy()
    assert np.isnan(o[1]).all()
    check_attention(o[0], ref[0], where="e4m3 valid request beside a faulty one")


def test_append_e4m3_special_values_bit_exact():
    """The quantizing append on values that probe every branch of the code
    conversion: zeros of both signs, saturation (large finite, infinities),
    NaN, exact ties (power-of-two scale), subnormal codes, underflow to zero,
    and inexact quotients (non-power-of-two scale)."""
    B, K, Hq, Hkv, D = 2, 3, 4, 2, 64
    wl = _case(B, K, Hq, Hkv, D, [10, 70], seed=4)
    t = wl.tensors
    specials = [0.0, -0.0, 1e30, -1e30, float("inf"), float("-inf"), float("nan"),
                1.0625, 1.1875, -1.0625, 448.0, 464.0, 2.0 ** -10, 3 * 2.0 ** -10,
                2.0 ** -7, 2.0 ** -30, -2.0 ** -9, 0.3, -7.77, 123.0, 0.0155]
    rng = np.random.default_rng(2)
    kn = rng.standard_normal((B, K + 1, Hkv, D)).astype(np.float32) * 3
    vn = rng.standard_normal((B, K + 1, Hkv, D)).astype(np.float32) * 0.01
    flat_k, flat_v = kn.reshape(-1), vn.reshape(-1)
    flat_k[:len(specials)] = specials
    flat_v[-len(specials):] = specials
    t["k_new"] = torch.from_numpy(kn).to(torch.bfloat16)
    t["v_new"] = torch.from_numpy(vn).to(torch.bfloat16)
    t["k_scale"] = torch.tensor([1.0, 0.0371], dtype=torch.float32)  # exact / inexact division
    t["v_scale"] = torch.tensor([2.0 ** -7, 0.0029], dtype=torch.float32)
    _, _, kc, vc, _ = _run_gpu(wl)
    kc_ref, vc_ref = t["k_cache"].numpy().copy(), t["v_cache"].numpy().copy()
    oracle.kv_append(wl.seq_lens, wl.page_table, wl.num_pages, host(t["k_new"]),
                     host(t["v_new"]), kc_ref, vc_ref, k_scale=t["k_scale"].numpy(),
                     v_scale=t["v_scale"].numpy())
    assert np.array_equal(kc.cpu().numpy(), kc_ref)
    assert np.array_equal(vc.cpu().numpy(), vc_ref)


def test_rollback_poison_e4m3_cache():
    rng = np.random.default_rng(5)
    B, K, Hkv, D = 20, 4, 2, 128
    lens = rng.integers(0, 300, B).astype(np.int32)
    wl = _case(B, K, 4, Hkv, D, lens, seed=11)
    acc = rng.integers(0, K + 1, B).astype(np.int32)
    i32 = dict(dtype=torch.int32, device=DEV)
    pt, sl, na = (torch.tensor(x, device=DEV) for x in (wl.page_table, lens, acc))
    slots = torch.full((B * (K + 1),), -9, **i32)
    soff = torch.empty(B + 1, **i32)
    freed = torch.full((B * 2,), -9, **i32)
    foff = torch.empty(B + 1, **i32)
    err = torch.zeros(1, **i32)
    kc, vc = wl.tensors["k_cache"].to(DEV), wl.tensors["v_cache"].to(DEV)
    d = sdv.rollback_desc(page_table=pt, num_accepted=na, seq_lens=sl, K=K, rollback_slots=slots,
                          rollback_offsets=soff, freed_pages=freed, freed_offsets=foff,
                          poison=True, k_cache=kc, v_cache=vc, n_kv_heads=Hkv, d_k=D, d_v=D,
                          num_pages=wl.num_pages, dev_error=err)
    assert d.dtype == sdv.SD_E4M3
    sdv.kv_rollback(d)
    torch.cuda.synchronize()
    kch, vch = wl.tensors["k_cache"].numpy().copy(), wl.tensors["v_cache"].numpy().copy()
    ref = oracle.kv_rollback(wl.page_table, acc, lens, K, poison=True, k_cache=kch,
                             v_cache=vch, n_kv_heads=Hkv, d_k=D, d_v=D)
    assert int(err.item()) == 0
    assert np.array_equal(sl.cpu().numpy(), ref["seq_lens"])
    assert np.array_equal(slots.cpu().numpy(), ref["rb_slots"])
    assert np.array_equal(kc.cpu().numpy(), kch) and np.array_equal(vc.cpu().numpy(), vch)


@pytest.mark.parametrize("kv,K", [("bf16", 3), ("e4m3", 3), ("e4m3", 9)])
def test_attention_ragged_batch_with_invalid_requests(kv, K):
    """Many requests of mixed lengths (zero included), one with a bad page
    entry: the waves' equal tile ranges cut pairs at arbitrary tiles, and the
    combine must find every pair's partials (and skip the invalid request).
    K = 9 gives 40 query rows per kv head (the 16-row-block E4M3 kernel)."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, D = 37, 16, 4, 128
    lens = rng.integers(0, 3000, B)
    lens[[0, 5, 9]] = [0, 1, 2999]
    if kv == "e4m3":
        wl = _case(B, K, Hq, Hkv, D, lens, seed=32)
    else:
        cfg = sdsynth.Config(name="case", batch=B, K=K, n_q_heads=Hq, n_kv_heads=Hkv, d_qk=D,
                             d_v=D, mla=False, hidden=Hq * D, vocab=8, dtype="bf16",
                             seq_len=None)
        wl = sdsynth.make_workload(cfg, 32, device="cpu", seq_lens=lens, with_lm_head=False)
    ref, _, _ = (_oracle(wl) if kv == "e4m3" else _oracle_bf16(wl))
    bad = 11
    wl.page_table[bad, 0] = wl.num_pages + 3
    if kv == "e4m3":
        out, _, _, _, err = _run_gpu(wl)
    else:
        out, err = _run_gpu_bf16(wl)
    o = out.cpu().numpy()
    assert err & sdv.SD_DERR_PAGE
    assert np.isnan(o[bad]).all()
    keep = np.arange(B) != bad
    check_attention(o[keep], ref[keep], where=f"ragged batch {kv} K={K}")


def _oracle_bf16(wl):
    t = wl.tensors
    kc, vc = host(t["k_cache"]).copy(), host(t["v_cache"]).copy()
    oracle.kv_append(wl.seq_lens, wl.page_table, wl.num_pages, host(t["k_new"]),
                     host(t["v_new"]), kc, vc)
    ref = oracle.verify_attn(host(t["q"]), kc, vc, wl.page_table, wl.seq_lens, wl.num_pages,
                             n_kv_heads=wl.cfg.n_kv_heads, d_v=wl.cfg.d_v)
    return ref, kc, vc


def _run_gpu_bf16(wl):
    t = wl.tensors
    q, kc, vc = t["q"].to(DEV), t["k_cache"].to(DEV), t["v_cache"].to(DEV)
    pt = torch.tensor(wl.page_table, device=DEV)
    sl = torch.tensor(wl.seq_lens, device=DEV)
    B, Q, Hq, D = q.shape
    out = torch.full((B, Q, Hq, D), -5.0, dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    d = sdv.attn_desc(q=q, k_cache=kc, v_cache=vc, page_table=pt, seq_lens=sl, out=out,
                      n_kv_heads=wl.cfg.n_kv_heads, num_pages=wl.num_pages,
                      max_seq_len=int(wl.seq_lens.max()), k_new=t["k_new"].to(DEV),
                      v_new=t["v_new"].to(DEV), dev_error=err)
    sdv.verify_attn(d)
    torch.cuda.synchronize()
    return out, int(err.item())


@pytest.mark.parametrize("seed", [0, 1, 4, 5, 6, 8])   # seeds with distinct (G, K)
def test_attention_e4m3_random_16row_shapes(seed):
    """Seeded random shapes with 33..48 query rows per kv head (the 16-row-
    block kernel): group size, draft count, kv heads and ragged lengths
    (zero, page edges and a long request) drawn per seed; every row against
    the oracle, the appended cache bytes bit-exact."""
    rng = np.random.default_rng(900 + seed)
    while True:
        G = int(rng.integers(2, 13))
        K = int(rng.integers(0, 24))
        if 32 < G * (K + 1) <= 48:
            break
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.integers(2, 7))
    lens = rng.integers(0, 1500, B)
    lens[0] = int(rng.choice([0, 63, 64, 65]))
    lens[-1] = int(rng.integers(3000, 6000))
    wl = _case(B, K, G * Hkv, Hkv, 128, lens, seed=910 + seed)
    out, _, kc, vc, err = _run_gpu(wl)
    ref, kc_ref, vc_ref = _oracle(wl)
    assert err == 0
    check_attention(out.cpu().numpy(), ref,
                    where=f"e4m3 16-row seed {seed}: G={G} K={K} Hkv={Hkv} lens={list(lens)}")
    assert np.array_equal(kc.cpu().numpy(), kc_ref) and np.array_equal(vc.cpu().numpy(), vc_ref)

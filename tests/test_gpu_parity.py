"""GPU parity of each C-ABI call against the fp64 oracle, on seeded synthetic
inputs small enough for the oracle to finish in seconds while spanning
several tiles, key chunks and ragged tails.  Tolerances: see tests/parity.py."""
import numpy as np
import pytest
import torch

import oracle
import sdsynth
import speculative_decoding_sd_amd as sdv
from parity import (DEV, bits, host, check_attention, check_logits_bf16, check_logits_f32,
                    compare_accept, run_accept)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def _gqa_case(B, K, Hq, Hkv, D, seq_lens, dtype, seed, extra=0):
    cfg = sdsynth.Config(name="case", batch=B, K=K, n_q_heads=Hq, n_kv_heads=Hkv, d_qk=D,
                         d_v=D, mla=False, hidden=Hq * D, vocab=8, dtype=dtype, seq_len=None)
    return sdsynth.make_workload(cfg, seed, device="cpu", seq_lens=np.array(seq_lens),
                                 extra_tokens=extra, with_lm_head=False)


def _run_gpu_attention(wl, max_seq_len=None, append=True, lowp=True):
    t = wl.tensors
    cfg = wl.cfg
    q, kc, vc = t["q"].to(DEV), t["k_cache"].to(DEV), t["v_cache"].to(DEV)
    kn = t["k_new"].to(DEV) if append else None
    vn = t["v_new"].to(DEV) if append else None
    pt = torch.tensor(wl.page_table, device=DEV)
    sl = torch.tensor(wl.seq_lens, device=DEV)
    B, Q, Hq, D = q.shape
    out = torch.full((B, Q, Hq, cfg.d_v), -5.0, dtype=torch.float32, device=DEV)
    out_lowp = torch.empty((B * Q, Hq * cfg.d_v), dtype=q.dtype, device=DEV) if lowp else None
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    d = sdv.attn_desc(q=q, k_cache=kc, v_cache=vc, page_table=pt, seq_lens=sl, out=out,
                      n_kv_heads=cfg.n_kv_heads, num_pages=wl.num_pages,
                      max_seq_len=int(max_seq_len or wl.seq_lens.max()), k_new=kn, v_new=vn,
                      out_lowp=out_lowp, dev_error=err)
    sdv.verify_attn(d)
    # The error word through the C ABI's own query (it waits for the stream).
    word = sdv.device_error(err)
    torch.cuda.synchronize()
    assert word == int(err.item())
    return out, out_lowp, kc, vc, word


def _oracle_attention(wl, sel=None, append=True):
    t = wl.tensors
    kc, vc = host(t["k_cache"]).copy(), host(t["v_cache"]).copy()
    if append:
        oracle.kv_append(wl.seq_lens, wl.page_table, wl.num_pages, host(t["k_new"]),
                         host(t["v_new"]), kc, vc)
    ref = oracle.verify_attn(host(t["q"]), kc, vc, wl.page_table, wl.seq_lens, wl.num_pages,
                             n_kv_heads=wl.cfg.n_kv_heads, d_v=wl.cfg.d_v, sel=sel)
    return ref, kc, vc


@pytest.mark.parametrize("B,K,Hq,Hkv,D,lens", [
    (3, 5, 16, 4, 128, [0, 61, 1300]),      # 24 rows/kv head; L=0; page-straddling append
    (2, 7, 10, 2, 64, [5, 700]),            # 40 rows/kv head (two row blocks), head dim 64
    (2, 7, 40, 8, 128, [3000, 1000]),       # long-context head layout, two row blocks
    (4, 4, 32, 8, 128, [512, 4097, 777, 64]),  # serving head layout, ragged
    (1, 0, 4, 1, 64, [33]),                 # K = 0: plain single-token decode
    (2, 7, 16, 2, 128, [100, 2000]),        # 64 rows per kv head: the largest supported
])
def test_attention_gqa_bf16(B, K, Hq, Hkv, D, lens):
    wl = _gqa_case(B, K, Hq, Hkv, D, lens, "bf16", seed=10 + B + K)
    out, lowp, kc, vc, err = _run_gpu_attention(wl)
    ref, kc_ref, vc_ref = _oracle_attention(wl)
    assert err == 0
    check_attention(out.cpu().numpy(), ref, where=f"gqa {B},{K},{Hq},{Hkv},{D}")
    assert np.array_equal(bits(kc), kc_ref) and np.array_equal(bits(vc), vc_ref)
    # out_lowp is the fp32 output rounded to nearest even.
    exp_lowp = oracle.round_bf16(out.cpu().numpy().astype(np.float64)).reshape(B * (K + 1), -1)
    assert np.array_equal(bits(lowp), exp_lowp)


def test_attention_gqa_bf16_long_chunks():
    """Enough (request, kv head) pairs that the key axis is cut into 1024-key
    chunks (eight tiles per wave, prefetch path); sampled rows."""
    B, K, Hq, Hkv, D = 8, 7, 40, 8, 128
    lens = [40000, 39001, 36000, 38111, 40031, 35555, 39999, 37000]
    wl = _gqa_case(B, K, Hq, Hkv, D, lens, "bf16", seed=77)
    out, _, _, _, err = _run_gpu_attention(wl)
    rng = np.random.default_rng(0)
    sel = np.stack([rng.integers(0, B, 48), rng.integers(0, K + 1, 48), rng.integers(0, Hq, 48)], 1)
    ref, _, _ = _oracle_attention(wl, sel=sel)
    o = out.cpu().numpy()
    got = np.stack([o[b, i, h] for b, i, h in sel])
    assert err == 0
    check_attention(got, ref, where="long chunks")


def test_attention_f32_tiny_config():
    """The tiny fp32 configuration at full size: B=1, K=3, 4 heads x 64, L=128."""
    cfg = sdsynth.CONFIGS[1]
    wl = sdsynth.make_workload(cfg, sdsynth.config_seed(1), device="cpu", with_lm_head=False)
    out, lowp, kc, vc, err = _run_gpu_attention(wl)
    ref, kc_ref, vc_ref = _oracle_attention(wl)
    assert err == 0
    rel = check_attention(out.cpu().numpy(), ref, where="f32")
    assert rel < 1e-5
    assert np.array_equal(kc.cpu().numpy(), kc_ref)
    assert np.array_equal(lowp.cpu().numpy().reshape(out.shape), out.cpu().numpy())


@pytest.mark.parametrize("B,K,Hq,Hkv,D,lens", [
    (2, 3, 4, 2, 128, [300, 700]),   # several 256-key tiles, later tiles' page entries
    (3, 2, 2, 1, 256, [0, 255, 513]),  # widest head dim (4 threads per value row), tile edges
    (2, 4, 8, 4, 16, [40, 260]),     # 64 key groups of the value pass
    (2, 1, 2, 2, 4, [3, 290]),       # head dim 4: one thread per value row, 256 groups
])
def test_attention_f32_shapes(B, K, Hq, Hkv, D, lens):
    """The float32 path at head dims 4..256 (rows of whole 16-byte units) and
    lengths spanning several 256-key tiles."""
    wl = _gqa_case(B, K, Hq, Hkv, D, lens, "f32", seed=70 + D)
    out, lowp, kc, vc, err = _run_gpu_attention(wl)
    ref, kc_ref, vc_ref = _oracle_attention(wl)
    assert err == 0
    rel = check_attention(out.cpu().numpy(), ref, where=f"f32 D={D}")
    assert rel < 1e-5
    assert np.array_equal(kc.cpu().numpy(), kc_ref) and np.array_equal(vc.cpu().numpy(), vc_ref)


def test_attention_preappended_cache():
    """k_new = NULL: the cache already holds the step's positions."""
    wl = _gqa_case(2, 3, 8, 2, 128, [100, 300], "bf16", seed=5)
    ref, kc_ref, vc_ref = _oracle_attention(wl)
    t = wl.tensors
    t["k_cache"] = torch.from_numpy(kc_ref.view(np.int16)).view(torch.bfloat16)
    t["v_cache"] = torch.from_numpy(vc_ref.view(np.int16)).view(torch.bfloat16)
    out, _, _, _, err = _run_gpu_attention(wl, append=False)
    assert err == 0
    check_attention(out.cpu().numpy(), ref, where="pre-appended")


def test_attention_device_errors_flag_and_nan():
    """A request over capacity and one with a bad page entry are flagged and
    get NaN rows; the others are untouched by the fault."""
    wl = _gqa_case(3, 3, 8, 2, 64, [10, 20, 30], "bf16", seed=6)
    orig = int(wl.page_table[2, 0])
    wl.page_table[2, 0] = wl.num_pages + 5          # bad page for request 2
    wl.seq_lens[1] = 10 ** 6                         # over capacity for request 1
    out, _, _, _, err = _run_gpu_attention(wl, max_seq_len=40)
    o = out.cpu().numpy()
    assert err & sdv.SD_DERR_PAGE and err & sdv.SD_DERR_CAPACITY
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all()
    wl.seq_lens[1] = 20
    wl.page_table[2, 0] = orig
    ref, _, _ = _oracle_attention(wl, sel=np.array([[0, i, h] for i in range(4) for h in range(8)]))
    check_attention(o[0].reshape(-1, 64), ref, where="valid request beside faulty ones")


# ---------------------------------------------------------------------------
# LM head
# ---------------------------------------------------------------------------
# (260, 640, 40001) and (300, 384, 40000) have at least 256 tiles of 256 x 256,
# so they take the five-slot ring kernel (ragged rows and vocabulary, odd and
# multiple-of-4 vocabulary for both epilogue paths, 10 and 6 k-slices so the
# slot rotation wraps and the tail re-reads run).  hidden = 128 gives two
# k-slices, fewer than any ring holds: (100, 128, 3000) and (40, 128, 5000)
# take the three- and four-stage streaming kernels, (260, 128, 40001) the
# five-slot ring, all with clamped prologue refills.  (150, 256, 3001) and
# (190, 128, 2003) take the 128 x 192 streaming tiles (more than 128 rows,
# fewer 256 x 256 tiles than CUs), with ragged rows and vocabulary and four or
# two k-slices for its four stages.
@pytest.mark.parametrize("M,hidden,V", [(130, 200, 333), (64, 512, 1000), (256, 7168, 640),
                                        (260, 640, 40001), (100, 128, 3000), (40, 128, 5000),
                                        (260, 128, 40001), (150, 256, 3001), (190, 128, 2003)])
def test_lm_head_exact_small_integers(M, hidden, V):
    """Small-integer bf16 operands: every fp32 partial sum is exact, so the
    bf16 logits must equal the oracle's exact values rounded to nearest even
    (pins indexing, tails and the epilogue bit for bit)."""
    rng = np.random.default_rng(M + V)
    H = torch.tensor(rng.integers(-3, 4, (M, hidden)), dtype=torch.bfloat16)
    W = torch.tensor(rng.integers(-3, 4, (V, hidden)), dtype=torch.bfloat16)
    logits = torch.empty((M, V), dtype=torch.bfloat16, device=DEV)
    sdv.lm_head(H.to(DEV), W.to(DEV), logits)
    torch.cuda.synchronize()
    exact = oracle.lm_head(bits(H), bits(W))
    assert np.array_equal(bits(logits), oracle.round_bf16(exact))


@pytest.mark.parametrize("M,hidden,V", [(192, 1024, 1500), (64, 5120, 1111), (300, 512, 700),
                                        (300, 384, 40000)])
def test_lm_head_bf16_random(M, hidden, V):
    H = sdsynth.normal((M, hidden), 1.0, 3, "H", torch.bfloat16, "cpu")
    W = sdsynth.normal((V, hidden), 0.02, 3, "W", torch.bfloat16, "cpu")
    logits = torch.empty((M, V), dtype=torch.bfloat16, device=DEV)
    sdv.lm_head(H.to(DEV), W.to(DEV), logits)
    torch.cuda.synchronize()
    exact = oracle.lm_head(bits(H), bits(W))
    check_logits_bf16(bits(logits), exact, where=f"lm_head {M}x{hidden}x{V}")


def test_lm_head_f32():
    H = sdsynth.normal((4, 256), 1.0, 4, "H", torch.float32, "cpu")
    W = sdsynth.normal((1024, 256), 0.02, 4, "W", torch.float32, "cpu")
    logits = torch.empty((4, 1024), dtype=torch.float32, device=DEV)
    sdv.lm_head(H.to(DEV), W.to(DEV), logits)
    torch.cuda.synchronize()
    check_logits_f32(logits.cpu().numpy(), oracle.lm_head(H.numpy(), W.numpy()))


# ---------------------------------------------------------------------------
# Acceptance (both sides receive the same generated logits)
# ---------------------------------------------------------------------------
def _logits(B, Q, V, dtype, seed, sigma=1.7):
    return sdsynth.normal((B, Q, V), sigma, seed, "H", dtype, "cpu")


def _greedy_inputs(lg, K, seed):
    B, Q, V = lg.shape
    tt, _ = oracle.argmax(host(lg))
    drafts = sdsynth.greedy_drafts(tt, K, V, seed)
    return drafts


@pytest.mark.parametrize("B,K,V,dtype", [(40, 4, 5000, "bf16"), (33, 3, 5003, "bf16"),
                                         (17, 5, 1024, "f32"), (9, 0, 700, "bf16")])
def test_accept_greedy(B, K, V, dtype):
    lg = _logits(B, K + 1, V, sdsynth.torch_dtype(dtype), seed=B + V)
    if dtype == "bf16":
        lg[0, 0, 10:20] = lg[0, 0].max()              # a tie at the maximum
    drafts = _greedy_inputs(lg, K, seed=B)
    temp = np.zeros(B, np.float32)
    ua = sdsynth.philox_uniforms(B, B, K + 1, 0)
    us = sdsynth.philox_uniforms(B, B, K + 1, 1)
    ref = oracle.accept(host(lg), drafts, temp, None, None, ua, us)
    gpu = run_accept(lg.to(DEV), torch.tensor(drafts, device=DEV), torch.tensor(temp, device=DEV),
                     None, None, torch.tensor(ua, device=DEV), torch.tensor(us, device=DEV))
    assert compare_accept(gpu, ref, allow_excluded=False, where="greedy") == 0
    assert gpu["dev_error"] == 0
    assert K == 0 or (ref["num_accepted"] > 0).any()


@pytest.mark.parametrize("B,K,V,T,top_p,dtype", [
    (64, 5, 3000, 1.0, None, "bf16"),
    (64, 7, 4096, 0.7, 0.95, "bf16"),
    (48, 4, 2500, 0.8, 0.5, "bf16"),
    (24, 3, 777, 1.3, 0.9, "f32"),
    (16, 0, 1000, 0.9, 0.8, "bf16"),
    (3, 2, 262144, 1.0, None, "bf16"),      # the largest supported vocab
])
def test_accept_stochastic(B, K, V, T, top_p, dtype):
    seed = 100 + B + K
    lg = _logits(B, K + 1, V, sdsynth.torch_dtype(dtype), seed=seed)
    lgh = host(lg)
    lf = oracle.bf16_to_f64(lgh) if dtype == "bf16" else lgh.astype(np.float64)
    pd = sdsynth.draft_probs(lf[:, :K], seed, 0.5, T, top_p or 1.0)
    drafts = sdsynth.sample_drafts(pd, seed) if K else np.zeros((B, 0), np.int32)
    temp = np.full(B, T, np.float32)
    tp = None if top_p is None else np.full(B, top_p, np.float32)
    ua = sdsynth.philox_uniforms(seed, B, K + 1, 0)
    us = sdsynth.philox_uniforms(seed, B, K + 1, 1)
    ref = oracle.accept(lgh, drafts, temp, tp, pd, ua, us)
    gpu = run_accept(lg.to(DEV), torch.tensor(drafts, device=DEV), torch.tensor(temp, device=DEV),
                     None if tp is None else torch.tensor(tp, device=DEV),
                     torch.tensor(pd, device=DEV), torch.tensor(ua, device=DEV),
                     torch.tensor(us, device=DEV))
    n_excl = compare_accept(gpu, ref, where=f"stochastic T={T} top_p={top_p}")
    assert n_excl <= B // 8
    assert gpu["dev_error"] == 0


@pytest.mark.parametrize("B,K,V,dtype", [(60, 4, 5000, "bf16"), (30, 3, 1031, "f32"),
                                         (12, 5, 129280, "bf16")])
def test_accept_relaxed(B, K, V, dtype):
    """Relaxed greedy acceptance next to strict greedy and sampled requests,
    plus a negative top-N and a NaN delta (both invalid).  Rows carry five
    boosted tokens so that the top-N / delta filter keeps some of them and
    drops others; drafts are mostly boosted tokens of the judging row."""
    rng = np.random.default_rng(B + V)
    Q = K + 1
    lgf = rng.normal(0.0, 1.0, (B, Q, V))
    boosted = np.stack([[rng.choice(V, 5, replace=False) for _ in range(Q)] for _ in range(B)])
    for t, add in enumerate([8.0, 7.6, 7.2, 6.8, 6.0]):
        np.put_along_axis(lgf, boosted[:, :, t:t + 1],
                          np.take_along_axis(lgf, boosted[:, :, t:t + 1], -1) + add, -1)
    lg = torch.tensor(lgf, dtype=torch.float32).to(sdsynth.torch_dtype(dtype))
    lgh = host(lg)
    drafts = np.where(rng.random((B, K)) < 0.75,
                      boosted[:, :K, :][np.arange(B)[:, None], np.arange(K)[None, :],
                                        rng.integers(0, 5, (B, K))],
                      rng.integers(0, V, (B, K))).astype(np.int32)
    modes = [(0, 0.0), (1, 0.3), (3, 0.1), (3, 0.3), (10, 0.6), (2, 0.05), (4, 0.2)]
    rk = np.array([modes[b % len(modes)][0] for b in range(B)], np.int32)
    rd = np.array([modes[b % len(modes)][1] for b in range(B)], np.float32)
    temp = np.zeros(B, np.float32)
    temp[5::8] = 0.8                      # sampled requests ignore the relaxed fields
    rk[3] = -1                            # invalid: negative top-N
    rd[4] = np.nan                        # invalid when that request is relaxed
    rk[4] = 3
    temp[3] = temp[4] = 0.0
    if K > 1:
        drafts[6, 1] = -1                 # a negative draft ends the chain
    lf = oracle.bf16_to_f64(lgh) if dtype == "bf16" else lgh.astype(np.float64)
    pd = sdsynth.draft_probs(lf[:, :K], B, 0.5, 0.8)
    ua = sdsynth.philox_uniforms(B, B, Q, 0)
    us = sdsynth.philox_uniforms(B, B, Q, 1)
    ref = oracle.accept(lgh, drafts, temp, None, pd, ua, us, relaxed_topk=rk, relaxed_delta=rd)
    gpu = run_accept(lg.to(DEV), torch.tensor(drafts, device=DEV), torch.tensor(temp, device=DEV),
                     None, torch.tensor(pd, device=DEV), torch.tensor(ua, device=DEV),
                     torch.tensor(us, device=DEV), torch.tensor(rk, device=DEV),
                     torch.tensor(rd, device=DEV))
    assert ref["n_invalid"] == 2
    n_excl = compare_accept(gpu, ref, where=f"relaxed {dtype} V={V}")
    assert n_excl <= B // 8
    assert list(gpu["num_accepted"][[3, 4]]) == [-1, -1]
    assert gpu["dev_error"] & sdv.SD_DERR_PARAM
    relaxed = (rk > 0) & (temp == 0)
    strict = oracle.accept(lgh, drafts, temp, None, pd, ua, us)
    ok = ref["num_accepted"] >= 0
    # The relaxed rule accepts at least as much as the strict one, and more here.
    assert (ref["num_accepted"][relaxed & ok] >= strict["num_accepted"][relaxed & ok]).all()
    assert ref["num_accepted"][relaxed & ok].sum() > strict["num_accepted"][relaxed & ok].sum()


def test_accept_mixed_modes_and_invalid_requests():
    """Serving-style batch: even requests greedy, odd sampled at T=0.8, plus a
    NaN row, an out-of-range draft and a negative temperature."""
    B, K, V = 32, 4, 2048
    lg = _logits(B, K + 1, V, torch.bfloat16, seed=9)
    lgh = host(lg)
    lf = oracle.bf16_to_f64(lgh)
    temp = np.where(np.arange(B) % 2 == 1, 0.8, 0.0).astype(np.float32)
    pd = sdsynth.draft_probs(lf[:, :K], 9, 0.5, 0.8)
    d_st = sdsynth.sample_drafts(pd, 9)
    d_gr = _greedy_inputs(lg, K, seed=9)
    drafts = np.where((np.arange(B) % 2 == 1)[:, None], d_st, d_gr).astype(np.int32)
    lgh = lgh.copy()
    lgh[4, 2, 7] = 0x7FC0       # NaN in request 4
    drafts[6, 1] = V + 3        # out-of-range draft in request 6
    temp[8] = -1.0              # bad temperature in request 8
    lg = torch.from_numpy(lgh.view(np.int16)).view(torch.bfloat16)
    ua = sdsynth.philox_uniforms(9, B, K + 1, 0)
    us = sdsynth.philox_uniforms(9, B, K + 1, 1)
    ref = oracle.accept(lgh, drafts, temp, None, pd, ua, us)
    gpu = run_accept(lg.to(DEV), torch.tensor(drafts, device=DEV), torch.tensor(temp, device=DEV),
                     None, torch.tensor(pd, device=DEV), torch.tensor(ua, device=DEV),
                     torch.tensor(us, device=DEV))
    assert ref["n_invalid"] == 3
    compare_accept(gpu, ref, where="mixed")
    assert list(gpu["num_accepted"][[4, 6, 8]]) == [-1, -1, -1]
    e = gpu["dev_error"]
    assert e & sdv.SD_DERR_NONFINITE and e & sdv.SD_DERR_TOKEN and e & sdv.SD_DERR_PARAM


@pytest.mark.parametrize("seed", range(6))
def test_accept_random_mixed_batches(seed):
    """Randomised batches that mix, request by request, greedy rows, sampled
    rows with and without a nucleus (temperatures 0.5-1.5), drafts that end
    early (-1), and draft distributions of three kinds: a noisy softmax, one
    equal to p_t within a few 1e-6 on most tokens (the residual's near-ties),
    and a one-hot.  K from 0 to 7, vocabularies from 999 to 32000, bf16 and
    float32 logits.  Compared with the oracle under its exclusion windows."""
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 41))
    K = int(rng.integers(0, 8))
    V = int(rng.choice([999, 4096, 5003, 32000]))
    dtype = "f32" if seed % 3 == 2 else "bf16"
    Q = K + 1
    lg = _logits(B, Q, V, sdsynth.torch_dtype(dtype), seed=600 + seed)
    lgh = host(lg)
    lf = oracle.bf16_to_f64(lgh) if dtype == "bf16" else lgh.astype(np.float64)
    temp = np.where(rng.random(B) < 0.3, 0.0, rng.uniform(0.5, 1.5, B)).astype(np.float32)
    top_p = np.where(rng.random(B) < 0.5, 1.0, rng.choice([0.5, 0.9, 0.97], B)).astype(np.float32)
    pd = np.zeros((B, K, V), np.float32)
    drafts = np.full((B, K), -1, np.int32)
    tt, _ = oracle.argmax(lgh)
    for b in range(B):
        T = float(temp[b]) if temp[b] > 0 else 1.0
        for n in range(K):
            kind = int(rng.integers(3))
            if kind == 0:
                x = lf[b, n] / T + rng.normal(0, 0.5, V)
                q = np.exp(x - x.max())
            elif kind == 1:
                x = lf[b, n] / T
                q = np.exp(x - x.max()) * (1.0 + rng.choice([-4e-6, 3e-6, 2e-3], V))
            else:
                q = np.zeros(V)
                q[int(rng.integers(V))] = 1.0
            pd[b, n] = (q / q.sum()).astype(np.float32)
        if temp[b] == 0:
            drafts[b] = sdsynth.greedy_drafts(tt[b:b + 1], K, V, seed + b)[0] if K else drafts[b]
        elif K:
            drafts[b] = sdsynth.sample_drafts(pd[b:b + 1], seed + b)[0]
        if K and rng.random() < 0.15:
            drafts[b, int(rng.integers(K)):] = -1
    ua = sdsynth.philox_uniforms(700 + seed, B, Q, 0)
    us = sdsynth.philox_uniforms(700 + seed, B, Q, 1)
    ref = oracle.accept(lgh, drafts, temp, top_p, pd, ua, us)
    t = lambda x: torch.tensor(x, device=DEV)
    gpu = run_accept(lg.to(DEV), t(drafts), t(temp), t(top_p), t(pd), t(ua), t(us))
    assert gpu["dev_error"] == 0
    print(f"seed {seed}: B={B} K={K} V={V} {dtype}", flush=True)
    n_excl = compare_accept(gpu, ref, where=f"random batch seed {seed}")
    assert n_excl <= max(1, B // 8), n_excl


def test_accept_chains_longer_than_a_wave():
    """K = 70 drafts: the decision takes a wave's 64 lanes and then the next
    64 (greedy chains that match past lane 63, sampled chains with a -1 past
    it), against the oracle."""
    B, K, V = 6, 70, 1000
    Q = K + 1
    lg = _logits(B, Q, V, torch.bfloat16, seed=77)
    lgh = host(lg)
    lf = oracle.bf16_to_f64(lgh)
    tt, _ = oracle.argmax(lgh)
    temp = np.array([0, 0, 0, 1.0, 0.8, 1.2], np.float32)
    pd = sdsynth.draft_probs(lf[:, :K], 77, 0.05, 1.0)
    drafts = sdsynth.sample_drafts(pd, 77)
    drafts[0] = tt[0, :K]                   # greedy: all 70 accepted
    drafts[1] = tt[1, :K]
    drafts[1, 66] = (tt[1, 66] + 1) % V     # greedy: the mismatch in the second 64
    drafts[2] = tt[2, :K]
    drafts[2, 65:] = -1                     # greedy: the chain ends in the second 64
    drafts[4, 68:] = -1                     # sampled: ends in the second 64
    ua = np.full((B, Q), 1e-6, np.float32)  # sampled drafts accepted unless p_t is tiny
    us = sdsynth.philox_uniforms(77, B, Q, 1)
    ref = oracle.accept(lgh, drafts, temp, None, pd, ua, us)
    t = lambda x: torch.tensor(x, device=DEV)
    gpu = run_accept(lg.to(DEV), t(drafts), t(temp), None, t(pd), t(ua), t(us))
    assert gpu["dev_error"] == 0
    compare_accept(gpu, ref, where="K = 70")
    assert list(ref["num_accepted"][:3]) == [70, 66, 65]
    assert ref["num_accepted"][3:].max() > 63


def test_accept_is_deterministic():
    B, K, V = 16, 5, 4096
    lg = _logits(B, K + 1, V, torch.bfloat16, seed=21)
    lf = oracle.bf16_to_f64(host(lg))
    pd = sdsynth.draft_probs(lf[:, :K], 21, 0.5, 0.7, 0.9)
    drafts = sdsynth.sample_drafts(pd, 21)
    args = (lg.to(DEV), torch.tensor(drafts, device=DEV),
            torch.full((B,), 0.7, device=DEV), torch.full((B,), 0.9, device=DEV),
            torch.tensor(pd, device=DEV),
            torch.tensor(sdsynth.philox_uniforms(21, B, K + 1, 0), device=DEV),
            torch.tensor(sdsynth.philox_uniforms(21, B, K + 1, 1), device=DEV))
    a = run_accept(*args)
    b = run_accept(*args)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


# ---------------------------------------------------------------------------
# Rollback
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K,poison", [(4, False), (7, True), (0, False)])
def test_rollback(K, poison):
    rng = np.random.default_rng(K)
    B, Hkv, D = 50, 2, 64
    lens = rng.integers(0, 300, B).astype(np.int32)
    lens[:4] = [63 - K, 64, 127, 0]
    wl = _gqa_case(B, K, 4, Hkv, D, lens, "bf16", seed=K, extra=0)
    acc = rng.integers(-1, K + 1, B).astype(np.int32)
    acc[5] = K + 3                                   # invalid count
    pt = torch.tensor(wl.page_table, device=DEV)
    sl = torch.tensor(lens, device=DEV)
    na = torch.tensor(acc, device=DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    slots = torch.full((B * (K + 1),), -9, **i32)
    soff = torch.empty(B + 1, **i32)
    freed = torch.full((B * (K // 64 + 2),), -9, **i32)
    foff = torch.empty(B + 1, **i32)
    err = torch.zeros(1, **i32)
    kc, vc = wl.tensors["k_cache"].to(DEV), wl.tensors["v_cache"].to(DEV)
    d = sdv.rollback_desc(page_table=pt, num_accepted=na, seq_lens=sl, K=K, rollback_slots=slots,
                          rollback_offsets=soff, freed_pages=freed, freed_offsets=foff,
                          poison=poison, k_cache=kc, v_cache=vc, n_kv_heads=Hkv, d_k=D, d_v=D,
                          num_pages=wl.num_pages, dev_error=err)
    sdv.kv_rollback(d)
    torch.cuda.synchronize()
    kch, vch = host(wl.tensors["k_cache"]).copy(), host(wl.tensors["v_cache"]).copy()
    ref = oracle.kv_rollback(wl.page_table, acc, lens, K, poison=poison, k_cache=kch,
                             v_cache=vch, n_kv_heads=Hkv, d_k=D, d_v=D)
    assert np.array_equal(sl.cpu().numpy(), ref["seq_lens"])
    assert np.array_equal(soff.cpu().numpy(), ref["rb_offsets"])
    assert np.array_equal(slots.cpu().numpy(), ref["rb_slots"])
    assert np.array_equal(foff.cpu().numpy(), ref["freed_offsets"])
    assert np.array_equal(freed.cpu().numpy(), ref["freed"])
    assert int(err.item()) == sdv.SD_DERR_ACCEPT_COUNT
    if poison:
        assert np.array_equal(bits(kc), kch) and np.array_equal(bits(vc), vch)


# ---------------------------------------------------------------------------
# Whole step on the tiny fp32 configuration
# ---------------------------------------------------------------------------
def test_chained_tiny_fp32_step():
    cfg = sdsynth.CONFIGS[1]
    seed = sdsynth.config_seed(1)
    wl = sdsynth.make_workload(cfg, seed, device="cpu")
    t = wl.tensors
    # Oracle chain: append + attention -> logits = o_flat W^T -> greedy accept -> rollback.
    ref_o, kc_ref, vc_ref = _oracle_attention(wl)
    Hrows = ref_o.reshape(cfg.batch * cfg.num_q, -1)
    exact = oracle.lm_head(Hrows, t["W"].numpy().astype(np.float64))
    ref_logits = exact.reshape(cfg.batch, cfg.num_q, cfg.vocab)
    tt, margin = oracle.argmax(ref_logits)
    drafts = sdsynth.greedy_drafts(tt, cfg.K, cfg.vocab, seed)
    ref_acc = oracle.accept(ref_logits, drafts, wl.temperature, None, None, wl.u_accept,
                            wl.u_sample)
    ref_rb = oracle.kv_rollback(wl.page_table, ref_acc["num_accepted"], wl.seq_lens, cfg.K)
    # GPU chain through VerifyStep (H = attention output).
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in t.items()}
    sl = torch.tensor(wl.seq_lens, device=DEV)
    step = sdv.VerifyStep(q=d["q"], k_cache=d["k_cache"], v_cache=d["v_cache"],
                          page_table=torch.tensor(wl.page_table, device=DEV), seq_lens=sl,
                          num_pages=wl.num_pages, max_seq_len=int(wl.seq_lens.max()),
                          n_kv_heads=cfg.n_kv_heads, W=d["W"],
                          drafts=torch.tensor(drafts, device=DEV),
                          temperature=torch.tensor(wl.temperature, device=DEV),
                          u_accept=torch.tensor(wl.u_accept, device=DEV),
                          u_sample=torch.tensor(wl.u_sample, device=DEV),
                          k_new=d["k_new"], v_new=d["v_new"])
    step.run()
    torch.cuda.synchronize()
    check_attention(step.out.cpu().numpy(), ref_o, where="chain attention")
    check_logits_f32(step.logits.cpu().numpy(), ref_logits, where="chain logits")
    keep = margin.reshape(-1).min() >= 1e-3
    if keep:
        assert step.num_accepted.cpu().numpy().tolist() == ref_acc["num_accepted"].tolist()
        assert np.array_equal(step.out_tokens.cpu().numpy(), ref_acc["out_tokens"])
        assert np.array_equal(sl.cpu().numpy(), ref_rb["seq_lens"])
        assert np.array_equal(step.rb_slots.cpu().numpy()[: ref_rb["rb_offsets"][-1]],
                              ref_rb["rb_slots"][: ref_rb["rb_offsets"][-1]])
    assert int(step.dev_error.item()) == 0


# ---------------------------------------------------------------------------
# MLA-shaped attention (latent 576 = keys, first 512 = values, one kv head)
# ---------------------------------------------------------------------------
def _mla_case(B, K, Hq, seq_lens, seed):
    cfg = sdsynth.Config(name="mla", batch=B, K=K, n_q_heads=Hq, n_kv_heads=1, d_qk=576,
                         d_v=512, mla=True, hidden=7168, vocab=8, dtype="bf16", seq_len=None)
    return sdsynth.make_workload(cfg, seed, device="cpu", seq_lens=np.array(seq_lens),
                                 with_lm_head=False)


def _run_gpu_mla(wl, max_seq_len=None):
    t = wl.tensors
    q, lat, kn = t["q"].to(DEV), t["k_cache"].to(DEV), t["k_new"].to(DEV)
    B, Q, Hq, _ = q.shape
    out = torch.full((B, Q, Hq, 512), -5.0, dtype=torch.float32, device=DEV)
    lowp = torch.empty((B * Q, Hq * 512), dtype=torch.bfloat16, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    d = sdv.attn_desc(q=q, k_cache=lat, v_cache=None, page_table=torch.tensor(wl.page_table, device=DEV),
                      seq_lens=torch.tensor(wl.seq_lens, device=DEV), out=out, n_kv_heads=1,
                      num_pages=wl.num_pages, max_seq_len=int(max_seq_len or wl.seq_lens.max()),
                      k_new=kn, mla=True, out_lowp=lowp, dev_error=err)
    sdv.verify_attn(d)
    torch.cuda.synchronize()
    return out, lowp, lat, int(err.item())


def _oracle_mla(wl, sel=None):
    t = wl.tensors
    lat = host(t["k_cache"]).copy()
    oracle.kv_append(wl.seq_lens, wl.page_table, wl.num_pages, host(t["k_new"]), None, lat,
                     None, mla=True)
    ref = oracle.verify_attn(host(t["q"]), lat, None, wl.page_table, wl.seq_lens, wl.num_pages,
                             n_kv_heads=1, d_v=512, mla=True, sel=sel)
    return ref, lat


@pytest.mark.parametrize("B,K,Hq,lens", [
    (2, 3, 32, [40, 1000]),       # one 128-row block, chunked keys, ragged
    (1, 3, 128, [300]),           # four row blocks (the MLA head count)
    (3, 1, 64, [0, 65, 2000]),    # L = 0 and a page-straddling append
])
def test_attention_mla_bf16(B, K, Hq, lens):
    wl = _mla_case(B, K, Hq, lens, seed=30 + B + Hq)
    out, lowp, lat, err = _run_gpu_mla(wl)
    ref, lat_ref = _oracle_mla(wl)
    assert err == 0
    check_attention(out.cpu().numpy(), ref, where=f"mla {B},{K},{Hq}")
    assert np.array_equal(bits(lat), lat_ref)
    exp_lowp = oracle.round_bf16(out.cpu().numpy().astype(np.float64)).reshape(B * (K + 1), -1)
    assert np.array_equal(bits(lowp), exp_lowp)


def test_attention_mla_invalid_request_gets_nan():
    """A request over capacity in the MLA path (one key chunk, so no combine
    pass) is flagged and gets NaN rows; its neighbour is unaffected."""
    wl = _mla_case(2, 3, 32, [40, 50], seed=77)
    wl.seq_lens[1] = 10 ** 6
    out, lowp, _, err = _run_gpu_mla(wl, max_seq_len=60)
    o = out.cpu().numpy()
    assert err & sdv.SD_DERR_CAPACITY
    assert np.isnan(o[1]).all()
    assert np.isnan(lowp.float().cpu().numpy().reshape(2, 4, -1)[1]).all()
    wl.seq_lens[1] = 50
    ref, _ = _oracle_mla(wl, sel=np.array([[0, i, h] for i in range(4) for h in range(32)]))
    check_attention(o[0].reshape(-1, 512), ref, where="valid MLA request beside a faulty one")


def test_attention_mla_full_config_sampled():
    """The MLA-shaped greedy configuration at full size (B=64, K=3, 128 heads,
    L=8192): every output of 8 requests' sampled rows against the oracle."""
    cfg = sdsynth.CONFIGS[3]
    wl = sdsynth.make_workload(cfg, sdsynth.config_seed(3), device=DEV, with_lm_head=False)
    out, _, _, err = _run_gpu_mla(wl)
    assert err == 0
    rng = np.random.default_rng(3)
    bs = rng.choice(cfg.batch, 2, replace=False)
    sel = np.stack([np.repeat(bs, 8), np.tile(rng.integers(0, cfg.num_q, 8), 2),
                    np.tile(rng.integers(0, cfg.n_q_heads, 8), 2)], 1)
    # Host copies of just the sampled requests' pages (renumbered).
    t = wl.tensors
    pt = wl.page_table[bs]
    used = np.unique(pt[pt >= 0])
    remap = {int(p): i for i, p in enumerate(used)}
    new_pt = np.vectorize(lambda x: remap.get(int(x), -1))(pt).astype(np.int32)
    lat = bits(t["k_cache"].index_select(0, torch.tensor(used, dtype=torch.long, device=DEV)))
    kn = bits(t["k_new"][torch.tensor(bs, device=DEV)])
    seq = wl.seq_lens[bs]
    oracle.kv_append(seq, new_pt, len(used), kn, None, lat, None, mla=True)
    sel_local = sel.copy()
    sel_local[:, 0] = np.searchsorted(bs, sel[:, 0]) if (np.diff(bs) > 0).all() else \
        np.array([list(bs).index(b) for b in sel[:, 0]])
    ref = oracle.verify_attn(bits(t["q"][torch.tensor(bs, device=DEV)]), lat, None, new_pt, seq,
                             len(used), n_kv_heads=1, d_v=512, mla=True, sel=sel_local)
    o = out.cpu().numpy()
    got = np.stack([o[b, i, h] for b, i, h in sel])
    check_attention(got, ref, where="mla full config")


@pytest.mark.parametrize("L,key_pos", [(300, 200), (3000, 1000)])
def test_attention_mla_exact_path(L, key_pos):
    """A latent row whose score for head 0 is ~67 (log2 units) above every
    other key, placed past the first tile of its chunk: the fast kernel leaves
    those rows to the exact path, which must still match the oracle (one chunk
    and several chunks)."""
    B, K, Hq = 1, 3, 32
    wl = _mla_case(B, K, Hq, [L], seed=91)
    t = wl.tensors
    rng = np.random.default_rng(5)
    u = rng.standard_normal(576)
    u /= np.linalg.norm(u)
    q = t["q"].float()
    q[0, :, 0, :] = torch.from_numpy(8.0 * u).float()
    t["q"] = q.to(torch.bfloat16)
    pg = int(wl.page_table[0, key_pos // 64])
    lat = t["k_cache"].float()
    lat[pg, key_pos % 64, :] = torch.from_numpy(140.0 * u).float()
    t["k_cache"] = lat.to(torch.bfloat16)
    out, lowp, lat_gpu, err = _run_gpu_mla(wl)
    ref, lat_ref = _oracle_mla(wl)
    assert err == 0
    o = out.cpu().numpy()
    # The dominant key carries the head-0 rows.
    dom = oracle.bf16_to_f64(bits(t["k_cache"]))[pg, key_pos % 64, :512]
    assert np.abs(ref[0, :, 0, :] - dom).max() < 1e-3 * np.abs(dom).max()
    check_attention(o, ref, where=f"mla exact path L={L}")

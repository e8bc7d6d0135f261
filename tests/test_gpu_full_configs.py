"""Parity at the full sizes of the four GPU configurations, in the launch
configuration that bench.py times (VerifyStep over device-resident inputs).
The oracle cannot redo these in seconds, so each call is checked on samples
it can compute one by one: attention rows of a few requests (their pages
copied to the host before the step), LM-head rows against exact fp64 dot
products, and acceptance plus rollback over the whole batch, with the GPU's
own logits as the acceptance input.

The sampled requests always include the longest and the shortest one; for
the GQA kernel at least one sampled (request, kv head) pair is cut between
waves (so its rows go through the partial slots and the combine), and the
attention rows include every row of such a pair's first query head.  At
least 64 attention rows and 32 LM-head rows are checked per configuration."""
import numpy as np
import pytest
import torch

import oracle
import sdsynth
import speculative_decoding_sd_amd as sdv
from parity import (DEV, bits, host, check_attention, check_logits_bf16, compare_accept,
                    gather_requests, gqa_wave_split_pairs, sample_requests)

pytestmark = pytest.mark.gpu


def _drafts(cfg, seed, lg, temperature, top_p):
    """Draft stand-in from the target logits: greedy requests copy the
    target's argmax for a Geometric(p) prefix; sampled requests draw from
    softmax((logits + noise) / T) (the recipe bench.py uses)."""
    B, Q, V = lg.shape
    K = Q - 1
    greedy = temperature == 0
    drafts = np.full((B, K), -1, np.int32)
    pd = np.zeros((B, K, V), np.float32)
    if greedy.any():
        tt = np.argmax(lg, axis=-1)
        drafts[greedy] = sdsynth.greedy_drafts(tt, K, V, seed, p=cfg.geom_p)[greedy]
    st = np.nonzero(~greedy)[0]
    if len(st) and K > 0:
        pd_st = sdsynth.draft_probs(lg[st, :K], seed, cfg.draft_noise, float(temperature[st[0]]),
                                    float(top_p[st[0]]))
        pd[st] = pd_st
        drafts[st] = sdsynth.sample_drafts(pd_st, seed)
    return drafts, pd


@pytest.mark.parametrize("ci", [2, 3, 4, 5])
def test_full_config_step(ci):
    cfg = sdsynth.CONFIGS[ci]
    seed = sdsynth.config_seed(ci)
    torch.cuda.empty_cache()
    wl = sdsynth.make_workload(cfg, seed, device=DEV, extra_tokens=cfg.num_q)
    t = wl.tensors
    B, Q = cfg.batch, cfg.num_q
    rng = np.random.default_rng(ci)
    reqs = sample_requests(wl.seq_lens, rng, n_random=1 if ci == 4 else 2)
    sample = gather_requests(wl, reqs)
    print(f"config {ci}: sampled requests {reqs.tolist()}", flush=True)

    L0 = wl.seq_lens.copy()
    seq_lens = torch.tensor(L0, device=DEV)
    page_table = torch.tensor(wl.page_table, device=DEV)
    temp = torch.tensor(wl.temperature, device=DEV)
    top_p = torch.tensor(wl.top_p, device=DEV) if (wl.top_p < 1).any() else None
    drafts = torch.full((B, cfg.K), -1, dtype=torch.int32, device=DEV)
    pd = torch.zeros((B, cfg.K, cfg.vocab), dtype=torch.float32, device=DEV)
    step = sdv.VerifyStep(q=t["q"], k_cache=t["k_cache"], v_cache=t["v_cache"],
                          page_table=page_table, seq_lens=seq_lens, num_pages=wl.num_pages,
                          max_seq_len=int(L0.max()), n_kv_heads=cfg.n_kv_heads, W=t["W"],
                          drafts=drafts, temperature=temp,
                          u_accept=torch.tensor(wl.u_accept, device=DEV),
                          u_sample=torch.tensor(wl.u_sample, device=DEV), k_new=t["k_new"],
                          v_new=t["v_new"], mla=cfg.mla, d_v=cfg.d_v, H=t.get("H"), top_p=top_p,
                          draft_probs=pd if (wl.temperature > 0).any() else None)
    step.attention()
    step.lm_head()
    torch.cuda.synchronize()
    assert int(step.dev_error.item()) == 0

    # Attention: at least 64 rows of the sampled requests.
    kc, vc = sample["k_cache"], sample["v_cache"]
    oracle.kv_append(sample["seq_lens"], sample["page_table"], sample["num_pages"],
                     sample["k_new"], sample["v_new"], kc, vc, mla=cfg.mla)
    longest_first = np.argsort(-sample["seq_lens"], kind="stable")
    sel, n_split = _attention_rows(cfg, wl, reqs, rng, cfg.mla, False)
    print(f"config {ci}: {len(sel)} attention rows, {n_split} sampled split pairs", flush=True)
    ref = oracle.verify_attn(sample["q"], kc, vc, sample["page_table"], sample["seq_lens"],
                             sample["num_pages"], n_kv_heads=cfg.n_kv_heads, d_v=cfg.d_v,
                             mla=cfg.mla, sel=sel)
    o = step.out.cpu().numpy()
    got = np.stack([o[reqs[b], i, h] for b, i, h in sel])
    check_attention(got, ref, where=f"config {ci} attention")

    # LM head: at least 32 rows, exact fp64 logits from the kernel's own input.
    rows = _lm_rows(B, Q, reqs[longest_first], rng)
    hin = bits(step.hin.index_select(0, torch.tensor(rows, dtype=torch.long, device=DEV)))
    exact = oracle.lm_head(hin, bits(t["W"]))
    lg_rows = bits(step.logits.view(B * Q, -1).index_select(
        0, torch.tensor(rows, dtype=torch.long, device=DEV)))
    check_logits_bf16(lg_rows, exact, where=f"config {ci} lm head")

    # Acceptance and rollback over the whole batch on the GPU's logits.
    lg_bits = bits(step.logits)
    lf = oracle.bf16_to_f64(lg_bits)
    d_h, pd_h = _drafts(cfg, seed, lf.astype(np.float32), wl.temperature, wl.top_p)
    drafts.copy_(torch.from_numpy(d_h))
    pd.copy_(torch.from_numpy(pd_h))
    del lf
    step.accept()
    step.rollback()
    torch.cuda.synchronize()
    ref_acc = oracle.accept(lg_bits, d_h, wl.temperature,
                            wl.top_p if (wl.top_p < 1).any() else None, pd_h, wl.u_accept,
                            wl.u_sample)
    gpu = {"num_accepted": step.num_accepted.cpu().numpy(),
           "out_tokens": step.out_tokens.cpu().numpy(),
           "next_token": step.next_token.cpu().numpy(),
           "out_offsets": step.out_offsets.cpu().numpy(),
           "packed_tokens": step.packed.cpu().numpy()}
    n_excl = compare_accept(gpu, ref_acc, where=f"config {ci} accept")
    assert n_excl <= max(1, B // 16)
    assert int(step.dev_error.item()) == 0
    rb = oracle.kv_rollback(wl.page_table, ref_acc["num_accepted"], L0, cfg.K)
    keep = ref_acc["num_accepted"] >= 0
    assert np.array_equal(seq_lens.cpu().numpy()[keep], rb["seq_lens"][keep])
    if n_excl == 0:
        assert np.array_equal(step.rb_offsets.cpu().numpy(), rb["rb_offsets"])
        assert np.array_equal(step.rb_slots.cpu().numpy(), rb["rb_slots"])


@pytest.mark.parametrize("ci,kv,tree", [(5, "e4m3", None), (4, "e4m3", None),
                                        (5, "as_dtype", "binary"), (5, "e4m3", "binary")])
def test_full_config_variants(ci, kv, tree):
    """The E4M3 cache and the draft-tree variants bench.py times, at full size:
    sampled attention rows, sampled LM-head rows, acceptance over the whole
    batch on the GPU's logits, and the rollback (with the tree gather)."""
    import dataclasses
    cfg = dataclasses.replace(sdsynth.CONFIGS[ci], kv_cache=kv)
    if tree:
        cfg = dataclasses.replace(cfg, temperature=0.0, top_p=1.0, mixed_modes=None)
    seed = sdsynth.config_seed(ci)
    torch.cuda.empty_cache()
    wl = sdsynth.make_workload(cfg, seed, device=DEV, extra_tokens=cfg.num_q)
    t = wl.tensors
    B, Q = cfg.batch, cfg.num_q
    par = sdsynth.tree_parents(tree, Q) if tree else None
    par_b = np.tile(par, (B, 1)) if tree else None
    rng = np.random.default_rng(ci + 10)
    reqs = sample_requests(wl.seq_lens, rng, n_random=1 if ci == 4 else 2)
    sample = gather_requests(wl, reqs)
    if kv == "e4m3":   # host() keeps uint8 codes as they are
        scales = dict(k_scale=t["k_scale"].cpu().numpy(), v_scale=t["v_scale"].cpu().numpy())
    else:
        scales = {}
    print(f"config {ci} {kv} {tree}: sampled requests {reqs.tolist()}", flush=True)
    L0 = wl.seq_lens.copy()
    seq_lens = torch.tensor(L0, device=DEV)
    page_table = torch.tensor(wl.page_table, device=DEV)
    temp = torch.tensor(wl.temperature, device=DEV)
    top_p = torch.tensor(wl.top_p, device=DEV) if (wl.top_p < 1).any() else None
    drafts = torch.full((B, cfg.K), -1, dtype=torch.int32, device=DEV)
    pd = torch.zeros((B, cfg.K, cfg.vocab), dtype=torch.float32, device=DEV)
    step = sdv.VerifyStep(q=t["q"], k_cache=t["k_cache"], v_cache=t["v_cache"],
                          page_table=page_table, seq_lens=seq_lens, num_pages=wl.num_pages,
                          max_seq_len=int(L0.max()), n_kv_heads=cfg.n_kv_heads, W=t["W"],
                          drafts=drafts, temperature=temp,
                          u_accept=torch.tensor(wl.u_accept, device=DEV),
                          u_sample=torch.tensor(wl.u_sample, device=DEV), k_new=t["k_new"],
                          v_new=t["v_new"], d_v=cfg.d_v, H=t.get("H"), top_p=top_p,
                          draft_probs=pd if (wl.temperature > 0).any() else None,
                          k_scale=t.get("k_scale"), v_scale=t.get("v_scale"),
                          tree_parent=torch.tensor(par_b, device=DEV) if tree else None)
    step.attention()
    step.lm_head()
    torch.cuda.synchronize()
    assert int(step.dev_error.item()) == 0

    kc, vc = sample["k_cache"], sample["v_cache"]
    oracle.kv_append(sample["seq_lens"], sample["page_table"], sample["num_pages"],
                     sample["k_new"], sample["v_new"], kc, vc, **scales)
    sel, n_split = _attention_rows(cfg, wl, reqs, rng, False, kv == "e4m3")
    print(f"config {ci} {kv} {tree}: {len(sel)} attention rows, {n_split} sampled split "
          f"pairs", flush=True)
    ref = oracle.verify_attn(sample["q"], kc, vc, sample["page_table"], sample["seq_lens"],
                             sample["num_pages"], n_kv_heads=cfg.n_kv_heads, d_v=cfg.d_v,
                             sel=sel, tree_parent=par_b[:len(reqs)] if tree else None, **scales)
    o = step.out.cpu().numpy()
    check_attention(np.stack([o[reqs[b], i, h] for b, i, h in sel]), ref,
                    where=f"config {ci} {kv} {tree} attention")

    rows = _lm_rows(B, Q, reqs[np.argsort(-sample["seq_lens"], kind="stable")], rng)
    ridx = torch.tensor(rows, dtype=torch.long, device=DEV)
    exact = oracle.lm_head(bits(step.hin.index_select(0, ridx)), bits(t["W"]))
    check_logits_bf16(bits(step.logits.view(B * Q, -1).index_select(0, ridx)), exact,
                      where=f"config {ci} {kv} {tree} lm head")

    lg_bits = bits(step.logits)
    lf = oracle.bf16_to_f64(lg_bits).astype(np.float32)
    if tree:
        d_h = sdsynth.tree_drafts(np.argmax(lf, axis=-1), par, cfg.vocab, seed)
        pd_h = None
    else:
        d_h, pd_h = _drafts(cfg, seed, lf, wl.temperature, wl.top_p)
        pd.copy_(torch.from_numpy(pd_h))
    del lf
    drafts.copy_(torch.from_numpy(d_h))
    step.accept()
    step.rollback()
    torch.cuda.synchronize()
    ref_acc = oracle.accept(lg_bits, d_h, wl.temperature,
                            wl.top_p if (wl.top_p < 1).any() else None, pd_h, wl.u_accept,
                            wl.u_sample, tree_parent=par_b)
    gpu = {"num_accepted": step.num_accepted.cpu().numpy(),
           "out_tokens": step.out_tokens.cpu().numpy(),
           "next_token": step.next_token.cpu().numpy(),
           "out_offsets": step.out_offsets.cpu().numpy(),
           "packed_tokens": step.packed.cpu().numpy()}
    n_excl = compare_accept(gpu, ref_acc, where=f"config {ci} {kv} {tree} accept")
    assert n_excl <= max(1, B // 16)
    assert int(step.dev_error.item()) == 0
    if tree:
        assert np.array_equal(step.accepted_nodes.cpu().numpy(), ref_acc["accepted_nodes"])
        assert ref_acc["num_accepted"].mean() > 0.5
    # Rollback: lengths for every kept request; the gathered cache rows of the
    # sampled requests against the oracle's gather of their host copies.
    rb = oracle.kv_rollback(sample["page_table"], ref_acc["num_accepted"][reqs],
                            sample["seq_lens"], cfg.K, k_cache=kc, v_cache=vc,
                            n_kv_heads=cfg.n_kv_heads, d_k=cfg.d_qk, d_v=cfg.d_v,
                            accepted_nodes=ref_acc["accepted_nodes"][reqs] if tree else None)
    keep = ref_acc["num_accepted"] >= 0
    assert np.array_equal(seq_lens.cpu().numpy()[keep], (L0 + ref_acc["num_accepted"] + 1)[keep])
    kc_gpu = t["k_cache"]
    for k, b in enumerate(reqs):
        for p in range(int(L0[b]), int(rb["seq_lens"][k])):
            pg_g, pg_s, off = wl.page_table[b, p // 64], sample["page_table"][k, p // 64], p % 64
            got = kc_gpu[pg_g, :, off]
            got = got.cpu().numpy() if kv == "e4m3" else bits(got)
            assert np.array_equal(got, kc[pg_s, :, off]), (b, p)


def _attention_rows(cfg, wl, reqs, rng, mla, e4m3, n_rows=64):
    """Rows (index into reqs, position, query head) to check: every position
    of one head of a wave-split pair among the sampled requests (GQA), then
    random rows up to n_rows, at least one per position of every sampled
    request."""
    Q, Hq, Hkv = cfg.num_q, cfg.n_q_heads, cfg.n_kv_heads
    rows = []
    split = []
    if not mla:
        cus = torch.cuda.get_device_properties(DEV).multi_processor_count
        R = (Hq // Hkv) * Q
        split = [(b, h) for b, h in gqa_wave_split_pairs(
            wl.seq_lens, Q, Hkv, R, int(wl.seq_lens.max()), e4m3, cus) if b in set(reqs.tolist())]
        assert split, "no sampled (request, kv head) pair is split between waves"
        b, h = split[int(rng.integers(len(split)))]
        k = int(np.nonzero(reqs == b)[0][0])
        G = Hq // Hkv
        rows += [(k, i, h * G + int(rng.integers(G))) for i in range(Q)]
    for k in range(len(reqs)):
        rows += [(k, i, int(rng.integers(Hq))) for i in range(Q)]
    while len(rows) < n_rows:
        rows.append((int(rng.integers(len(reqs))), int(rng.integers(Q)), int(rng.integers(Hq))))
    return np.array(rows, np.int64), len(split)


def _lm_rows(B, Q, reqs, rng, n_rows=32):
    """LM-head rows to check: every row of the longest sampled request (the
    first one listed), then random rows up to n_rows."""
    rows = set(int(reqs[0]) * Q + i for i in range(Q))
    while len(rows) < n_rows:
        rows.add(int(rng.integers(B * Q)))
    return np.array(sorted(rows), np.int32)

"""The verify step captured as one HIP graph ([TRT-MTP] 基本實現方式 Fig. 4:
verify and draft run as one graph, rollback outside it; 評估 Fig. 7: the
graph speed-up), checked against the oracle on every replay.

A decode loop of replays: each replay continues from the state the previous
one left (seq_lens advanced by the rollback, the cache holding the appended
rows).  Before each replay the sampled requests' cache pages are copied to
the host; after it, the oracle recomputes from those copies and the
replay's own inputs:
  * attention rows of the sampled requests (append + causal attention);
  * LM-head rows against exact fp64 dot products of the replay's input rows;
  * acceptance over the whole batch on the replay's logits (stage-wise);
  * the rollback: new lengths, rejected slots and freed pages.
The same state is also run eagerly once per replay, and the replay must
equal it bit for bit (same kernels, fixed-order reductions).  Replays are
interleaved with eager work and host synchronisation, so a graph node that
behaves differently after its first replay is caught.  Sizes: the tiny
float32 configuration and the GQA sampling configuration at full size, and
a 24-request slice of the ragged serving batch."""
import numpy as np
import pytest
import torch

import oracle
import sdsynth
import speculative_decoding_sd_amd as sdv
from parity import (DEV, bits, host, check_attention, check_logits_bf16, check_logits_f32,
                    compare_accept, gather_requests, sample_requests)
from test_gpu_full_configs import _drafts

pytestmark = pytest.mark.gpu


def _outputs(step):
    return {"out": step.out.clone(), "logits": step.logits.clone(),
            "num_accepted": step.num_accepted.clone(), "packed": step.packed.clone(),
            "out_offsets": step.out_offsets.clone(), "rb_slots": step.rb_slots.clone(),
            "rb_offsets": step.rb_offsets.clone(), "freed": step.freed.clone(),
            "freed_offsets": step.freed_offsets.clone()}


@pytest.mark.parametrize("ci,batch", [(1, None), (2, None), (5, 24)])
def test_graph_replays_match_oracle(ci, batch):
    cfg = sdsynth.CONFIGS[ci]
    seed = sdsynth.config_seed(ci)
    n_steps = 3
    wl = sdsynth.make_workload(cfg, seed, device=DEV, batch=batch,
                               extra_tokens=(2 * n_steps + 2) * cfg.num_q)
    t = wl.tensors
    B, Q = len(wl.seq_lens), cfg.num_q
    f32 = cfg.dtype == "f32"
    rng = np.random.default_rng(100 + ci)
    L0 = wl.seq_lens.copy()
    seq_lens = torch.tensor(L0, device=DEV)
    page_table = torch.tensor(wl.page_table, device=DEV)
    temp = torch.tensor(wl.temperature, device=DEV)
    top_p = torch.tensor(wl.top_p, device=DEV) if (wl.top_p < 1).any() else None
    drafts = torch.full((B, cfg.K), -1, dtype=torch.int32, device=DEV)
    pd = torch.zeros((B, cfg.K, cfg.vocab), dtype=torch.float32, device=DEV)
    step = sdv.VerifyStep(q=t["q"], k_cache=t["k_cache"], v_cache=t["v_cache"],
                          page_table=page_table, seq_lens=seq_lens, num_pages=wl.num_pages,
                          max_seq_len=int(L0.max()) + (2 * n_steps + 1) * Q,
                          n_kv_heads=cfg.n_kv_heads, W=t["W"], drafts=drafts, temperature=temp,
                          u_accept=torch.tensor(wl.u_accept, device=DEV),
                          u_sample=torch.tensor(wl.u_sample, device=DEV), k_new=t["k_new"],
                          v_new=t["v_new"], mla=cfg.mla, d_v=cfg.d_v, H=t.get("H"), top_p=top_p,
                          draft_probs=pd if (wl.temperature > 0).any() else None)
    step.attention()
    step.lm_head()
    torch.cuda.synchronize()
    d_h, pd_h = _drafts(cfg, seed, step.logits.float().cpu().numpy(), wl.temperature, wl.top_p)
    drafts.copy_(torch.from_numpy(d_h))
    pd.copy_(torch.from_numpy(pd_h))
    seq_lens.copy_(torch.from_numpy(L0))
    step.run()                       # eager first step (also loads every kernel)
    torch.cuda.synchronize()
    step.capture()
    torch.cuda.synchronize()
    reqs = sample_requests(L0, rng, n_random=2)
    W_bits = host(t["W"])
    top_p_h = wl.top_p if (wl.top_p < 1).any() else None
    for r in range(n_steps):
        L_r = seq_lens.cpu().numpy().copy()
        # Host copies of the sampled requests' pages as the replay will find them.
        sample = gather_requests(wl, reqs)
        sample["seq_lens"] = L_r[reqs].copy()
        L_before = seq_lens.clone()
        step.run()                   # eager step from state S_r
        torch.cuda.synchronize()
        ref = _outputs(step)
        L_eager = seq_lens.clone()
        seq_lens.copy_(L_before)     # back to S_r (the cache rows it rewrites are the same)
        torch.cuda.synchronize()
        step.replay()                # graph step from S_r
        torch.cuda.synchronize()
        got = _outputs(step)
        print(f"config {ci} replay {r}: accepted {got['num_accepted'].sum().item()}", flush=True)
        for k in ref:
            assert torch.equal(ref[k], got[k]), (r, k)
        assert torch.equal(seq_lens, L_eager), r
        assert int(step.dev_error.item()) == 0

        # Attention rows against the oracle on the host copies.
        kc, vc = sample["k_cache"], sample["v_cache"]
        oracle.kv_append(sample["seq_lens"], sample["page_table"], sample["num_pages"],
                         sample["k_new"], sample["v_new"], kc, vc, mla=cfg.mla)
        n_rows = min(32, len(reqs) * Q * cfg.n_q_heads)
        sel = np.array([(k, i, int(rng.integers(cfg.n_q_heads)))
                        for k in range(len(reqs)) for i in range(Q)] +
                       [(int(rng.integers(len(reqs))), int(rng.integers(Q)),
                         int(rng.integers(cfg.n_q_heads)))
                        for _ in range(max(0, n_rows - len(reqs) * Q))], np.int64)
        ref_o = oracle.verify_attn(sample["q"], kc, vc, sample["page_table"],
                                   sample["seq_lens"], sample["num_pages"],
                                   n_kv_heads=cfg.n_kv_heads, d_v=cfg.d_v, mla=cfg.mla,
                                   sel=sel)
        o = got["out"].cpu().numpy()
        check_attention(np.stack([o[reqs[k], i, h] for k, i, h in sel]), ref_o,
                        where=f"config {ci} replay {r} attention")

        # LM-head rows: exact dot products of the replay's input rows.
        rows = np.unique(np.concatenate([[int(reqs[0]) * Q],
                                         rng.integers(0, B * Q, 8)])).astype(np.int32)
        ridx = torch.tensor(rows, dtype=torch.long, device=DEV)
        hin = host(step.hin.index_select(0, ridx))
        lg_rows = got["logits"].view(B * Q, -1).index_select(0, ridx)
        if f32:
            exact = oracle.lm_head(hin.astype(np.float64), W_bits.astype(np.float64))
            check_logits_f32(lg_rows.cpu().numpy(), exact,
                             where=f"config {ci} replay {r} lm head")
        else:
            exact = oracle.lm_head(hin, W_bits)
            check_logits_bf16(bits(lg_rows), exact, where=f"config {ci} replay {r} lm head")

        # Acceptance over the whole batch on the replay's logits, then rollback.
        ref_acc = oracle.accept(host(got["logits"]), d_h, wl.temperature, top_p_h, pd_h,
                                wl.u_accept, wl.u_sample)
        gpu = {"num_accepted": got["num_accepted"].cpu().numpy(),
               "out_tokens": step.out_tokens.cpu().numpy(),
               "next_token": step.next_token.cpu().numpy(),
               "out_offsets": got["out_offsets"].cpu().numpy(),
               "packed_tokens": got["packed"].cpu().numpy()}
        n_excl = compare_accept(gpu, ref_acc, where=f"config {ci} replay {r} accept")
        assert n_excl <= max(1, B // 16)
        # Rollback stage-wise, from the accepted counts the replay produced.
        rb = oracle.kv_rollback(wl.page_table, gpu["num_accepted"], L_r, cfg.K)
        assert np.array_equal(seq_lens.cpu().numpy(), rb["seq_lens"]), r
        for k_g, k_r in (("rb_offsets", "rb_offsets"), ("rb_slots", "rb_slots"),
                         ("freed_offsets", "freed_offsets")):
            assert np.array_equal(got[k_g].cpu().numpy(), rb[k_r]), (r, k_g)
        n_freed = int(rb["freed_offsets"][-1])
        assert np.array_equal(got["freed"].cpu().numpy()[:n_freed], rb["freed"][:n_freed]), r

"""The verify step captured as one HIP graph: every replay must equal the
eager step taken from the same state (same kernels, same inputs, fixed-order
reductions, so bit for bit).  Replays are interleaved with eager work and
host synchronisation, and each is checked, so a graph node that behaves
differently after its first replay is caught."""
import numpy as np
import pytest
import torch

import sdsynth
import speculative_decoding_sd_amd as sdv
from parity import DEV
from test_gpu_full_configs import _drafts

pytestmark = pytest.mark.gpu


def _outputs(step):
    return {"out": step.out.clone(), "logits": step.logits.clone(),
            "num_accepted": step.num_accepted.clone(), "packed": step.packed.clone(),
            "out_offsets": step.out_offsets.clone(), "rb_slots": step.rb_slots.clone(),
            "freed": step.freed.clone()}


@pytest.mark.parametrize("ci,batch", [(2, 16), (5, 24)])
def test_graph_replay_matches_eager(ci, batch):
    cfg = sdsynth.CONFIGS[ci]
    seed = sdsynth.config_seed(ci)
    n_steps = 3
    wl = sdsynth.make_workload(cfg, seed, device=DEV, batch=batch,
                               extra_tokens=(2 * n_steps + 2) * cfg.num_q)
    t = wl.tensors
    B, Q = batch, cfg.num_q
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
    for r in range(n_steps):
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
        print(f"config {ci} replay {r}: accepted {ref['num_accepted'].sum().item()}", flush=True)
        for k in ref:
            assert torch.equal(ref[k], got[k]), (r, k)
        assert torch.equal(seq_lens, L_eager), r
    assert int(step.dev_error.item()) == 0

"""One verify step of a draft chain: the four library calls on one stream.

VerifyStep owns the outputs and workspaces for one configuration and issues
sd_verify_attn -> sd_lm_head -> sd_accept -> sd_kv_rollback, eagerly (run) or
as one captured HIP graph (capture / replay).  The LM-head
input is either a caller-supplied hidden matrix H [B*(K+1), hidden] or the
attention output itself (rounded to q's dtype) when H is None.  An E4M3
(uint8) cache takes its per-kv-head k_scale / v_scale.  A tree of drafts
(tree_parent [B, K+1]) goes to the attention and the acceptance, and the
accepted node path to the rollback.
"""
from __future__ import annotations

import torch

from . import (accept_desc, attn_desc, rollback_desc, sd_accept, sd_accept_workspace_size,
               sd_kv_rollback, sd_lm_head, sd_verify_attn, sd_verify_attn_workspace_size,
               sd_dtype, workspace, _aligned, current_stream)


class VerifyStep:
    def __init__(self, *, q, k_cache, v_cache, page_table, seq_lens, num_pages, max_seq_len,
                 n_kv_heads, W, drafts, temperature, u_accept, u_sample, k_new=None,
                 v_new=None, mla=False, d_v=None, H=None, top_p=None, draft_probs=None,
                 poison=False, k_scale=None, v_scale=None, tree_parent=None):
        dev = q.device
        B, Q, Hq, dqk = q.shape
        self.B, self.Q, self.K = B, Q, Q - 1
        d_v = d_v if d_v is not None else (v_cache.shape[-1] if v_cache is not None else dqk)
        self.out = torch.empty((B, Q, Hq, d_v), dtype=torch.float32, device=dev)
        self.H = H
        self.out_lowp = None
        if H is None:
            self.out_lowp = torch.empty((B * Q, Hq * d_v), dtype=q.dtype, device=dev)
        self.dev_error = torch.zeros(1, dtype=torch.int32, device=dev)
        self.attn = attn_desc(q=q, k_cache=k_cache, v_cache=v_cache, page_table=page_table,
                              seq_lens=seq_lens, out=self.out, n_kv_heads=n_kv_heads,
                              num_pages=num_pages, max_seq_len=max_seq_len, k_new=k_new,
                              v_new=v_new, mla=mla, out_lowp=self.out_lowp,
                              dev_error=self.dev_error, k_scale=k_scale, v_scale=v_scale,
                              tree_parent=tree_parent)
        self.attn_ws = workspace(sd_verify_attn_workspace_size(self.attn), dev)
        hin = H if H is not None else self.out_lowp
        self.W = W
        self.hin = hin
        V = W.shape[0]
        self.vocab = V
        self.logits = torch.empty((B, Q, V), dtype=W.dtype, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.num_accepted = torch.empty(B, **i32)
        self.out_tokens = torch.empty((B, Q), **i32)
        self.next_token = torch.empty(B, **i32)
        self.out_offsets = torch.empty(B + 1, **i32)
        self.packed = torch.empty(B * Q, **i32)
        # A tree's accepted node path: the rollback gathers the kept rows by it.
        self.accepted_nodes = torch.empty((B, Q), **i32) if tree_parent is not None else None
        self.acc = accept_desc(logits=self.logits, draft_tokens=drafts, temperature=temperature,
                               u_accept=u_accept, u_sample=u_sample,
                               num_accepted=self.num_accepted, out_tokens=self.out_tokens,
                               next_token=self.next_token, out_offsets=self.out_offsets,
                               packed_tokens=self.packed, top_p=top_p, draft_probs=draft_probs,
                               dev_error=self.dev_error, tree_parent=tree_parent,
                               accepted_nodes=self.accepted_nodes)
        self.acc_ws = workspace(sd_accept_workspace_size(self.acc), dev)
        ps = 64
        self.rb_slots = torch.empty(B * Q, **i32)
        self.rb_offsets = torch.empty(B + 1, **i32)
        self.freed = torch.empty(B * ((Q - 1) // ps + 2), **i32)
        self.freed_offsets = torch.empty(B + 1, **i32)
        self.rb = rollback_desc(page_table=page_table, num_accepted=self.num_accepted,
                                seq_lens=seq_lens, K=Q - 1, rollback_slots=self.rb_slots,
                                rollback_offsets=self.rb_offsets, freed_pages=self.freed,
                                freed_offsets=self.freed_offsets, poison=poison,
                                k_cache=k_cache, v_cache=v_cache, mla=mla,
                                n_kv_heads=n_kv_heads, d_k=dqk, d_v=d_v, num_pages=num_pages,
                                dev_error=self.dev_error, accepted_nodes=self.accepted_nodes)
        self._keep = (q, k_cache, v_cache, page_table, seq_lens, W, drafts, temperature,
                      u_accept, u_sample, k_new, v_new, H, top_p, draft_probs, k_scale, v_scale,
                      tree_parent)

    def _ws(self, t):
        return _aligned(t), t.numel() - (_aligned(t) - t.data_ptr())

    def attention(self, stream=None):
        s = current_stream() if stream is None else stream
        p, n = self._ws(self.attn_ws)
        sd_verify_attn(self.attn, p, n, s)

    def lm_head(self, stream=None):
        s = current_stream() if stream is None else stream
        M, hidden = self.hin.shape
        sd_lm_head(M, hidden, self.vocab, sd_dtype(self.W), self.hin.data_ptr(),
                   self.W.data_ptr(), self.logits.data_ptr(), s)

    def accept(self, stream=None):
        s = current_stream() if stream is None else stream
        p, n = self._ws(self.acc_ws)
        sd_accept(self.acc, p, n, s)

    def rollback(self, stream=None):
        s = current_stream() if stream is None else stream
        sd_kv_rollback(self.rb, s)

    def run(self, stream=None):
        self.attention(stream)
        self.lm_head(stream)
        self.accept(stream)
        self.rollback(stream)

    def capture(self):
        """Records the four calls of one step into a HIP graph (torch's
        CUDAGraph on ROCm), so that replay() re-issues the whole step with one
        launch.  The library allocates nothing and records no memsets, and the
        step reads its state (seq_lens, page table, cache) from device memory,
        so every replay is the next step.  Call run() once before capturing."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()

"""GPU parity of the rejection-sampling rule's edge branches.

The constructions of tests/test_oracle_accept_edges.py, injected into a
batch at full vocabulary sizes ([SD-PRACTICE] s4.4, [VLLM-MTP] s3 stage 3):
a draft whose draft probability is 0 (accepted when its target probability
is positive, rejected when both are 0), an all-zero residual after a
rejection (the replacement comes from p_t), and draws at u = 1, where no
running sum exceeds u * S and the largest id of positive weight is taken,
both for a residual and for the bonus token, and rows whose leading logits
are -inf (masked tokens) with the drafts among them.  Each of these is exact on both
sides (the decisions do not depend on summation order), so every request is
compared, with no exclusion window.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import DEV, compare_accept, host, run_accept

pytestmark = pytest.mark.gpu

U_MAX = np.float32(1.0) - np.float32(2.0 ** -24)


def _softmax(x, T=1.0):
    z = np.exp((x - x.max()) / T)
    return z / z.sum()


def _edge_batch(V, dtype, seed):
    rng = np.random.default_rng(seed)
    K = 3
    Q = K + 1
    kinds = ["pd0_accept", "pd0_pt0_reject", "zero_residual", "u1_residual", "u1_bonus",
             "u1_bonus_full", "neg_inf_reject", "greedy"]
    B = len(kinds) * 2
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    lg = (torch.randn((B, Q, V), generator=torch.Generator().manual_seed(seed)) * 1.7).to(tdt)
    lg_f = lg.float().numpy().astype(np.float64)
    temp = np.ones(B, np.float32)
    top_p = np.ones(B, np.float32)
    drafts = rng.integers(0, V, (B, K)).astype(np.int32)
    pd = np.zeros((B, K, V), np.float32)
    for b in range(B):
        for n in range(K):
            pd[b, n] = _softmax(lg_f[b, n] + rng.normal(0, 0.5, V))
    ua = rng.random((B, Q)).astype(np.float32)
    us = rng.random((B, Q)).astype(np.float32)
    for b in range(B):
        kind = kinds[b % len(kinds)]
        if kind == "pd0_accept":
            # Every draft has p_d = 0 and p_t > 0: all accepted at u < 1.
            for n in range(K):
                pd[b, n, drafts[b, n]] = 0.0
                pd[b, n] /= pd[b, n].sum()
            ua[b] = U_MAX
        elif kind == "pd0_pt0_reject":
            # Draft 1 is the row's smallest logit, outside the 0.5 nucleus, and
            # has p_d = 0: ratio 0, rejected even at u = 0.
            temp[b], top_p[b] = 0.8, 0.5
            d = int(np.argmin(lg_f[b, 0]))
            drafts[b, 0] = d
            pd[b, 0, d] = 0.0
            pd[b, 0] /= pd[b, 0].sum()
            ua[b] = 0.0
        elif kind == "zero_residual":
            # Equal logits in row 0: p_t = 1/V; p_d a little above it everywhere,
            # so the draft is rejected at u = 1 - 2^-24 with an empty residual.
            lg[b, 0] = 0.0
            pt = 1.0 / V
            pd[b, 0] = np.float32(pt * (1.0 + 2.0 ** -21))
            assert (pd[b, 0].astype(np.float64) > pt).all()
            assert pt / float(pd[b, 0, 0]) < float(U_MAX)
            ua[b] = U_MAX
        elif kind == "u1_residual":
            # Draft 1 outside the 0.9 nucleus with a one-hot p_d: rejected; the
            # residual is p_t and u = 1 finds no crossing.
            top_p[b] = 0.9
            d = int(np.argmin(lg_f[b, 0]))
            drafts[b, 0] = d
            pd[b, 0] = 0.0
            pd[b, 0, d] = 1.0
            ua[b] = 0.0
            us[b, 0] = 1.0
        elif kind in ("u1_bonus", "u1_bonus_full"):
            # Every draft is its row's argmax with p_d = 0: all accepted; the
            # bonus token is drawn at u = 1 from row K (with or without a
            # nucleus).
            if kind == "u1_bonus":
                top_p[b] = 0.9
            for n in range(K):
                drafts[b, n] = int(np.argmax(lg.float().numpy()[b, n]))
                pd[b, n, drafts[b, n]] = 0.0
            us[b, K] = 1.0
        elif kind == "neg_inf_reject":
            # The first 40% of every row are -inf (masked tokens, p_t = 0),
            # the drafts sit there with p_d > 0: ratio 0, draft 1 rejected,
            # and the residual is p_t over the finite tokens.
            cut = (2 * V) // 5
            lg[b, :, :cut] = float("-inf")
            drafts[b] = rng.integers(0, cut, K)
            for n in range(K):
                pd[b, n, drafts[b, n]] = max(pd[b, n, drafts[b, n]], np.float32(1e-3))
        else:
            temp[b] = 0.0
    return kinds, lg, drafts, temp, top_p, pd, ua, us


@pytest.mark.parametrize("V,dtype", [(1000, "bf16"), (1000, "f32"), (32000, "bf16"),
                                     (129280, "bf16")])
def test_accept_edge_branches(V, dtype):
    kinds, lg, drafts, temp, top_p, pd, ua, us = _edge_batch(V, dtype, seed=V % 97 + 3)
    B, Q, _ = lg.shape
    lg_h = host(lg)
    ref = oracle.accept(lg_h, drafts, temp, top_p, pd, ua, us)
    t = lambda x: torch.tensor(x, device=DEV)
    gpu = run_accept(lg.to(DEV), t(drafts), t(temp), t(top_p), t(pd), t(ua), t(us))
    assert gpu["dev_error"] == 0
    for k_g, k_r in (("num_accepted", "num_accepted"), ("next_token", "next_token"),
                     ("out_tokens", "out_tokens"), ("out_offsets", "out_offsets"),
                     ("packed_tokens", "packed")):
        assert np.array_equal(gpu[k_g], ref[k_r]), (k_g, gpu[k_g], ref[k_r])
    # The constructions reached the branches they were built for.
    lg_f = lg.float().numpy()
    for b in range(B):
        kind = kinds[b % len(kinds)]
        j = ref["num_accepted"][b]
        if kind in ("pd0_accept", "u1_bonus", "u1_bonus_full"):
            assert j == Q - 1, (b, kind)
        if kind in ("pd0_pt0_reject", "zero_residual", "u1_residual", "neg_inf_reject"):
            assert j == 0, (b, kind)
        if kind == "u1_bonus_full":
            assert ref["next_token"][b] == V - 1
        if kind in ("u1_residual", "u1_bonus"):
            # the largest id inside the row's nucleus
            row = lg_f[b, 0 if kind == "u1_residual" else Q - 1].astype(np.float64)
            order = np.lexsort((np.arange(V), -row))
            p = np.exp(row - row.max())
            cum = np.cumsum(p[order]) / p.sum()
            lam = row[order[np.argmax(cum >= top_p[b])]]
            assert ref["next_token"][b] == np.nonzero(row >= lam)[0].max(), (b, kind)


@pytest.mark.parametrize("V", [32000, 129280])
def test_accept_residual_near_equal(V):
    """Residual draws where p_d sits within a few 1e-5 of p_t on every token
    (the residual is the small negative part of that difference).  The GPU
    sorts each token into or out of the residual's support with the row
    pass's Z, and sums again with the fp64 Z every chunk holding a token
    within 1e-5 (relative) of p_t = p_d.  Even requests only have tokens
    outside that margin (every chunk takes a/Z - b), odd ones mostly inside
    it.  Draft 1 has p_d = 2 p_t, so it is rejected at u = 1 - 2^-24 and the
    final token is drawn from the residual of row 0.  Compared with the
    oracle's draws under its exclusion windows."""
    rng = np.random.default_rng(V + 11)
    B, K = 12, 3
    Q = K + 1
    lg = (torch.randn((B, Q, V), generator=torch.Generator().manual_seed(V)) * 1.7).to(
        torch.bfloat16)
    lg_f = lg.float().numpy().astype(np.float64)
    temp = np.ones(B, np.float32)
    top_p = np.ones(B, np.float32)
    drafts = rng.integers(0, V, (B, K)).astype(np.int32)
    pd = np.zeros((B, K, V), np.float32)
    clean = np.array([-3e-5, -1.2e-5, 1.2e-5, 3e-5])
    mixed = np.array([-3e-5, -1.2e-5, -8e-6, -2e-6, 2e-6, 8e-6, 1.2e-5, 3e-5])
    for b in range(B):
        for n in range(K):
            p = _softmax(lg_f[b, n])
            eps = rng.choice(clean if b % 2 == 0 else mixed, V)
            pd[b, n] = (p * (1.0 + eps)).astype(np.float32)
            d = drafts[b, n]
            pd[b, n, d] = np.float32(2.0 * p[d])
    ua = np.full((B, Q), U_MAX, np.float32)
    us = rng.random((B, Q)).astype(np.float32)
    ref = oracle.accept(host(lg), drafts, temp, None, pd, ua, us)
    assert (ref["num_accepted"] == 0).all()
    t = lambda x: torch.tensor(x, device=DEV)
    gpu = run_accept(lg.to(DEV), t(drafts), t(temp), None, t(pd), t(ua), t(us))
    assert gpu["dev_error"] == 0
    n_excl = compare_accept(gpu, ref, where=f"near-equal residual V={V}")
    assert n_excl <= 1, n_excl

"""Pins of the oracle's acceptance rule (CPU only).

Worked examples come from tests/golden/*.json (each with its citation);
the rest are special cases with hand-derived answers and the losslessness
property checked by a chi-square test.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _greedy_from_fixture(orc, fx):
    vocab = fx["vocab"]
    ids = {t: i for i, t in enumerate(vocab)}
    V = len(vocab)
    drafts = np.array([[ids[t] for t in fx["drafts"]]], np.int32)
    K = drafts.shape[1]
    logits = np.zeros((1, K + 1, V), np.float32)
    for i, t in enumerate(fx["target_argmax_per_row"]):
        logits[0, i, ids[t]] = 4.0
    z = np.zeros(1, np.float32)
    u = np.zeros((1, K + 1), np.float32)
    out = orc.accept(logits, drafts, z, np.ones(1, np.float32), None, u, u)
    return out, ids, vocab


@pytest.mark.parametrize("name", ["trt_mtp_fig1_greedy.json", "vllm_mtp_sec4_greedy.json",
                                  "vllm_mtp_sec4_counterexample.json"])
def test_greedy_worked_examples(orc, name):
    fx = _load(name)
    out, ids, vocab = _greedy_from_fixture(orc, fx)
    exp = fx["expected"]
    j = int(out["num_accepted"][0])
    assert j == exp["num_accepted"]
    emitted = [vocab[t] for t in out["out_tokens"][0, : j + 1]]
    assert emitted == exp["emitted"]
    assert vocab[out["next_token"][0]] == exp["next_token"]
    assert list(out["out_tokens"][0, j + 1:]) == [-1] * (len(fx["drafts"]) - j)
    assert list(out["out_offsets"]) == [0, j + 1]
    assert [vocab[t] for t in out["packed"][: j + 1]] == exp["emitted"]
    # Rejected drafts are exactly the tail after the accepted prefix.
    assert fx["drafts"][j:] == exp["rejected_drafts"]


def test_stochastic_worked_example_one_hot_draft(orc):
    """SD practice s2.3 with s4.4's simplified rule: p_d one-hot at the draft."""
    fx = _load("sd_practice_sec2_3_stochastic.json")
    probs = fx["draft_target_probs"]
    K = len(probs)
    V = 6
    drafts = np.arange(K, dtype=np.int32)[None, :]  # tokens 0..4, token 5 never drafted
    pt = np.zeros((1, K + 1, V))
    for n, p in enumerate(probs):
        pt[0, n, :] = (1.0 - p) / (V - 1)
        pt[0, n, n] = p
    pt[0, K, :] = 1.0 / V
    logits = np.log(pt)  # softmax(log p) = p at T = 1
    pd = np.zeros((1, K, V), np.float32)
    for n in range(K):
        pd[0, n, n] = 1.0
    u_acc = np.full((1, K + 1), fx["u_accept"], np.float32)
    u_smp = np.full((1, K + 1), 0.5, np.float32)
    out = orc.accept(logits, drafts, np.ones(1, np.float32), np.ones(1, np.float32), pd,
                     u_acc, u_smp)
    assert out["num_accepted"][0] == fx["expected"]["num_accepted"]
    assert out["out_offsets"][1] == fx["expected"]["emitted_count"]
    # Residual of row 2 = p_t with token 2 removed: tokens 0,1,3,4,5 at 0.7/5 each,
    # S = 0.7, u*S = 0.35; running sums 0.14, 0.28, (token 2: 0.28), 0.42 > 0.35 -> 3.
    assert list(out["out_tokens"][0, :3]) == [0, 1, 3]


def test_greedy_argmax_ties_go_to_smallest_id(orc):
    V, K = 7, 2
    logits = np.zeros((1, K + 1, V), np.float32)
    logits[0, 0, [2, 5]] = 3.0   # tie between 2 and 5 -> 2
    logits[0, 1, [1, 4]] = 2.0   # tie -> 1
    logits[0, 2, [6, 3]] = 1.0   # tie -> 3
    drafts = np.array([[2, 1]], np.int32)
    z = np.zeros(1, np.float32)
    u = np.zeros((1, K + 1), np.float32)
    out = orc.accept(logits, drafts, z, z + 1, None, u, u)
    assert out["num_accepted"][0] == 2 and out["next_token"][0] == 3
    drafts = np.array([[5, 1]], np.int32)
    out = orc.accept(logits, drafts, z, z + 1, None, u, u)
    assert out["num_accepted"][0] == 0 and out["next_token"][0] == 2


def test_negative_draft_ends_chain(orc):
    V, K = 5, 3
    logits = np.zeros((1, K + 1, V), np.float32)
    for i in range(K + 1):
        logits[0, i, i] = 1.0
    drafts = np.array([[0, -1, 2]], np.int32)
    z = np.zeros(1, np.float32)
    u = np.zeros((1, K + 1), np.float32)
    out = orc.accept(logits, drafts, z, z + 1, None, u, u)
    assert out["num_accepted"][0] == 1 and out["next_token"][0] == 1


def test_invalid_requests_emit_nothing(orc):
    V, K, B = 4, 2, 5
    logits = np.zeros((B, K + 1, V), np.float32)
    logits[1, 2, 3] = np.nan
    drafts = np.zeros((B, K), np.int32)
    drafts[2, 1] = V  # out of range
    temp = np.zeros(B, np.float32)
    temp[3] = -1.0
    temp[4] = 1.0
    top_p = np.ones(B, np.float32)
    top_p[4] = 0.0
    pd = np.full((B, K, V), 1.0 / V, np.float32)
    u = np.zeros((B, K + 1), np.float32)
    out = orc.accept(logits, drafts, temp, top_p, pd, u, u)
    assert out["n_invalid"] == 4
    assert list(out["num_accepted"][1:]) == [-1] * 4
    assert list(out["next_token"][1:]) == [-1] * 4
    assert (out["out_tokens"][1:] == -1).all()
    assert out["num_accepted"][0] >= 0
    n0 = out["num_accepted"][0] + 1
    assert list(out["out_offsets"]) == [0] + [n0] * B


def test_identical_distributions_accept_everything(orc):
    rng = np.random.default_rng(3)
    B, K, V = 64, 4, 11
    logits = rng.standard_normal((B, K + 1, V))
    pt = np.exp(logits) / np.exp(logits).sum(-1, keepdims=True)
    pd = pt[:, :K].astype(np.float32)
    drafts = rng.integers(0, V, (B, K)).astype(np.int32)
    u = rng.random((B, K + 1)).astype(np.float32)
    # ratio = p_t / p_d is 1 up to the float32 rounding of p_d; u < 1 - 1e-6
    u = np.minimum(u, 0.999).astype(np.float32)
    out = orc.accept(logits, drafts, np.ones(B, np.float32), np.ones(B, np.float32), pd, u, u)
    assert (out["num_accepted"] == K).all()


def test_k0_is_plain_sampling(orc):
    V = 4
    logits = np.log(np.array([[[0.1, 0.2, 0.3, 0.4]]]))
    for u_s, expect in [(0.0, 0), (0.09, 0), (0.11, 1), (0.29, 1), (0.31, 2), (0.59, 2),
                        (0.61, 3), (0.999, 3)]:
        out = orc.accept(logits, np.zeros((1, 0), np.int32), np.ones(1, np.float32),
                         np.ones(1, np.float32), np.zeros((1, 0, V), np.float32),
                         np.zeros((1, 1), np.float32), np.array([[u_s]], np.float32))
        assert out["num_accepted"][0] == 0
        assert out["next_token"][0] == expect, (u_s, out["next_token"])


def test_top_p_hand_example(orc):
    """logits [3, 1, 1, 0] at T=1: probs e^3, e, e, 1 over Z = e^3 + 2e + 1,
    i.e. 0.7573, 0.1025, 0.1025, 0.0377.  top_p 0.8: 0.7573 < 0.8 <= 0.8598,
    the prefix ends on a logit-1 token and both logit-1 tokens are kept.
    top_p 0.7: only token 0.  Checked through K=0 sampling at u just below 1."""
    logits = np.array([[[3.0, 1.0, 1.0, 0.0]]], np.float32)
    Z = math.e ** 3 + 2 * math.e + 1
    p0 = math.e ** 3 / Z
    assert abs(p0 - 0.7573) < 1e-4

    def draw(tp, u_s):
        out = orc.accept(logits, np.zeros((1, 0), np.int32), np.ones(1, np.float32),
                         np.array([tp], np.float32), np.zeros((1, 0, 4), np.float32),
                         np.zeros((1, 1), np.float32), np.array([[u_s]], np.float32))
        return out["next_token"][0]

    # kept {0,1,2}: renormalised masses e^3, e, e over e^3 + 2e.
    keep_z = math.e ** 3 + 2 * math.e
    c0 = math.e ** 3 / keep_z
    c1 = (math.e ** 3 + math.e) / keep_z
    assert draw(0.8, c0 - 1e-4) == 0
    assert draw(0.8, c0 + 1e-4) == 1
    assert draw(0.8, c1 + 1e-4) == 2
    assert draw(0.8, 0.99999) == 2        # token 3 is filtered out
    assert draw(0.7, 0.99999) == 0        # only token 0 survives
    assert draw(1.0, 0.99999) == 3        # top_p = 1: no filtering
    # tie extension: top_p exactly reached inside a tied level keeps the level
    assert draw(0.76, 0.99999) == 2


def test_temperature_zero_is_greedy_even_with_probs(orc):
    rng = np.random.default_rng(5)
    B, K, V = 16, 3, 9
    logits = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    tstar = logits.argmax(-1)
    drafts = tstar[:, :K].astype(np.int32).copy()
    drafts[::2, 1] = (drafts[::2, 1] + 1) % V
    pd = np.full((B, K, V), 1.0 / V, np.float32)
    u = np.full((B, K + 1), 0.5, np.float32)
    out = orc.accept(logits, drafts, np.zeros(B, np.float32), np.ones(B, np.float32), pd, u, u)
    assert (out["num_accepted"][::2] == 1).all() and (out["num_accepted"][1::2] == K).all()
    assert (out["next_token"][1::2] == tstar[1::2, K]).all()
    assert (out["next_token"][::2] == tstar[::2, 1]).all()


def _chi2_trials(orc, seed, T, top_p, N=1_000_000, V=16, K=3, chunk=200_000):
    """N independent verify steps of one request with fixed target logits and
    draft distributions (drafts drawn from p_d), run through the oracle in
    chunks.  Returns the concatenated outputs, the target rows and p_d."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((K + 1, V)) * 1.5
    pd_rows = rng.dirichlet(np.full(V, 0.7), size=K)
    # The target distribution the rule must reproduce, written out from the
    # definition (tempered softmax, nucleus kept with ties, renormalised).
    def target(row):
        e = np.exp((row - row.max()) / T)
        p = e / e.sum()
        if top_p < 1:
            order = sorted(range(V), key=lambda v: (-row[v], v))
            cum, lam = 0.0, None
            for v in order:
                cum += p[v]
                if cum >= top_p:
                    lam = row[v]
                    break
            p = np.where(row >= lam, p, 0.0)
            p = p / p.sum()
        return p
    pt = np.stack([target(logits[i]) for i in range(K + 1)])
    pdf = pd_rows.astype(np.float32)
    cdf = np.cumsum(pdf.astype(np.float64), -1)
    outs = []
    for c0 in range(0, N, chunk):
        n = min(chunk, N - c0)
        ud = rng.random((n, K))
        drafts = np.stack([np.minimum(np.searchsorted(cdf[k] / cdf[k, -1], ud[:, k],
                                                      side="right"), V - 1)
                           for k in range(K)], 1).astype(np.int32)
        L = np.broadcast_to(logits.astype(np.float64), (n, K + 1, V))
        P = np.broadcast_to(pdf, (n, K, V))
        ua = rng.random((n, K + 1)).astype(np.float32)
        us = rng.random((n, K + 1)).astype(np.float32)
        outs.append(orc.accept(L, drafts, np.full(n, T, np.float32),
                               np.full(n, top_p, np.float32), P, ua, us))
    out = {k: np.concatenate([o[k] for o in outs]) for k in ("out_tokens", "num_accepted")}
    return out, pt, pdf


@pytest.mark.parametrize("seed,T,top_p", [(11, 1.0, 1.0), (12, 0.7, 0.9), (13, 1.0, 1.0),
                                         (14, 0.7, 0.9), (15, 1.3, 0.8)])
def test_rejection_sampling_is_lossless_chi2(orc, seed, T, top_p):
    """The first emitted token is distributed as the target row 0, and the
    token emitted after an accepted first draft as target row 1 (the rows do
    not depend on the drafts here), whatever the draft distribution.  Five
    seeds of 10^6 verify steps each, V = 16 (15 degrees of freedom at most),
    each required to pass at p > 1e-4."""
    N, V, K = 1_000_000, 16, 3
    out, pt, pdf = _chi2_trials(orc, seed, T, top_p, N, V, K)
    first = out["out_tokens"][:, 0]
    obs = np.bincount(first, minlength=V)
    exp = pt[0] * N
    m = exp > 0
    assert obs[~m].sum() == 0
    chi2 = ((obs[m] - exp[m]) ** 2 / exp[m]).sum()
    p = stats.chi2.sf(chi2, m.sum() - 1)
    assert p > 1e-4, (chi2, p)
    sel = out["num_accepted"] >= 1
    second = out["out_tokens"][sel, 1]
    obs2 = np.bincount(second, minlength=V)
    exp2 = pt[1] * sel.sum()
    m2 = exp2 > 0
    assert obs2[~m2].sum() == 0
    chi2b = ((obs2[m2] - exp2[m2]) ** 2 / exp2[m2]).sum()
    assert stats.chi2.sf(chi2b, m2.sum() - 1) > 1e-4
    # Closed forms: alpha_n = sum_v min(p_t, p_d) at row n-1; P(j >= n) = prod alpha.
    alpha = np.minimum(pt[:K], pdf.astype(np.float64)).sum(-1)
    acc1 = (out["num_accepted"] >= 1).mean()
    sd = math.sqrt(alpha[0] * (1 - alpha[0]) / N)
    assert abs(acc1 - alpha[0]) < 4 * sd
    ej = sum(np.prod(alpha[:n]) for n in range(1, K + 1))
    js = out["num_accepted"].astype(np.float64)
    assert abs(js.mean() - ej) < 4 * js.std() / math.sqrt(N)


def test_argmax_rows_ties_and_margin(orc):
    x = np.array([[1.0, 3.0, 3.0, 2.0], [5.0, -1.0, 4.5, 5.0], [-np.inf, -2.0, -3.0, -2.5]],
                 np.float32)
    idx, mg = orc.argmax(x)
    assert list(idx) == [1, 0, 1]
    assert list(mg) == [0.0, 0.0, 0.5]

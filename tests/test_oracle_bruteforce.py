"""Brute-force pin: one verify step equals K+1 sequential greedy decode steps.

A toy one-layer attention language model (each token's query/key/value rows
are embedding rows; the output layer is a vocab x hidden matrix) is decoded
one token at a time with plain numpy (one query, softmax over every cached
key).  The oracle's verify path -- append, causal attention over the paged
cache, LM head, greedy acceptance, rollback -- must emit exactly the
sequential tokens for every accepted length j, and leave the cache equal to
the sequential cache.  This pins the causal diagonal, the row-(n-1)-judges-
draft-n convention, the final-token choice and the rollback length.
"""
import numpy as np
import pytest

V, HQ, HKV, D, PS = 1024, 4, 4, 64, 64
HIDDEN = HQ * D


class ToyLM:
    def __init__(self, seed):
        rng = np.random.default_rng(seed)
        self.Eq = rng.standard_normal((V, HQ, D)).astype(np.float32)
        self.Ek = rng.standard_normal((V, HKV, D)).astype(np.float32)
        self.Ev = rng.standard_normal((V, HKV, D)).astype(np.float32)
        self.W = (rng.standard_normal((V, HIDDEN)) * 0.5).astype(np.float32)

    def step(self, ks, vs, tok):
        """Sequential decode of one token: append its k/v, attend, project."""
        ks.append(self.Ek[tok].astype(np.float64))
        vs.append(self.Ev[tok].astype(np.float64))
        K_ = np.stack(ks)          # [n, HKV, D]
        V_ = np.stack(vs)
        q = self.Eq[tok].astype(np.float64)
        o = np.zeros((HQ, D))
        for h in range(HQ):
            kv = h * HKV // HQ
            s = K_[:, kv] @ q[h] / np.sqrt(D)
            w = np.exp(s - s.max())
            o[h] = (w[:, None] * V_[:, kv]).sum(0) / w.sum()
        logits = self.W.astype(np.float64) @ o.reshape(-1)
        return int(np.argmax(logits))


@pytest.mark.parametrize("j_target", [0, 1, 2, 3])
def test_verify_equals_sequential_greedy(orc, j_target):
    K = 3
    lm = ToyLM(100 + j_target)
    rng = np.random.default_rng(200 + j_target)
    L = 62  # the K+1 new positions 62..65 straddle a page boundary
    prompt = rng.integers(0, V, L)
    ks, vs = [], []
    for t in prompt:
        ks.append(lm.Ek[t].astype(np.float64))
        vs.append(lm.Ev[t].astype(np.float64))
    root = int(rng.integers(0, V))
    # Sequential greedy continuation from the root: K+1 steps.
    ks_seq, vs_seq = list(ks), list(vs)
    seq_tokens = []
    tok = root
    for _ in range(K + 1):
        tok = lm.step(ks_seq, vs_seq, tok)
        seq_tokens.append(tok)
    # Drafts: follow the sequential tokens for j_target positions, then diverge.
    drafts = []
    for n in range(K):
        if n < j_target:
            drafts.append(seq_tokens[n])
        elif n == j_target:
            drafts.append((seq_tokens[n] + 1) % V)
        else:
            drafts.append(int(rng.integers(0, V)))
    chain = [root] + drafts
    # Paged cache with a shuffled page table; prompt written at positions 0..L-1.
    n_pages = (L + K + 1 + PS - 1) // PS + 1
    perm = rng.permutation(n_pages + 2).astype(np.int32)
    table = perm[:n_pages].reshape(1, n_pages)
    P = n_pages + 2
    kc = np.full((P, HKV, PS, D), 7.0, np.float32)
    vc = np.full((P, HKV, PS, D), 7.0, np.float32)
    for p, t in enumerate(prompt):
        kc[table[0, p // PS], :, p % PS] = lm.Ek[t]
        vc[table[0, p // PS], :, p % PS] = lm.Ev[t]
    seq = np.array([L], np.int32)
    q = lm.Eq[chain][None]                     # [1, K+1, HQ, D]
    kn = lm.Ek[chain][None]
    vn = lm.Ev[chain][None]
    orc.kv_append(seq, table, P, kn, vn, kc, vc)
    o = orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=HKV, d_v=D)
    Hrows = o.reshape(K + 1, HIDDEN)
    logits = orc.lm_head(Hrows, lm.W.astype(np.float64))
    out = orc.accept(logits[None], np.array([drafts], np.int32), np.zeros(1, np.float32),
                     np.ones(1, np.float32), None, np.zeros((1, K + 1), np.float32),
                     np.zeros((1, K + 1), np.float32))
    j = int(out["num_accepted"][0])
    assert j == j_target
    emitted = list(out["out_tokens"][0, : j + 1])
    assert emitted == seq_tokens[: j + 1]
    rb = orc.kv_rollback(table, out["num_accepted"], seq, K, poison=True, k_cache=kc,
                         v_cache=vc, n_kv_heads=HKV, d_k=D, d_v=D)
    new_len = int(rb["seq_lens"][0])
    assert new_len == L + j + 1
    # Kept cache == sequential cache over the kept positions (root + accepted).
    for p in range(new_len):
        assert np.array_equal(kc[table[0, p // PS], :, p % PS].astype(np.float64), ks_seq[p])
        assert np.array_equal(vc[table[0, p // PS], :, p % PS].astype(np.float64), vs_seq[p])
    for p in range(new_len, L + K + 1):
        assert not kc[table[0, p // PS], :, p % PS].any()

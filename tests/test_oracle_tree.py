"""Pins of the oracle's tree verification (CPU only).

The pages name tree drafting only as the next step after chains ([TRT-MTP]
"工作展望", Fig. 9, an image: full or dynamic trees widen the candidate
set).  The oracle's reading: nodes in topological order (node 0 the root,
parent[i] < i); node i attends to the cache and to its ancestors and itself;
greedy verification walks down from the root taking, at each accepted node,
its first child whose draft equals that node's argmax; rollback gathers the
accepted path's rows to contiguous slots.  These tests pin it against the
already-pinned chain path (a chain is a tree), against causal attention over
each node's root path, and against brute-force sequential greedy decoding of
a toy language model.
"""
import numpy as np
import pytest

from test_oracle_bruteforce import ToyLM, V as TV, HQ as THQ, HKV as THKV, D as TD, PS as TPS, \
    HIDDEN as THIDDEN


def _pages(B, Q, L, ps=64, seed=0):
    need = (int(np.max(L)) + Q + ps - 1) // ps
    rng = np.random.default_rng(seed)
    perm = rng.permutation(B * need).astype(np.int32)
    return perm.reshape(B, need), B * need


def _rand_tree(rng, Q):
    par = np.full(Q, -1, np.int32)
    for i in range(1, Q):
        par[i] = rng.integers(0, i)
    return par


def _gqa(rng, B, Q, Hq, Hkv, d, L):
    table, P = _pages(B, Q, L, seed=int(rng.integers(1 << 30)))
    kc = rng.standard_normal((P, Hkv, 64, d)).astype(np.float32)
    vc = rng.standard_normal((P, Hkv, 64, d)).astype(np.float32)
    q = rng.standard_normal((B, Q, Hq, d)).astype(np.float32)
    kn = rng.standard_normal((B, Q, Hkv, d)).astype(np.float32)
    vn = rng.standard_normal((B, Q, Hkv, d)).astype(np.float32)
    return table, P, kc, vc, q, kn, vn


def test_chain_shaped_tree_equals_chain(orc):
    rng = np.random.default_rng(1)
    B, Q, Hq, Hkv, d = 3, 5, 4, 2, 16
    L = np.array([0, 70, 129], np.int32)
    table, P, kc, vc, q, kn, vn = _gqa(rng, B, Q, Hq, Hkv, d, L)
    orc.kv_append(L, table, P, kn, vn, kc, vc)
    chain = np.tile(np.arange(-1, Q - 1, dtype=np.int32), (B, 1))
    o_tree = orc.verify_attn(q, kc, vc, table, L, P, n_kv_heads=Hkv, d_v=d, tree_parent=chain)
    o_chain = orc.verify_attn(q, kc, vc, table, L, P, n_kv_heads=Hkv, d_v=d)
    assert np.array_equal(o_tree, o_chain)
    # greedy acceptance: identical outputs, path 0..j
    Vv = 50
    logits = rng.standard_normal((B, Q, Vv))
    t, _ = orc.argmax(logits)
    drafts = np.array([[t[0, 0], t[0, 1], 7, 8], [t[1, 0], 3, 4, 5], [9, 9, 9, 9]], np.int32)
    drafts[1, 1] = (t[1, 1] + 1) % Vv
    z = np.zeros((B, Q), np.float32)
    a = orc.accept(logits, drafts, np.zeros(B, np.float32), None, None, z, z)
    c = orc.accept(logits, drafts, np.zeros(B, np.float32), None, None, z, z, tree_parent=chain)
    for k in ("num_accepted", "out_tokens", "next_token", "out_offsets", "packed"):
        assert np.array_equal(a[k], c[k]), k
    for bb in range(B):
        j = a["num_accepted"][bb]
        assert list(c["accepted_nodes"][bb]) == list(range(j + 1)) + [-1] * (Q - 1 - j)
        assert list(a["accepted_nodes"][bb]) == list(range(j + 1)) + [-1] * (Q - 1 - j)


def test_tree_attention_equals_causal_attention_over_the_root_path(orc):
    """Node i's output equals the last query of a chain problem whose new
    positions are the root path of i, over the same cached keys."""
    rng = np.random.default_rng(2)
    B, Q, Hq, Hkv, d = 2, 9, 6, 3, 8
    L = np.array([37, 100], np.int32)
    table, P, kc, vc, q, kn, vn = _gqa(rng, B, Q, Hq, Hkv, d, L)
    par = np.stack([_rand_tree(rng, Q) for _ in range(B)])
    kc0, vc0 = kc.copy(), vc.copy()
    orc.kv_append(L, table, P, kn, vn, kc, vc)
    o_tree = orc.verify_attn(q, kc, vc, table, L, P, n_kv_heads=Hkv, d_v=d, tree_parent=par)
    for b in range(B):
        for i in range(Q):
            path = []
            a = i
            while a >= 0:
                path.append(a)
                a = par[b, a]
            path = path[::-1]
            n = len(path)
            kc1, vc1 = kc0.copy(), vc0.copy()
            t1 = table[b:b + 1]
            L1 = L[b:b + 1]
            orc.kv_append(L1, t1, P, kn[b:b + 1, path], vn[b:b + 1, path], kc1, vc1)
            o1 = orc.verify_attn(q[b:b + 1, path], kc1, vc1, t1, L1, P, n_kv_heads=Hkv, d_v=d)
            assert np.array_equal(o_tree[b, i], o1[0, n - 1]), (b, i, path)


def test_tree_attention_rejects_malformed_trees(orc):
    rng = np.random.default_rng(3)
    B, Q, Hq, Hkv, d = 1, 4, 2, 1, 8
    L = np.array([5], np.int32)
    table, P, kc, vc, q, kn, vn = _gqa(rng, B, Q, Hq, Hkv, d, L)
    for bad in ([0, 0, 1, 2], [-1, 1, 1, 2], [-1, 0, 3, 1], [-1, -1, 0, 0]):
        with pytest.raises(ValueError):
            orc.verify_attn(q, kc, vc, table, L, P, n_kv_heads=Hkv, d_v=d,
                            tree_parent=np.array([bad], np.int32))


def test_tree_acceptance_hand_example(orc):
    """parent = [-1, 0, 0, 1, 2], drafts of nodes 1..4 = 1, 2, 3, 4.  Row 0's
    argmax is 2: node 1 (token 1) does not match, node 2 does; row 2's argmax
    is 4: node 4; row 4's argmax 5 is the final token."""
    Vv = 8
    logits = np.zeros((1, 5, Vv))
    for row, tok in ((0, 2), (1, 3), (2, 4), (3, 6), (4, 5)):
        logits[0, row, tok] = 3.0
    drafts = np.array([[1, 2, 3, 4]], np.int32)
    par = np.array([[-1, 0, 0, 1, 2]], np.int32)
    z = np.zeros((1, 5), np.float32)
    out = orc.accept(logits, drafts, np.zeros(1, np.float32), None, None, z, z, tree_parent=par)
    assert out["num_accepted"][0] == 2
    assert list(out["out_tokens"][0]) == [2, 4, 5, -1, -1]
    assert list(out["accepted_nodes"][0]) == [0, 2, 4, -1, -1]
    assert out["next_token"][0] == 5
    assert list(out["packed"][:3]) == [2, 4, 5]
    # Duplicate sibling tokens: nodes 1 and 2 both carry row 0's argmax 2.
    # Through node 1 the path ends there (row 1's argmax is 3, its child
    # node 4 carries 4); through node 2 it goes on to node 3 (row 2's argmax
    # 4).  The longest accepted path 0-2-3 is kept, not the first match 0-1.
    par2 = np.array([[-1, 0, 0, 2, 1]], np.int32)
    drafts2 = np.array([[2, 2, 4, 4]], np.int32)
    out = orc.accept(logits, drafts2, np.zeros(1, np.float32), None, None, z, z, tree_parent=par2)
    assert out["num_accepted"][0] == 2
    assert list(out["accepted_nodes"][0]) == [0, 2, 3, -1, -1]
    assert list(out["out_tokens"][0]) == [2, 4, 6, -1, -1]
    assert out["next_token"][0] == 6
    # Two accepted paths of equal length (0-1-3 and 0-2-4): the one ending at
    # the smaller node index is kept; its final token is row 3's argmax.
    par3 = np.array([[-1, 0, 0, 1, 2]], np.int32)
    drafts3 = np.array([[2, 2, 3, 4]], np.int32)
    out = orc.accept(logits, drafts3, np.zeros(1, np.float32), None, None, z, z, tree_parent=par3)
    assert out["num_accepted"][0] == 2
    assert list(out["accepted_nodes"][0]) == [0, 1, 3, -1, -1]
    assert list(out["out_tokens"][0]) == [2, 3, 6, -1, -1]
    # A deeper path behind a later sibling beats a shallower one that ends
    # at a smaller index: node 2's subtree reaches depth 2 while node 1 is a
    # leaf.
    par4 = np.array([[-1, 0, 0, 2, 0]], np.int32)
    drafts4 = np.array([[2, 2, 4, 2]], np.int32)
    out = orc.accept(logits, drafts4, np.zeros(1, np.float32), None, None, z, z, tree_parent=par4)
    assert list(out["accepted_nodes"][0]) == [0, 2, 3, -1, -1]
    # A matching node under a rejected parent is not accepted: node 3
    # (token 4 = row 2's argmax) hangs under node 2, whose draft 7 fails.
    drafts5 = np.array([[2, 7, 4, 4]], np.int32)
    out = orc.accept(logits, drafts5, np.zeros(1, np.float32), None, None, z, z, tree_parent=par2)
    assert list(out["accepted_nodes"][0]) == [0, 1, -1, -1, -1]
    assert list(out["out_tokens"][0]) == [2, 3, -1, -1, -1]
    # a negative draft marks an unused node: it is never accepted
    out = orc.accept(logits, np.array([[1, -1, 3, 4]], np.int32), np.zeros(1, np.float32), None,
                     None, z, z, tree_parent=par)
    assert out["num_accepted"][0] == 0 and out["out_tokens"][0, 0] == 2


def test_tree_acceptance_invalid_requests(orc):
    Vv = 8
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((4, 4, Vv))
    drafts = np.zeros((4, 3), np.int32)
    par = np.array([[-1, 0, 0, 1], [-1, 0, 2, 1], [-1, 0, 0, 1], [-1, 0, 0, 1]], np.int32)
    temp = np.array([0, 0, 0.8, 0], np.float32)
    pd = np.full((4, 3, Vv), 1.0 / Vv, np.float32)
    rk = np.array([0, 0, 0, 5], np.int32)
    rd = np.full(4, 0.1, np.float32)
    z = np.zeros((4, 4), np.float32)
    out = orc.accept(logits, drafts, temp, None, pd, z, z, relaxed_topk=rk, relaxed_delta=rd,
                     tree_parent=par)
    # request 1: malformed tree; 2: sampled; 3: relaxed -- all invalid
    assert list(out["num_accepted"][1:]) == [-1, -1, -1]
    assert out["num_accepted"][0] >= 0
    assert (out["accepted_nodes"][1:] == -1).all()


def test_rollback_gathers_the_accepted_path(orc):
    """Path [0, 2, 3] of a 4-node step: slot L+1 <- node 2 and slot L+2 <-
    node 3 (node 2's slot is read before it is overwritten); slot L+3 is
    rejected."""
    K, Hkv, d = 3, 2, 4
    L = np.array([62], np.int32)  # the step straddles a page boundary
    table = np.array([[3, 0, 2]], np.int32)
    P = 4
    kc = np.zeros((P, Hkv, 64, d), np.float32)
    vc = np.zeros((P, Hkv, 64, d), np.float32)

    def slot(p):
        return table[0, p // 64], p % 64

    for a in range(K + 1):
        pg, off = slot(62 + a)
        kc[pg, :, off] = 10 + a
        vc[pg, :, off] = 20 + a
    out = orc.kv_rollback(table, np.array([2], np.int32), L, K, poison=True, k_cache=kc,
                          v_cache=vc, n_kv_heads=Hkv, d_k=d, d_v=d,
                          accepted_nodes=np.array([[0, 2, 3, -1]], np.int32))
    assert out["seq_lens"][0] == 65 and out["n_bad"] == 0
    def row(arr, p):
        pg, off = slot(p)
        return arr[pg, :, off]

    assert [row(kc, 62 + t)[0, 0] for t in range(4)] == [10, 12, 13, 0]
    assert [row(vc, 62 + t)[1, 3] for t in range(4)] == [20, 22, 23, 0]
    # a path that is not increasing counts as an invalid count: nothing kept
    kc2 = kc.copy()
    out = orc.kv_rollback(table, np.array([2], np.int32), L, K, k_cache=kc2, v_cache=vc.copy(),
                          n_kv_heads=Hkv, d_k=d, d_v=d,
                          accepted_nodes=np.array([[0, 3, 2, -1]], np.int32))
    assert out["seq_lens"][0] == 62 and out["n_bad"] == 1
    assert np.array_equal(kc2, kc)


@pytest.mark.parametrize("k_target", [0, 1, 2, 3])
def test_tree_verify_equals_sequential_greedy(orc, k_target):
    """A toy one-layer LM decoded greedily one token at a time gives g1..g4
    from the root.  The tree holds the greedy path to depth k_target, each
    path node placed after a distractor sibling (and the node at depth
    k_target has distractor children only).  Append + tree attention + LM
    head + tree acceptance must accept exactly that path and emit g1..g(k+1);
    the rollback gather must leave the sequential cache in the kept slots."""
    lm = ToyLM(300 + k_target)
    rng = np.random.default_rng(400 + k_target)
    L = 60
    prompt = rng.integers(0, TV, L)
    ks, vs = [], []
    for t in prompt:
        ks.append(lm.Ek[t].astype(np.float64))
        vs.append(lm.Ev[t].astype(np.float64))
    root = int(rng.integers(0, TV))
    ks_seq, vs_seq = list(ks), list(vs)
    greedy, tok = [], root
    for _ in range(4):
        tok = lm.step(ks_seq, vs_seq, tok)
        greedy.append(tok)
    # Build the tree: tokens[node], parent[node].
    tokens, parent = [root], [-1]
    cur, path = 0, [0]
    for depth in range(k_target + 1):
        wrong = (greedy[depth] + 1 + int(rng.integers(0, TV - 1))) % TV
        if wrong == greedy[depth]:
            wrong = (wrong + 1) % TV
        tokens.append(wrong)
        parent.append(cur)               # distractor sibling first
        if depth < k_target:
            tokens.append(greedy[depth])
            parent.append(cur)
            cur = len(tokens) - 1
            path.append(cur)
    # one more unrelated leaf hanging off the root
    tokens.append(int(rng.integers(0, TV)))
    parent.append(0)
    Q = len(tokens)
    K = Q - 1
    par = np.array([parent], np.int32)
    # Paged cache, shuffled pages; prompt at 0..L-1; the step straddles a page.
    n_pages = (L + Q + TPS - 1) // TPS + 1
    table = rng.permutation(n_pages + 1).astype(np.int32)[:n_pages].reshape(1, n_pages)
    P = n_pages + 1
    kc = np.full((P, THKV, TPS, TD), 7.0, np.float32)
    vc = np.full((P, THKV, TPS, TD), 7.0, np.float32)
    for p, t in enumerate(prompt):
        kc[table[0, p // TPS], :, p % TPS] = lm.Ek[t]
        vc[table[0, p // TPS], :, p % TPS] = lm.Ev[t]
    seq = np.array([L], np.int32)
    q = lm.Eq[tokens][None]
    orc.kv_append(seq, table, P, lm.Ek[tokens][None], lm.Ev[tokens][None], kc, vc)
    o = orc.verify_attn(q, kc, vc, table, seq, P, n_kv_heads=THKV, d_v=TD, tree_parent=par)
    logits = orc.lm_head(o.reshape(Q, THIDDEN), lm.W.astype(np.float64))
    z = np.zeros((1, Q), np.float32)
    out = orc.accept(logits[None], np.array([tokens[1:]], np.int32), np.zeros(1, np.float32),
                     None, None, z, z, tree_parent=par)
    j = int(out["num_accepted"][0])
    assert j == k_target
    assert list(out["accepted_nodes"][0, : j + 1]) == path
    assert list(out["out_tokens"][0, : j + 1]) == greedy[: j + 1]
    rb = orc.kv_rollback(table, out["num_accepted"], seq, K, poison=True, k_cache=kc,
                         v_cache=vc, n_kv_heads=THKV, d_k=TD, d_v=TD,
                         accepted_nodes=out["accepted_nodes"])
    new_len = int(rb["seq_lens"][0])
    assert new_len == L + j + 1
    for p in range(new_len):
        assert np.array_equal(kc[table[0, p // TPS], :, p % TPS].astype(np.float64), ks_seq[p])
        assert np.array_equal(vc[table[0, p // TPS], :, p % TPS].astype(np.float64), vs_seq[p])
    for p in range(new_len, L + Q):
        assert not kc[table[0, p // TPS], :, p % TPS].any()

"""GPU parity of tree verification against the fp64 oracle: tree-masked verify
attention (bf16 and E4M3 caches, float32 path), greedy tree acceptance with
the accepted node path, and the rollback gather of the path's rows.
Tolerances: see tests/parity.py (attention rows within 2e-3 of the row's
largest magnitude; integers and cache bytes bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
import sdsynth
import speculative_decoding_sd_amd as sdv
from parity import DEV, bits, host, check_attention

pytestmark = pytest.mark.gpu


def _rand_trees(rng, B, Q, chainy=0.3):
    par = np.full((B, Q), -1, np.int32)
    for b in range(B):
        for i in range(1, Q):
            par[b, i] = i - 1 if rng.random() < chainy else rng.integers(0, i)
    return par


def _case(B, K, Hq, Hkv, D, lens, seed, kv, dtype="bf16"):
    cfg = sdsynth.Config(name="case", batch=B, K=K, n_q_heads=Hq, n_kv_heads=Hkv, d_qk=D,
                         d_v=D, mla=False, hidden=Hq * D, vocab=8, dtype=dtype, seq_len=None,
                         kv_cache=kv)
    return sdsynth.make_workload(cfg, seed, device="cpu", seq_lens=np.array(lens),
                                 with_lm_head=False)


def _run_attention(wl, par, max_seq_len=None):
    t = wl.tensors
    q, kc, vc = t["q"].to(DEV), t["k_cache"].to(DEV), t["v_cache"].to(DEV)
    pt = torch.tensor(wl.page_table, device=DEV)
    sl = torch.tensor(wl.seq_lens, device=DEV)
    B, Q, Hq, D = q.shape
    out = torch.full((B, Q, Hq, D), -5.0, dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    tp = torch.tensor(par, device=DEV)
    ks = t["k_scale"].to(DEV) if "k_scale" in t else None
    vs = t["v_scale"].to(DEV) if "v_scale" in t else None
    d = sdv.attn_desc(q=q, k_cache=kc, v_cache=vc, page_table=pt, seq_lens=sl, out=out,
                      n_kv_heads=wl.cfg.n_kv_heads, num_pages=wl.num_pages,
                      max_seq_len=int(max_seq_len or wl.seq_lens.max()),
                      k_new=t["k_new"].to(DEV), v_new=t["v_new"].to(DEV), dev_error=err,
                      k_scale=ks, v_scale=vs, tree_parent=tp)
    sdv.verify_attn(d)
    torch.cuda.synchronize()
    return out.cpu().numpy(), kc, vc, int(err.item())


def _oracle_attention(wl, par):
    t = wl.tensors
    kc, vc = host(t["k_cache"]).copy(), host(t["v_cache"]).copy()
    kw = {}
    if "k_scale" in t:
        kw = dict(k_scale=t["k_scale"].numpy(), v_scale=t["v_scale"].numpy())
    oracle.kv_append(wl.seq_lens, wl.page_table, wl.num_pages, host(t["k_new"]),
                     host(t["v_new"]), kc, vc, **kw)
    ref = oracle.verify_attn(host(t["q"]), kc, vc, wl.page_table, wl.seq_lens, wl.num_pages,
                             n_kv_heads=wl.cfg.n_kv_heads, d_v=wl.cfg.d_v, tree_parent=par, **kw)
    return ref, kc, vc


@pytest.mark.parametrize("kv,dtype,B,K,Hq,Hkv,D,lens", [
    ("as_dtype", "bf16", 4, 7, 16, 4, 128, [0, 61, 1300, 700]),   # 32 rows per kv head
    ("as_dtype", "bf16", 2, 9, 20, 4, 64, [5, 2000]),             # 50 rows: two row blocks
    ("e4m3", "bf16", 4, 7, 16, 4, 128, [3, 64, 999, 4100]),
    ("e4m3", "bf16", 3, 15, 8, 2, 128, [10, 127, 3000]),          # 16 nodes, 64 rows
    ("e4m3", "bf16", 3, 11, 12, 4, 128, [5, 400, 2100]),          # 36 rows: 16-row blocks
    ("as_dtype", "f32", 2, 5, 4, 2, 64, [7, 130]),                # float32 path
    ("as_dtype", "bf16", 2, 63, 2, 2, 64, [17, 500]),             # 64 nodes: the largest tree
])
def test_tree_attention(kv, dtype, B, K, Hq, Hkv, D, lens):
    rng = np.random.default_rng(K * 10 + B)
    wl = _case(B, K, Hq, Hkv, D, lens, seed=50 + K, kv=kv, dtype=dtype)
    par = _rand_trees(rng, B, K + 1)
    out, kc, vc, err = _run_attention(wl, par)
    ref, kc_ref, vc_ref = _oracle_attention(wl, par)
    assert err == 0
    check_attention(out, ref, where=f"tree {kv} {dtype} {B},{K}")
    if kv == "e4m3":
        assert np.array_equal(kc.cpu().numpy(), kc_ref)
    elif dtype == "bf16":
        assert np.array_equal(bits(kc), kc_ref) and np.array_equal(bits(vc), vc_ref)


def test_tree_attention_malformed_tree_is_flagged():
    rng = np.random.default_rng(3)
    B, K, Hq, Hkv, D = 3, 4, 8, 2, 128
    wl = _case(B, K, Hq, Hkv, D, [40, 300, 90], seed=9, kv="as_dtype")
    par = _rand_trees(rng, B, K + 1)
    ref, _, _ = _oracle_attention(wl, par)
    bad = par.copy()
    bad[1, 3] = 3            # a node that is its own parent
    out, _, _, err = _run_attention(wl, bad)
    assert err & sdv.SD_DERR_TREE
    assert np.isnan(out[1]).all()
    check_attention(out[[0, 2]], ref[[0, 2]], where="valid requests beside a malformed tree")


def _run_accept(lg_t, drafts, temp, par, relaxed=None):
    B, Q, V = lg_t.shape
    i32 = dict(dtype=torch.int32, device=DEV)
    out = dict(num_accepted=torch.full((B,), -7, **i32), out_tokens=torch.full((B, Q), -7, **i32),
               next_token=torch.full((B,), -7, **i32), out_offsets=torch.full((B + 1,), -7, **i32),
               packed_tokens=torch.full((B * Q,), -7, **i32),
               accepted_nodes=torch.full((B, Q), -7, **i32))
    err = torch.zeros(1, **i32)
    z = torch.zeros((B, Q), dtype=torch.float32, device=DEV)
    rk = rd = None
    if relaxed is not None:
        rk = torch.tensor(relaxed[0], device=DEV)
        rd = torch.tensor(relaxed[1], device=DEV)
    pd = torch.full((B, Q - 1, V), 1.0 / V, dtype=torch.float32, device=DEV)
    d = sdv.accept_desc(logits=lg_t, draft_tokens=torch.tensor(drafts, device=DEV),
                        temperature=torch.tensor(temp, device=DEV), u_accept=z, u_sample=z,
                        draft_probs=pd, dev_error=err, relaxed_topk=rk, relaxed_delta=rd,
                        tree_parent=torch.tensor(par, device=DEV), **out)
    sdv.accept(d)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["dev_error"] = int(err.item())
    return res


@pytest.mark.parametrize("B,K,V,dtype", [(40, 7, 5000, "bf16"), (25, 15, 1031, "f32"),
                                         (8, 4, 129280, "bf16"), (6, 63, 3000, "bf16")])
def test_tree_accept_greedy(B, K, V, dtype):
    rng = np.random.default_rng(B + K)
    Q = K + 1
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    lg_t = (torch.randn((B, Q, V), generator=torch.Generator().manual_seed(B * K),
                        dtype=torch.float32) * 1.7).to(tdt).to(DEV)
    lg_h = host(lg_t)
    tmax, _ = oracle.argmax(lg_h.astype(np.float64) if dtype == "f32"
                            else oracle.bf16_to_f64(lg_h))
    par = _rand_trees(rng, B, Q, chainy=0.4)
    drafts = rng.integers(0, V, (B, K)).astype(np.int32)
    for b in range(B):        # most nodes carry their parent's argmax: long paths, ties of siblings
        for n in range(1, Q):
            if rng.random() < 0.7:
                drafts[b, n - 1] = tmax[b, par[b, n]]
        if b % 9 == 4:
            drafts[b, rng.integers(0, K)] = -1       # an unused node
    temp = np.zeros(B, np.float32)
    ref = oracle.accept(lg_h, drafts, temp, None, None, np.zeros((B, Q), np.float32),
                        np.zeros((B, Q), np.float32), tree_parent=par)
    gpu = _run_accept(lg_t, drafts, temp, par)
    assert gpu["dev_error"] == 0
    for k_g, k_r in (("num_accepted", "num_accepted"), ("out_tokens", "out_tokens"),
                     ("next_token", "next_token"), ("out_offsets", "out_offsets"),
                     ("packed_tokens", "packed"), ("accepted_nodes", "accepted_nodes")):
        assert np.array_equal(gpu[k_g], ref[k_r]), k_g
    assert ref["num_accepted"].max() >= 3        # the walk went deep somewhere
    # The batch holds requests where descending through the first matching
    # child would stop short of the longest accepted path.
    shorter = 0
    for b in range(B):
        cur, depth = 0, 0
        while True:
            nxt = [c for c in range(cur + 1, Q)
                   if par[b, c] == cur and drafts[b, c - 1] == tmax[b, cur]]
            if not nxt:
                break
            cur, depth = nxt[0], depth + 1
        shorter += depth < ref["num_accepted"][b]
    assert shorter > 0


def test_tree_accept_invalid_requests():
    rng = np.random.default_rng(5)
    B, K, V = 6, 4, 300
    Q = K + 1
    lg_t = torch.randn((B, Q, V), generator=torch.Generator().manual_seed(1)).to(DEV)
    par = _rand_trees(rng, B, Q)
    par[1, 2] = 2                                   # malformed
    temp = np.zeros(B, np.float32)
    temp[2] = 0.9                                   # sampled: not with a tree
    rk = np.zeros(B, np.int32)
    rk[3] = 5                                       # relaxed: not with a tree
    rd = np.full(B, 0.1, np.float32)
    drafts = rng.integers(0, V, (B, K)).astype(np.int32)
    gpu = _run_accept(lg_t, drafts, temp, par, relaxed=(rk, rd))
    ref = oracle.accept(lg_t.cpu().numpy(), drafts, temp, None,
                        np.full((B, K, V), 1.0 / V, np.float32), np.zeros((B, Q), np.float32),
                        np.zeros((B, Q), np.float32), relaxed_topk=rk, relaxed_delta=rd,
                        tree_parent=par)
    assert gpu["dev_error"] & sdv.SD_DERR_TREE
    assert list(gpu["num_accepted"][1:4]) == [-1, -1, -1]
    for k_g, k_r in (("num_accepted", "num_accepted"), ("out_tokens", "out_tokens"),
                     ("accepted_nodes", "accepted_nodes"), ("packed_tokens", "packed")):
        assert np.array_equal(gpu[k_g], ref[k_r]), k_g


@pytest.mark.parametrize("poison,kv", [(False, "as_dtype"), (True, "as_dtype"), (True, "e4m3")])
def test_tree_rollback_gather(poison, kv):
    rng = np.random.default_rng(7 + poison)
    B, K, Hkv, D = 30, 7, 2, 128
    Q = K + 1
    lens = rng.integers(0, 300, B).astype(np.int32)
    lens[:3] = [57, 64, 0]                          # steps straddling / starting a page
    wl = _case(B, K, 4, Hkv, D, lens, seed=13, kv=kv)
    par = _rand_trees(rng, B, Q)
    # Accepted paths of random depth down the tree (as sd_accept would return).
    paths = np.full((B, Q), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):
        cur, path = 0, [0]
        while rng.random() < 0.75:
            kids = [c for c in range(cur + 1, Q) if par[b, c] == cur]
            if not kids:
                break
            cur = int(rng.choice(kids))
            path.append(cur)
        paths[b, :len(path)] = path
        acc[b] = len(path) - 1
    acc[5] = -1
    paths[5] = -1                                   # an invalid request keeps nothing
    paths[6, 1:3] = [3, 2] if acc[6] >= 2 else paths[6, 1:3]   # possibly malformed
    i32 = dict(dtype=torch.int32, device=DEV)
    pt, sl, na = (torch.tensor(x, device=DEV) for x in (wl.page_table, lens, acc))
    slots = torch.full((B * Q,), -9, **i32)
    soff = torch.empty(B + 1, **i32)
    freed = torch.full((B * 2,), -9, **i32)
    foff = torch.empty(B + 1, **i32)
    err = torch.zeros(1, **i32)
    kc, vc = wl.tensors["k_cache"].to(DEV), wl.tensors["v_cache"].to(DEV)
    d = sdv.rollback_desc(page_table=pt, num_accepted=na, seq_lens=sl, K=K, rollback_slots=slots,
                          rollback_offsets=soff, freed_pages=freed, freed_offsets=foff,
                          poison=poison, k_cache=kc, v_cache=vc, n_kv_heads=Hkv, d_k=D, d_v=D,
                          num_pages=wl.num_pages, dev_error=err,
                          accepted_nodes=torch.tensor(paths, device=DEV))
    sdv.kv_rollback(d)
    torch.cuda.synchronize()
    to_np = (lambda t: t.numpy()) if kv == "e4m3" else host
    kch, vch = to_np(wl.tensors["k_cache"]).copy(), to_np(wl.tensors["v_cache"]).copy()
    ref = oracle.kv_rollback(wl.page_table, acc, lens, K, poison=poison, k_cache=kch, v_cache=vch,
                             n_kv_heads=Hkv, d_k=D, d_v=D, accepted_nodes=paths)
    assert np.array_equal(sl.cpu().numpy(), ref["seq_lens"])
    assert np.array_equal(slots.cpu().numpy(), ref["rb_slots"])
    assert np.array_equal(soff.cpu().numpy(), ref["rb_offsets"])
    assert np.array_equal(freed.cpu().numpy(), ref["freed"])
    got_k = kc.cpu().numpy() if kv == "e4m3" else bits(kc)
    got_v = vc.cpu().numpy() if kv == "e4m3" else bits(vc)
    assert np.array_equal(got_k, kch) and np.array_equal(got_v, vch)
    bad_path = ref["n_bad"] > 1
    assert bool(int(err.item()) & sdv.SD_DERR_TREE) == bad_path


def test_chained_tiny_fp32_tree_step():
    """The tiny fp32 configuration (B=1, 4 heads x 64, L=128) with its K=3
    drafts as a binary tree, through VerifyStep (tree attention -> LM head on
    the attention output -> tree acceptance -> rollback gather), against the
    oracle's chain of the same calls.  The kept cache rows must equal the
    oracle's gathered rows."""
    import dataclasses
    cfg = dataclasses.replace(sdsynth.CONFIGS[1], K=6)
    seed = sdsynth.config_seed(1)
    wl = sdsynth.make_workload(cfg, seed, device="cpu")
    t = wl.tensors
    Q = cfg.num_q
    par = np.tile(sdsynth.tree_parents("binary", Q), (cfg.batch, 1))
    ref_o, kc_ref, vc_ref = _oracle_attention(wl, par)
    exact = oracle.lm_head(ref_o.reshape(cfg.batch * Q, -1), t["W"].numpy().astype(np.float64))
    ref_logits = exact.reshape(cfg.batch, Q, cfg.vocab)
    tt, margin = oracle.argmax(ref_logits)
    drafts = sdsynth.tree_drafts(tt, par[0], cfg.vocab, seed, p_match=0.8)
    ref_acc = oracle.accept(ref_logits, drafts, wl.temperature, None, None, wl.u_accept,
                            wl.u_sample, tree_parent=par)
    ref_rb = oracle.kv_rollback(wl.page_table, ref_acc["num_accepted"], wl.seq_lens, cfg.K,
                                k_cache=kc_ref, v_cache=vc_ref, n_kv_heads=cfg.n_kv_heads,
                                d_k=cfg.d_qk, d_v=cfg.d_v, accepted_nodes=ref_acc["accepted_nodes"])
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
                          k_new=d["k_new"], v_new=d["v_new"],
                          tree_parent=torch.tensor(par, device=DEV))
    step.run()
    torch.cuda.synchronize()
    check_attention(step.out.cpu().numpy(), ref_o, where="tree attention")
    assert int(step.dev_error.item()) == 0
    assert margin.reshape(-1).min() >= 1e-3, "seeded case must not sit on an argmax tie"
    assert step.num_accepted.cpu().numpy().tolist() == ref_acc["num_accepted"].tolist()
    assert ref_acc["num_accepted"][0] >= 1
    assert np.array_equal(step.out_tokens.cpu().numpy(), ref_acc["out_tokens"])
    assert np.array_equal(step.accepted_nodes.cpu().numpy(), ref_acc["accepted_nodes"])
    assert np.array_equal(sl.cpu().numpy(), ref_rb["seq_lens"])
    # kept rows: the GPU's appended-and-gathered f32 rows equal the oracle's
    kc = d["k_cache"].cpu().numpy()
    L, new_len = int(wl.seq_lens[0]), int(ref_rb["seq_lens"][0])
    for p in range(L, new_len):
        pg, off = wl.page_table[0, p // 64], p % 64
        assert np.array_equal(kc[pg, :, off], kc_ref[pg, :, off]), p

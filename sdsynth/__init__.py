"""Seeded synthetic inputs for the speculative-decoding verify step.

This module is test and benchmark infrastructure shared by the HIP path's
tests, the benchmark and the CPU oracle's tests.  It produces *inputs* only:
query/key/value tensors, paged-cache layouts, LM-head operands, the uniforms
the acceptance rule consumes, and a stand-in for the draft model (its tokens
and its probability rows).  It holds none of the verify step's own
arithmetic: no attention, no LM-head product, no target softmax, no
acceptance decision, no rollback.  Those live in the oracle (C, fp64) and in
the HIP kernels, which share no code with each other or with this module.

Random numbers the verify step draws (the acceptance uniform per draft and the
sampling uniform per position) come from Philox4x32-10, the counter-based
generator of Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3" (SC'11), implemented here from that paper's definition.  Bulk
tensor data comes from torch's seeded generators (CPU or GPU); every tensor has
its own seed so a tensor can be regenerated alone.

Workload recipes follow the five configurations the build is measured on
(tiny fp32 greedy; GQA bf16 stochastic; MLA-shaped greedy; long-context top-p;
ragged paged serving batch).  The pages themselves measure on summarisation
prompts and unnamed datasets; these seeded shapes stand in for them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# ----------------------------------------------------------------------------
# Philox4x32-10 (Salmon et al., SC'11, section 3: the Philox round function,
# multipliers and Weyl key schedule).
# ----------------------------------------------------------------------------
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter: np.ndarray, key) -> np.ndarray:
    """Philox4x32 with 10 rounds over an array of 128-bit counters.

    counter: uint32 array [..., 4]; key: two 32-bit words.  Returns uint32
    [..., 4].  Each round multiplies words 0 and 2 by the two Philox
    multipliers, takes the 64-bit products apart into hi/lo halves, and mixes
    the hi halves with the other two words and the round key; the key is
    bumped by the two Weyl constants between rounds.
    """
    c = np.asarray(counter, dtype=np.uint32)
    c0 = c[..., 0].astype(np.uint64)
    c1 = c[..., 1].astype(np.uint64)
    c2 = c[..., 2].astype(np.uint64)
    c3 = c[..., 3].astype(np.uint64)
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    out = np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)
    return out


# Stream ids used in the counter's third word.
STREAM_ACCEPT = 0   # u_accept[b, n-1]: acceptance test of draft n
STREAM_SAMPLE = 1   # u_sample[b, i]: final-token draw from row i
STREAM_DRAFT = 2    # draft-model stand-in: sampling draft tokens
STREAM_GEOM = 3     # draft-model stand-in: greedy prefix length


def philox_uniforms(seed: int, rows: int, cols: int, stream: int) -> np.ndarray:
    """u[r, c] in [0, 1) as float32, from counter (r, c, stream, 0), key = seed.

    u = (x >> 8) * 2^-24 keeps 24 random bits, so every value is exactly
    representable in float32 and u < 1 always.
    """
    r = np.arange(rows, dtype=np.uint32)[:, None]
    cc = np.arange(cols, dtype=np.uint32)[None, :]
    ctr = np.zeros((rows, cols, 4), dtype=np.uint32)
    ctr[..., 0] = r
    ctr[..., 1] = cc
    ctr[..., 2] = np.uint32(stream)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    x = philox4x32_10(ctr, key)[..., 0]
    return ((x >> np.uint32(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


# ----------------------------------------------------------------------------
# Bulk tensors
# ----------------------------------------------------------------------------
_TAGS = {
    "q": 1, "k_new": 2, "v_new": 3, "k_cache": 4, "v_cache": 5, "H": 6, "W": 7,
    "pages": 8, "seq_lens": 9, "noise": 10, "modes": 11, "kv_new": 12, "kv_scale": 13,
}


def _generator(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 8) + _TAGS[tag])
    return g


def normal(shape, std: float, seed: int, tag: str, dtype, device) -> torch.Tensor:
    """N(0, std^2) tensor of `dtype`, drawn in float32 and rounded once."""
    dev = torch.device(device)
    g = _generator(seed, tag, dev)
    out = torch.empty(shape, dtype=dtype, device=dev)
    flat = out.view(-1)
    n = flat.numel()
    chunk = 1 << 28  # bound the float32 staging buffer
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        t = torch.randn(e - s, generator=g, dtype=torch.float32, device=dev)
        if std != 1.0:
            t.mul_(std)
        flat[s:e].copy_(t)
        del t
    return out


# ----------------------------------------------------------------------------
# Paged cache layout
# ----------------------------------------------------------------------------
def paged_layout(seq_lens: np.ndarray, num_q: int, page_size: int, extra_tokens: int,
                 seed: int, spare_pages: int = 0):
    """Page table for requests of length L_b that must hold L_b + num_q +
    extra_tokens positions.  Physical pages are a seeded permutation of the
    pool, so logical order never matches physical order.  Unused table
    entries are -1.  Returns (page_table int32 [B, max_pages], num_pages)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    need = (seq_lens + num_q + extra_tokens + page_size - 1) // page_size
    max_pages = int(need.max()) if len(need) else 1
    total = int(need.sum()) + spare_pages
    rng = np.random.default_rng(seed * 7919 + _TAGS["pages"])
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((len(seq_lens), max(max_pages, 1)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += int(n)
    return table, total


# ----------------------------------------------------------------------------
# Workload configurations
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Config:
    name: str
    batch: int
    K: int                      # drafts per request; num_q = K + 1
    n_q_heads: int
    n_kv_heads: int
    d_qk: int
    d_v: int
    mla: bool
    hidden: int
    vocab: int
    dtype: str                  # "f32" or "bf16"
    seq_len: Optional[int]      # fixed KV length, or None for ragged
    seq_len_range: Optional[tuple] = None
    temperature: float = 0.0    # 0 -> greedy
    top_p: float = 1.0
    mixed_modes: Optional[float] = None  # odd b stochastic at this T, even b greedy
    chain_attn_to_lm_head: bool = False  # LM-head input = attention output
    page_size: int = 64
    draft_noise: float = 0.5
    geom_p: float = 0.4
    kv_cache: str = "as_dtype"  # or "e4m3": FP8 cache codes with per-kv-head scales

    @property
    def num_q(self) -> int:
        return self.K + 1


CONFIGS = {
    1: Config("tiny-fp32-greedy", batch=1, K=3, n_q_heads=4, n_kv_heads=4, d_qk=64,
              d_v=64, mla=False, hidden=256, vocab=1024, dtype="f32", seq_len=128,
              chain_attn_to_lm_head=True),
    2: Config("gqa-bf16-stochastic", batch=32, K=5, n_q_heads=32, n_kv_heads=8,
              d_qk=128, d_v=128, mla=False, hidden=4096, vocab=32000, dtype="bf16",
              seq_len=2048, temperature=1.0),
    3: Config("mla-greedy-mtp-eagle", batch=64, K=3, n_q_heads=128, n_kv_heads=1,
              d_qk=576, d_v=512, mla=True, hidden=7168, vocab=129280, dtype="bf16",
              seq_len=8192),
    4: Config("long-context-topp", batch=8, K=7, n_q_heads=40, n_kv_heads=8, d_qk=128,
              d_v=128, mla=False, hidden=5120, vocab=152064, dtype="bf16",
              seq_len=131072, temperature=0.7, top_p=0.95),
    5: Config("ragged-paged-serving", batch=256, K=4, n_q_heads=32, n_kv_heads=8,
              d_qk=128, d_v=128, mla=False, hidden=7168, vocab=129280, dtype="bf16",
              seq_len=None, seq_len_range=(512, 16384), mixed_modes=0.8),
}


def config_seed(index: int) -> int:
    return 1000 + index


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def seq_lens_for(cfg: Config, seed: int) -> np.ndarray:
    if cfg.seq_len is not None:
        return np.full(cfg.batch, cfg.seq_len, dtype=np.int32)
    lo, hi = cfg.seq_len_range
    rng = np.random.default_rng(seed * 7919 + _TAGS["seq_lens"])
    return rng.integers(lo, hi + 1, size=cfg.batch).astype(np.int32)


def sampling_params(cfg: Config):
    """Per-request temperature and top-p (float32 [B])."""
    temp = np.full(cfg.batch, cfg.temperature, dtype=np.float32)
    if cfg.mixed_modes is not None:
        temp[:] = 0.0
        temp[1::2] = cfg.mixed_modes
    top_p = np.full(cfg.batch, cfg.top_p, dtype=np.float32)
    return temp, top_p


@dataclasses.dataclass
class Workload:
    cfg: Config
    seed: int
    seq_lens: np.ndarray        # int32 [B], L_b before the step
    page_table: np.ndarray      # int32 [B, max_pages]
    num_pages: int
    tensors: dict               # torch tensors on `device`
    temperature: np.ndarray
    top_p: np.ndarray
    u_accept: np.ndarray        # float32 [B, K+1]
    u_sample: np.ndarray        # float32 [B, K+1]


def make_workload(cfg: Config, seed: int, device="cpu", extra_tokens: int = 0,
                  batch: Optional[int] = None, seq_lens: Optional[np.ndarray] = None,
                  with_lm_head: bool = True, with_attention: bool = True) -> Workload:
    """Every input of one verify step except the drafts (which depend on the
    target logits; see `greedy_drafts` / `draft_probs` / `sample_drafts`)."""
    if batch is not None:
        cfg = dataclasses.replace(cfg, batch=batch)
    B, Q = cfg.batch, cfg.num_q
    if seq_lens is None:
        seq_lens = seq_lens_for(cfg, seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    table, num_pages = paged_layout(seq_lens, Q, cfg.page_size, extra_tokens, seed)
    dt = torch_dtype(cfg.dtype)
    t = {}
    if with_attention:
        t["q"] = normal((B, Q, cfg.n_q_heads, cfg.d_qk), 1.0, seed, "q", dt, device)
        if cfg.mla:
            t["k_new"] = normal((B, Q, cfg.d_qk), 1.0, seed, "kv_new", dt, device)
            t["v_new"] = None
            t["k_cache"] = normal((num_pages, cfg.page_size, cfg.d_qk), 1.0, seed,
                                  "k_cache", dt, device)
            t["v_cache"] = None
        else:
            t["k_new"] = normal((B, Q, cfg.n_kv_heads, cfg.d_qk), 1.0, seed, "k_new", dt, device)
            t["v_new"] = normal((B, Q, cfg.n_kv_heads, cfg.d_v), 1.0, seed, "v_new", dt, device)
            if cfg.kv_cache == "e4m3":
                # Codes: torch's float8_e4m3fn cast of N(0, 32^2) draws, stored as
                # bytes; scales ~1/32 per kv head, so the cached values are
                # roughly N(0, 1) like the bf16 cache.
                f8 = torch.float8_e4m3fn
                t["k_cache"] = normal((num_pages, cfg.n_kv_heads, cfg.page_size, cfg.d_qk), 32.0,
                                      seed, "k_cache", f8, device).view(torch.uint8)
                t["v_cache"] = normal((num_pages, cfg.n_kv_heads, cfg.page_size, cfg.d_v), 32.0,
                                      seed, "v_cache", f8, device).view(torch.uint8)
                rng = np.random.default_rng(seed * 7919 + _TAGS["kv_scale"])
                sc = ((0.75 + 0.5 * rng.random((2, cfg.n_kv_heads))) / 32.0).astype(np.float32)
                t["k_scale"] = torch.from_numpy(sc[0].copy()).to(device)
                t["v_scale"] = torch.from_numpy(sc[1].copy()).to(device)
            elif cfg.kv_cache == "as_dtype":
                t["k_cache"] = normal((num_pages, cfg.n_kv_heads, cfg.page_size, cfg.d_qk), 1.0,
                                      seed, "k_cache", dt, device)
                t["v_cache"] = normal((num_pages, cfg.n_kv_heads, cfg.page_size, cfg.d_v), 1.0,
                                      seed, "v_cache", dt, device)
            else:
                raise ValueError(f"unknown kv_cache {cfg.kv_cache!r}")
    if with_lm_head:
        if not cfg.chain_attn_to_lm_head:
            # Stand-in for the normalised hidden state that feeds the output layer.
            t["H"] = normal((B * Q, cfg.hidden), 1.0, seed, "H", dt, device)
        t["W"] = normal((cfg.vocab, cfg.hidden), 0.02, seed, "W", dt, device)
    temp, top_p = sampling_params(cfg)
    ua = philox_uniforms(seed, B, Q, STREAM_ACCEPT)
    us = philox_uniforms(seed, B, Q, STREAM_SAMPLE)
    return Workload(cfg, seed, seq_lens, table, num_pages, t, temp, top_p, ua, us)


# ----------------------------------------------------------------------------
# Draft-model stand-in.  The verify step receives draft tokens and the draft
# model's probability rows as inputs; these helpers synthesise them.
# ----------------------------------------------------------------------------
def truncated_geometric(seed: int, B: int, K: int, p: float) -> np.ndarray:
    """j_b with P(j = k) = p (1-p)^k for k < K and P(j = K) = (1-p)^K, by
    inversion of the Philox uniform (b, 0, STREAM_GEOM)."""
    u = philox_uniforms(seed, B, 1, STREAM_GEOM)[:, 0].astype(np.float64)
    j = np.zeros(B, dtype=np.int64)
    for b in range(B):
        # P(j >= k) = (1-p)^k: count successes of u < (1-p)^k.
        k = 0
        while k < K and u[b] < (1.0 - p) ** (k + 1):
            k += 1
        j[b] = k
    return j


def greedy_drafts(target_tokens: np.ndarray, K: int, vocab: int, seed: int,
                  p: float = 0.4, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Drafts that copy the given target tokens for the first j_b positions
    (j_b ~ truncated Geometric(p)) and are random afterwards.

    target_tokens[b, i] is the token the target model prefers after position i
    (supplied by the caller).  Draft j_b + 1 is drawn uniformly from the vocab
    minus target_tokens[b, j_b], so the realised greedy prefix is exactly j_b.
    rows: optional subset of requests to fill; other rows are left -1.
    """
    target_tokens = np.asarray(target_tokens)
    B = target_tokens.shape[0]
    d = np.full((B, K), -1, dtype=np.int32)
    j = truncated_geometric(seed, B, K, p)
    u = philox_uniforms(seed, B, K, STREAM_DRAFT).astype(np.float64)
    sel = range(B) if rows is None else rows
    for b in sel:
        for n in range(1, K + 1):
            if n <= j[b]:
                d[b, n - 1] = target_tokens[b, n - 1]
            elif n == j[b] + 1:
                avoid = int(target_tokens[b, n - 1])
                r = int(u[b, n - 1] * (vocab - 1))
                d[b, n - 1] = r if r < avoid else r + 1
            else:
                d[b, n - 1] = int(u[b, n - 1] * vocab)
    return d


def tree_parents(kind: str, Q: int) -> np.ndarray:
    """Parent array of a draft tree of Q nodes in topological order (node 0
    the root, parent -1).  "binary": the complete binary tree in
    breadth-first order (parent[i] = (i - 1) / 2); "chain": parent[i] = i - 1."""
    i = np.arange(Q)
    if kind == "binary":
        par = (i - 1) // 2
    elif kind == "chain":
        par = i - 1
    else:
        raise ValueError(f"unknown tree kind {kind!r}")
    par[0] = -1
    return par.astype(np.int32)


def tree_drafts(target_tokens: np.ndarray, parent: np.ndarray, vocab: int, seed: int,
                p_match: float = 0.6) -> np.ndarray:
    """Drafts for a tree: node n (1-based draft n) copies the target's token
    after its parent, target_tokens[b, parent[n]], with probability p_match
    (Philox uniform (b, n-1, STREAM_GEOM)), else a uniform token that avoids
    it (uniform (b, n-1, STREAM_DRAFT))."""
    target_tokens = np.asarray(target_tokens)
    B, Q = target_tokens.shape
    K = Q - 1
    um = philox_uniforms(seed, B, max(K, 1), STREAM_GEOM).astype(np.float64)
    ud = philox_uniforms(seed, B, max(K, 1), STREAM_DRAFT).astype(np.float64)
    d = np.full((B, K), -1, dtype=np.int32)
    for b in range(B):
        for n in range(1, Q):
            want = int(target_tokens[b, parent[n]])
            if um[b, n - 1] < p_match:
                d[b, n - 1] = want
            else:
                r = int(ud[b, n - 1] * (vocab - 1))
                d[b, n - 1] = r if r < want else r + 1
    return d


def draft_probs(logits_rows: np.ndarray, seed: int, sigma: float, temperature: float,
                top_p: float = 1.0) -> np.ndarray:
    """Draft distribution rows: softmax((l + N(0, sigma^2)) / T), optionally
    restricted to its own nucleus, renormalised.  logits_rows: [B, K, V]
    (the target's rows 0..K-1, as float).  Returns float32 [B, K, V]."""
    x = np.asarray(logits_rows, dtype=np.float64)
    rng = np.random.default_rng(seed * 7919 + _TAGS["noise"])
    x = x + rng.standard_normal(x.shape) * sigma
    t = temperature if temperature > 0 else 1.0
    x = x / t
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    pd = e / e.sum(axis=-1, keepdims=True)
    if top_p < 1.0:
        order = np.argsort(-pd, axis=-1, kind="stable")
        srt = np.take_along_axis(pd, order, axis=-1)
        csum = np.cumsum(srt, axis=-1)
        keep_sorted = (csum - srt) < top_p
        keep = np.zeros_like(keep_sorted)
        np.put_along_axis(keep, order, keep_sorted, axis=-1)
        pd = np.where(keep, pd, 0.0)
        pd = pd / pd.sum(axis=-1, keepdims=True)
    return pd.astype(np.float32)


def sample_drafts(pd: np.ndarray, seed: int) -> np.ndarray:
    """d[b, n-1] ~ pd[b, n-1, :] by inversion of Philox uniforms
    (b, n-1, STREAM_DRAFT).  Tokens with zero draft probability are never
    drawn."""
    B, K, V = pd.shape
    u = philox_uniforms(seed, B, K, STREAM_DRAFT).astype(np.float64)
    d = np.zeros((B, K), dtype=np.int32)
    for b in range(B):
        for n in range(K):
            c = np.cumsum(pd[b, n].astype(np.float64))
            idx = int(np.searchsorted(c, u[b, n] * c[-1], side="right"))
            idx = min(idx, V - 1)
            while pd[b, n, idx] <= 0 and idx > 0:
                idx -= 1
            d[b, n] = idx
    return d


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a bfloat16 tensor, as a host uint16 array."""
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

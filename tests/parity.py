"""Shared helpers of the GPU parity tests: moving synthetic inputs between
torch and the oracle's numpy formats, and the tolerance rules.

Tolerances (the rule each parity test applies):
  attention (fp32 output): per output row (b, i, h), max |gpu - oracle| <=
      2e-3 * max |oracle row|;
  bf16 logits: |gpu - exact| <= max(2e-2, one bf16 spacing at |exact|), i.e.
      within 2e-2 or a faithful rounding of the exact fp64 value where the
      bf16 grid is coarser than 2e-2 (|x| >= 4);
  fp32 logits: |gpu - exact| <= 1e-4;
  integer outputs (accepted counts, token ids, offsets, slots, pages): equal;
  sampling decisions: excluded only where the oracle's own diagnostics show
      |u - min(1, p_t/p_d)| < 1e-3, an inverse-CDF draw within 1e-9 of a
      bucket edge, or a top-p mass within 1e-9 of top_p.
"""
import numpy as np
import torch

import oracle
import speculative_decoding_sd_amd as sdv

DEV = torch.device("cuda", 0)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> host uint16 bit patterns (the oracle's bf16 format)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    """Oracle-format copy: uint16 bits for bf16, float32 otherwise."""
    if t.dtype == torch.bfloat16:
        return bits(t)
    return t.detach().contiguous().cpu().numpy()


def check_attention(out_gpu: np.ndarray, ref: np.ndarray, rel=2e-3, where=""):
    o = out_gpu.reshape(-1, out_gpu.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1])
    assert np.isfinite(o).all(), f"non-finite attention output {where}"
    err = np.abs(o - r).max(axis=1)
    scale = np.abs(r).max(axis=1)
    bad = err > rel * scale
    assert not bad.any(), (f"{where}: {bad.sum()} rows over tolerance; worst ratio "
                           f"{(err / np.maximum(scale, 1e-30)).max():.3e}")
    return float((err / np.maximum(scale, 1e-30)).max())


def bf16_spacing(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    e = np.floor(np.log2(ax))
    return 2.0 ** (e - 7)


def check_logits_bf16(gpu_bits: np.ndarray, exact: np.ndarray, where=""):
    g = oracle.bf16_to_f64(gpu_bits).reshape(exact.shape)
    tol = np.maximum(2e-2, bf16_spacing(exact))
    err = np.abs(g - exact)
    bad = err > tol
    assert not bad.any(), f"{where}: {bad.sum()} logits over tolerance, max err {err.max():.4g}"
    return float(err.max())


def check_logits_f32(gpu: np.ndarray, exact: np.ndarray, atol=1e-4, where=""):
    err = np.abs(gpu.astype(np.float64).reshape(exact.shape) - exact)
    assert err.max() <= atol, f"{where}: max err {err.max():.3g}"
    return float(err.max())


def excluded_requests(diag: np.ndarray) -> np.ndarray:
    """Requests whose sampling decision sits inside the exclusion windows."""
    return (diag[:, 1] < 1e-3) | (diag[:, 2] < 1e-9) | (diag[:, 3] < 1e-9)


def run_accept(logits_t, drafts_t, temp_t, top_p_t, pd_t, ua_t, us_t, relaxed_topk_t=None,
               relaxed_delta_t=None):
    B, Q, V = logits_t.shape
    i32 = dict(dtype=torch.int32, device=DEV)
    out = dict(num_accepted=torch.full((B,), -7, **i32), out_tokens=torch.full((B, Q), -7, **i32),
               next_token=torch.full((B,), -7, **i32), out_offsets=torch.full((B + 1,), -7, **i32),
               packed_tokens=torch.full((B * Q,), -7, **i32))
    err = torch.zeros(1, **i32)
    d = sdv.accept_desc(logits=logits_t, draft_tokens=drafts_t, temperature=temp_t,
                        u_accept=ua_t, u_sample=us_t, top_p=top_p_t, draft_probs=pd_t,
                        dev_error=err, relaxed_topk=relaxed_topk_t,
                        relaxed_delta=relaxed_delta_t, **out)
    sdv.accept(d)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["dev_error"] = int(err.item())
    return res


def compare_accept(gpu: dict, ref: dict, allow_excluded=True, where=""):
    excl = excluded_requests(ref["diag"]) if allow_excluded else np.zeros(len(ref["diag"]), bool)
    keep = ~excl
    for k_g, k_r in (("num_accepted", "num_accepted"), ("next_token", "next_token"),
                     ("out_tokens", "out_tokens")):
        g, r = gpu[k_g][keep], ref[k_r][keep]
        assert np.array_equal(g, r), (f"{where}: {k_g} mismatch at requests "
                                      f"{np.nonzero(keep)[0][np.any((g != r).reshape(len(g), -1), 1)][:10]}")
    if not excl.any():
        assert np.array_equal(gpu["out_offsets"], ref["out_offsets"]), where
        assert np.array_equal(gpu["packed_tokens"], ref["packed"]), where
    return int(excl.sum())


def gather_requests(wl, reqs):
    """Host copies (oracle formats) of the inputs of requests `reqs` of a
    device-resident workload, pages renumbered into a compact pool.  Taken
    before any library call touches the cache."""
    t = wl.tensors
    reqs = np.asarray(reqs)
    pt = wl.page_table[reqs]
    used = pt[pt >= 0]
    remap = np.full(wl.num_pages, -1, np.int64)
    remap[used] = np.arange(len(used))
    new_pt = np.where(pt >= 0, remap[np.maximum(pt, 0)], -1).astype(np.int32)
    idx = torch.tensor(used, dtype=torch.long, device=t["k_cache"].device)
    ridx = torch.tensor(reqs, dtype=torch.long, device=t["q"].device)
    return {
        "reqs": reqs, "page_table": new_pt, "num_pages": int(len(used)),
        "seq_lens": wl.seq_lens[reqs].copy(),
        "q": host(t["q"].index_select(0, ridx)),
        "k_new": host(t["k_new"].index_select(0, ridx)),
        "v_new": host(t["v_new"].index_select(0, ridx)) if t.get("v_new") is not None else None,
        "k_cache": host(t["k_cache"].index_select(0, idx)),
        "v_cache": host(t["v_cache"].index_select(0, idx)) if t.get("v_cache") is not None else None,
    }


def sample_requests(seq_lens, rng, n_random=2):
    """Requests a full-size test checks row by row: the longest and the
    shortest request, plus n_random others drawn at random."""
    L = np.asarray(seq_lens)
    picks = {int(np.argmax(L)), int(np.argmin(L))}
    others = [b for b in range(len(L)) if b not in picks]
    if others:
        picks |= set(int(b) for b in rng.choice(others, min(n_random, len(others)),
                                                 replace=False))
    return np.array(sorted(picks))


def gqa_wave_split_pairs(seq_lens, num_q, n_kv_heads, R, max_seq_len, e4m3, cus):
    """(request, kv head) pairs whose key tiles the streaming GQA kernel
    divides between two or more waves, so that their output goes through
    the partial slots and the log-sum-exp combine.  Mirrors the launch: every
    pair holds ceil((L_b + K + 1) / 32) tiles, kv-head-major then request;
    waves = 4 x min(CUs x workgroups per CU, max_waves / 4), max_waves the
    tile count at max_seq_len rounded up to 4 waves (at most 2048); wave w of
    n = min(waves, T) takes tiles [floor(wT/n), floor((w+1)T/n))."""
    L = np.asarray(seq_lens, np.int64)
    B = len(L)
    n_b = (L + num_q + 31) // 32
    first = np.concatenate([[0], np.cumsum(n_b)])
    T = n_kv_heads * int(first[-1])
    groups = 2 if (e4m3 and R <= 32) else 1
    max_tiles = B * n_kv_heads * ((max_seq_len + num_q + 31) // 32)
    max_waves = min(2048, 4 * ((max_tiles + 3) // 4))
    n = min(4 * min(cus * groups, max_waves // 4), T)

    def wave(x):  # the wave that holds tile x: ceil((x + 1) n / T) - 1
        return -(-(x + 1) * n // T) - 1

    out = []
    for h in range(n_kv_heads):
        for b in range(B):
            if n_b[b] == 0:
                continue
            g0 = h * int(first[-1]) + int(first[b])
            if wave(g0) != wave(g0 + int(n_b[b]) - 1):
                out.append((b, h))
    return out

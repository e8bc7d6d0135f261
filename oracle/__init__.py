"""Python access to the fp64 CPU oracle (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  It wraps `liboracle.so` (built from `sd_oracle.c` by `build()`)
with ctypes; it performs no arithmetic of its own beyond allocating outputs.
Arrays are host numpy arrays: float32, float64, uint16 holding bfloat16 bit
patterns, or (FP8 KV caches) uint8 holding OCP E4M3 codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, F64, E4M3 = 0, 1, 2, 3


def build(verbose: bool = False) -> str:
    """Compile sd_oracle.c with gcc (fp contraction off, OpenMP on)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.orc_num_threads.restype = ctypes.c_int
    return _lib


def _ptr(a):
    if a is None:
        return None
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError(f"unsupported oracle dtype {a.dtype}")


def _c(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))
    return a


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(ctypes.c_int(n))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of fp64 values to bfloat16 bit patterns."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_round_bf16(_ptr(x), _ptr(out), ctypes.c_size_t(x.size))
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (a widening, no rounding)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact value of OCP E4M3 (fn) codes (NaN for 0x7F / 0xFF)."""
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    lib().orc_e4m3_decode(_ptr(codes), _ptr(out), ctypes.c_size_t(codes.size))
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """E4M3 code nearest to each fp64 value (ties to even, saturating at 448,
    NaN -> 0x7F)."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().orc_e4m3_encode(_ptr(x), _ptr(out), ctypes.c_size_t(x.size))
    return out


def kv_append(seq_lens, page_table, num_pages, k_new, v_new, k_cache, v_cache, *,
              mla=False, page_size=64, k_scale=None, v_scale=None):
    """In-place append of the step's K+1 keys/values into the cache copies.
    uint8 caches hold E4M3 codes of value / scale[kv head] (k_scale, v_scale:
    float32 [n_kv_heads])."""
    k_new = _c(k_new)
    v_new = _c(v_new)
    seq_lens = _c(seq_lens, np.int32)
    page_table = _c(page_table, np.int32)
    assert k_cache.flags["C_CONTIGUOUS"] and (v_cache is None or v_cache.flags["C_CONTIGUOUS"])
    if k_cache.dtype == np.uint8:
        assert not mla and v_cache.dtype == np.uint8
        B, Q, Hkv, dk = k_new.shape
        k_scale = _c(k_scale, np.float32)
        v_scale = _c(v_scale, np.float32)
        assert k_scale.shape == (Hkv,) and v_scale.shape == (Hkv,)
        rc = lib().orc_kv_append_e4m3(
            B, Q, Hkv, dk, v_new.shape[-1], page_size, page_table.shape[1], int(num_pages),
            _dtype_code(k_new), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
            _ptr(page_table), _ptr(seq_lens), _ptr(k_scale), _ptr(v_scale))
        if rc != 0:
            raise ValueError(f"orc_kv_append_e4m3 failed ({rc})")
        return
    if mla:
        B, Q, dk = k_new.shape
        Hkv, dv = 1, 0
    else:
        B, Q, Hkv, dk = k_new.shape
        dv = v_new.shape[-1]
    rc = lib().orc_kv_append(
        B, Q, Hkv, dk, dv, int(mla), page_size, page_table.shape[1], int(num_pages),
        _dtype_code(k_new), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(page_table), _ptr(seq_lens))
    if rc != 0:
        raise ValueError(f"orc_kv_append failed ({rc})")


def verify_attn(q, k_cache, v_cache, page_table, seq_lens, num_pages, *, n_kv_heads,
                d_v, mla=False, page_size=64, scale=None, sel=None, k_scale=None,
                v_scale=None, tree_parent=None):
    """fp64 attention outputs.  q: [B, Q, Hq, d_qk].  sel: optional int array
    [n, 3] of (b, i, h).  uint8 caches hold E4M3 codes scaled per kv head by
    k_scale / v_scale.  tree_parent: optional int [B, Q] parent of each new
    position (tree attention mask).  Returns [B, Q, Hq, d_v] or [n, d_v]."""
    q = _c(q)
    B, Q, Hq, dqk = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dqk)
    page_table = _c(page_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    if sel is not None:
        sel = _c(sel, np.int32).reshape(-1, 3)
        out = np.empty((sel.shape[0], d_v), dtype=np.float64)
        n_sel = sel.shape[0]
    else:
        out = np.empty((B, Q, Hq, d_v), dtype=np.float64)
        n_sel = 0
    dt = _dtype_code(q)
    kdt = _dtype_code(k_cache)
    if kdt == E4M3:
        k_scale = _c(k_scale, np.float32)
        v_scale = _c(v_scale, np.float32)
        assert k_scale.shape == (n_kv_heads,) and v_scale.shape == (n_kv_heads,)
    else:
        assert kdt == dt
        k_scale = v_scale = None
    rc = lib().orc_verify_attn_ex(
        B, Q, Hq, n_kv_heads, dqk, d_v, int(mla), page_size, page_table.shape[1],
        int(num_pages), ctypes.c_double(scale), dt, kdt, _ptr(q), _ptr(k_cache),
        _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(page_table), _ptr(seq_lens),
        n_sel, _ptr(sel), _ptr(out), _ptr(_c(tree_parent, np.int32)))
    if rc != 0:
        raise ValueError(f"orc_verify_attn failed ({rc})")
    return out


def lm_head(H, W, rows=None):
    """fp64 logits H @ W^T.  rows: optional row indices of H."""
    H = _c(H)
    W = _c(W)
    M, hidden = H.shape
    V = W.shape[0]
    assert W.shape[1] == hidden and _dtype_code(H) == _dtype_code(W)
    if rows is not None:
        rows = _c(rows, np.int32).reshape(-1)
        out = np.empty((rows.shape[0], V), dtype=np.float64)
        nr = rows.shape[0]
    else:
        out = np.empty((M, V), dtype=np.float64)
        nr = 0
    lib().orc_lm_head(M, hidden, V, _dtype_code(H), _ptr(H), _ptr(W), nr, _ptr(rows),
                      _ptr(out))
    return out


def accept(logits, drafts, temperature, top_p, draft_probs, u_accept, u_sample,
           relaxed_topk=None, relaxed_delta=None, tree_parent=None):
    """Returns dict with num_accepted, out_tokens, next_token, out_offsets,
    packed, accepted_nodes, diag, n_invalid.  logits: [B, K+1, V]
    float32/float64/bf16 bits.  relaxed_topk / relaxed_delta ([B] int /
    float, optional): relaxed acceptance for greedy requests with top-N > 0.
    tree_parent ([B, K+1] int, optional): greedy tree verification."""
    logits = _c(logits)
    B, Q, V = logits.shape
    K = Q - 1
    drafts = _c(drafts, np.int32).reshape(B, K) if K > 0 else np.zeros((B, 0), np.int32)
    temperature = _c(temperature, np.float32)
    top_p = np.ones(B, np.float32) if top_p is None else _c(top_p, np.float32)
    draft_probs = _c(draft_probs, np.float32) if draft_probs is not None else None
    u_accept = _c(u_accept, np.float32)
    u_sample = _c(u_sample, np.float32)
    out = dict(
        num_accepted=np.empty(B, np.int32), out_tokens=np.empty((B, Q), np.int32),
        next_token=np.empty(B, np.int32), out_offsets=np.empty(B + 1, np.int32),
        packed=np.empty(B * Q, np.int32), diag=np.empty((B, 4), np.float64),
        accepted_nodes=np.empty((B, Q), np.int32))
    tp_arr = _c(tree_parent, np.int32) if tree_parent is not None else None
    rk = _c(relaxed_topk, np.int32) if relaxed_topk is not None else None
    rd = _c(relaxed_delta, np.float32) if relaxed_delta is not None else None
    n_bad = lib().orc_accept_ex(
        B, K, V, _dtype_code(logits), _ptr(logits), _ptr(drafts), _ptr(temperature),
        _ptr(top_p), _ptr(draft_probs), _ptr(u_accept), _ptr(u_sample), _ptr(rk), _ptr(rd),
        _ptr(out["num_accepted"]), _ptr(out["out_tokens"]), _ptr(out["next_token"]),
        _ptr(out["out_offsets"]), _ptr(out["packed"]), _ptr(out["diag"]), _ptr(tp_arr),
        _ptr(out["accepted_nodes"]))
    out["n_invalid"] = n_bad
    return out


def argmax(logits):
    """Greedy target token per row (smallest id on ties) and top-2 margin.
    logits: [..., V]; returns (int32 [...], float64 [...])."""
    logits = _c(logits)
    V = logits.shape[-1]
    n = logits.size // V
    out = np.empty(n, np.int32)
    mg = np.empty(n, np.float64)
    lib().orc_argmax_rows(n, V, _dtype_code(logits), _ptr(logits), _ptr(out), _ptr(mg))
    return out.reshape(logits.shape[:-1]), mg.reshape(logits.shape[:-1])


def kv_rollback(page_table, num_accepted, seq_lens, K, *, page_size=64, poison=False,
                k_cache=None, v_cache=None, n_kv_heads=1, d_k=0, d_v=0, mla=False,
                accepted_nodes=None):
    """Returns dict with new seq_lens, rb_slots, rb_offsets, freed, freed_offsets,
    n_bad.  Poison zeroes rejected slots of the given cache copies in place.
    accepted_nodes ([B, K+1], tree of drafts): the accepted path's rows are
    gathered to contiguous slots first (in place in the cache copies)."""
    page_table = _c(page_table, np.int32)
    num_accepted = _c(num_accepted, np.int32)
    sl = np.array(seq_lens, dtype=np.int32, copy=True)
    B = sl.shape[0]
    out = dict(rb_slots=np.full(B * (K + 1), -1, np.int32), rb_offsets=np.empty(B + 1, np.int32),
               freed=np.full(B * (K // page_size + 2), -1, np.int32),
               freed_offsets=np.empty(B + 1, np.int32))
    dt = _dtype_code(k_cache) if k_cache is not None else F32
    n_bad = lib().orc_kv_rollback(
        B, K, page_size, page_table.shape[1], _ptr(page_table), _ptr(num_accepted),
        _ptr(sl), _ptr(out["rb_slots"]), _ptr(out["rb_offsets"]), _ptr(out["freed"]),
        _ptr(out["freed_offsets"]), int(poison), n_kv_heads, d_k, d_v, int(mla), dt,
        _ptr(k_cache), _ptr(v_cache), _ptr(_c(accepted_nodes, np.int32)))
    out["seq_lens"] = sl
    out["n_bad"] = n_bad
    return out

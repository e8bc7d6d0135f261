"""MI355X-native speculative-decoding verify step.

Python binding of libsdv.so (ctypes).  It only marshals arguments: every step
of the verify path (append, attention, combine, LM head, acceptance, packing,
rollback) runs in the library's gfx950 HIP kernels.  PyTorch supplies device
memory and streams.  If the library is missing, loading fails with an error;
there is no fallback path.

Entry points mirror include/sdv.h: sd_verify_attn, sd_lm_head, sd_accept,
sd_kv_rollback (plus workspace-size queries), and VerifyStep, which owns the
workspaces of one configuration and runs the four calls on one stream.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdv.so")

SD_OK, SD_EINVAL, SD_EUNSUPPORTED, SD_EWORKSPACE, SD_EDEVICE = 0, 1, 2, 3, 4
SD_F32, SD_BF16, SD_E4M3 = 0, 1, 2
SD_KV_AS_DTYPE, SD_KV_E4M3 = 0, 1
SD_ATTN_GQA, SD_ATTN_MLA = 0, 1
SD_DERR_PAGE, SD_DERR_CAPACITY, SD_DERR_TOKEN = 1, 2, 4
SD_DERR_NONFINITE, SD_DERR_PARAM, SD_DERR_ACCEPT_COUNT = 8, 16, 32
SD_DERR_TREE = 64

_P = ctypes.c_void_p
_I = ctypes.c_int


class SdvError(RuntimeError):
    def __init__(self, name, code, text):
        super().__init__(f"{name} failed with status {code}: {text}")
        self.code = code


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", _I), ("num_q", _I), ("n_q_heads", _I), ("n_kv_heads", _I), ("d_qk", _I),
        ("d_v", _I), ("kind", _I), ("dtype", _I), ("page_size", _I), ("max_pages", _I),
        ("num_pages", _I), ("max_seq_len", _I), ("softmax_scale", ctypes.c_float),
        ("q", _P), ("k_new", _P), ("v_new", _P), ("k_cache", _P), ("v_cache", _P),
        ("page_table", _P), ("seq_lens", _P), ("out", _P), ("out_lowp", _P), ("dev_error", _P),
        ("kv_format", _I), ("k_scale", _P), ("v_scale", _P), ("tree_parent", _P),
    ]


class AcceptDesc(ctypes.Structure):
    _fields_ = [
        ("batch", _I), ("K", _I), ("vocab", _I), ("logits_dtype", _I), ("logits", _P),
        ("draft_tokens", _P), ("temperature", _P), ("top_p", _P), ("draft_probs", _P),
        ("u_accept", _P), ("u_sample", _P), ("num_accepted", _P), ("out_tokens", _P),
        ("next_token", _P), ("out_offsets", _P), ("packed_tokens", _P), ("dev_error", _P),
        ("relaxed_topk", _P), ("relaxed_delta", _P), ("tree_parent", _P), ("accepted_nodes", _P),
    ]


class RollbackDesc(ctypes.Structure):
    _fields_ = [
        ("batch", _I), ("K", _I), ("page_size", _I), ("max_pages", _I), ("page_table", _P),
        ("num_accepted", _P), ("seq_lens", _P), ("rollback_slots", _P),
        ("rollback_offsets", _P), ("freed_pages", _P), ("freed_offsets", _P),
        ("poison_rejected", _I), ("kind", _I), ("dtype", _I), ("n_kv_heads", _I), ("d_k", _I),
        ("d_v", _I), ("num_pages", _I), ("k_cache", _P), ("v_cache", _P), ("dev_error", _P),
        ("accepted_nodes", _P),
    ]


# Every symbol include/sdv.h declares.
EXPORTS = ["sd_abi_version", "sd_last_error", "sd_get_device_error",
           "sd_verify_attn_workspace_size", "sd_verify_attn", "sd_lm_head",
           "sd_accept_workspace_size", "sd_accept", "sd_accept_noalloc", "sd_kv_rollback"]

_lib = None


def lib():
    """The loaded libsdv.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        L.sd_abi_version.restype = _I
        L.sd_last_error.restype = ctypes.c_char_p
        L.sd_verify_attn_workspace_size.argtypes = [ctypes.POINTER(AttnDesc),
                                                    ctypes.POINTER(ctypes.c_size_t)]
        L.sd_verify_attn.argtypes = [ctypes.POINTER(AttnDesc), _P, ctypes.c_size_t, _P]
        L.sd_lm_head.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P]
        L.sd_accept_workspace_size.argtypes = [ctypes.POINTER(AcceptDesc),
                                               ctypes.POINTER(ctypes.c_size_t)]
        L.sd_accept.argtypes = [ctypes.POINTER(AcceptDesc), _P, ctypes.c_size_t, _P]
        L.sd_accept_noalloc.argtypes = [ctypes.POINTER(AcceptDesc), _P]
        L.sd_kv_rollback.argtypes = [ctypes.POINTER(RollbackDesc), _P]
        L.sd_get_device_error.argtypes = [_P, ctypes.POINTER(ctypes.c_int32), _P]
        for name in EXPORTS:
            getattr(L, name).restype = getattr(L, name).restype or _I
        L.sd_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc, name):
    if rc != SD_OK:
        raise SdvError(name, rc, lib().sd_last_error().decode(errors="replace"))


def last_error() -> str:
    return lib().sd_last_error().decode(errors="replace")


# ---------------------------------------------------------------------------
# Raw C-ABI calls (descriptors with plain integer pointers).
# ---------------------------------------------------------------------------
def sd_verify_attn_workspace_size(desc: AttnDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().sd_verify_attn_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "sd_verify_attn_workspace_size")
    return n.value


def sd_verify_attn(desc: AttnDesc, workspace: int, ws_bytes: int, stream: int) -> None:
    _check(lib().sd_verify_attn(ctypes.byref(desc), _P(workspace), ws_bytes, _P(stream)),
           "sd_verify_attn")


def sd_lm_head(M, hidden, vocab, dtype, H, W, logits, stream) -> None:
    _check(lib().sd_lm_head(M, hidden, vocab, dtype, _P(H), _P(W), _P(logits), _P(stream)),
           "sd_lm_head")


def sd_accept_workspace_size(desc: AcceptDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().sd_accept_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "sd_accept_workspace_size")
    return n.value


def sd_accept(desc: AcceptDesc, workspace: int, ws_bytes: int, stream: int) -> None:
    _check(lib().sd_accept(ctypes.byref(desc), _P(workspace), ws_bytes, _P(stream)),
           "sd_accept")


def sd_accept_noalloc(desc: AcceptDesc, stream: int) -> None:
    _check(lib().sd_accept_noalloc(ctypes.byref(desc), _P(stream)), "sd_accept_noalloc")


def sd_kv_rollback(desc: RollbackDesc, stream: int) -> None:
    _check(lib().sd_kv_rollback(ctypes.byref(desc), _P(stream)), "sd_kv_rollback")


def sd_get_device_error(dev_error: int, stream: int) -> int:
    """The SD_DERR_* word at device address dev_error, once `stream` has
    passed the calls issued on it (synchronises the host)."""
    code = ctypes.c_int32(0)
    _check(lib().sd_get_device_error(_P(dev_error), ctypes.byref(code), _P(stream)),
           "sd_get_device_error")
    return code.value


# ---------------------------------------------------------------------------
# Tensor helpers (marshalling only).
# ---------------------------------------------------------------------------
def _ptr(t):
    return 0 if t is None else t.data_ptr()


def sd_dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SD_BF16
    if t.dtype == torch.float32:
        return SD_F32
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return SD_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def workspace(nbytes: int, device):
    """Device workspace of at least nbytes, 256-byte aligned (torch allocator)."""
    import torch
    return torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)


def _aligned(ws) -> int:
    p = ws.data_ptr()
    return (p + 255) // 256 * 256


def _keeping(tensors, desc):
    """Attaches the tensors whose device pointers desc holds, so that they
    stay allocated as long as the descriptor does (a temporary passed in would
    otherwise return its memory to torch's caching allocator while the
    descriptor still points at it)."""
    desc._keep = tuple(t for t in tensors if t is not None)
    return desc


def attn_desc(*, q, k_cache, v_cache, page_table, seq_lens, out, n_kv_heads, num_pages,
              max_seq_len, k_new=None, v_new=None, mla=False, out_lowp=None,
              softmax_scale=0.0, dev_error=None, page_size=64, k_scale=None,
              v_scale=None, tree_parent=None) -> AttnDesc:
    """Caches of dtype uint8 or float8_e4m3fn hold E4M3 codes and take float32
    per-kv-head k_scale / v_scale.  tree_parent: optional int32 [B, K+1]
    parent of each new position (a tree of drafts)."""
    B, NQ, Hq, dqk = q.shape
    d_v = out.shape[-1]
    fp8 = sd_dtype(k_cache) == SD_E4M3
    return _keeping((q, k_cache, v_cache, page_table, seq_lens, out, k_new, v_new, out_lowp,
                     dev_error, k_scale, v_scale, tree_parent), AttnDesc(
        batch=B, num_q=NQ, n_q_heads=Hq, n_kv_heads=n_kv_heads, d_qk=dqk, d_v=d_v,
        kind=SD_ATTN_MLA if mla else SD_ATTN_GQA, dtype=sd_dtype(q), page_size=page_size,
        max_pages=page_table.shape[1], num_pages=num_pages, max_seq_len=max_seq_len,
        softmax_scale=softmax_scale, q=_ptr(q), k_new=_ptr(k_new), v_new=_ptr(v_new),
        k_cache=_ptr(k_cache), v_cache=_ptr(v_cache), page_table=_ptr(page_table),
        seq_lens=_ptr(seq_lens), out=_ptr(out), out_lowp=_ptr(out_lowp),
        dev_error=_ptr(dev_error), kv_format=SD_KV_E4M3 if fp8 else SD_KV_AS_DTYPE,
        k_scale=_ptr(k_scale) if fp8 else None, v_scale=_ptr(v_scale) if fp8 else None,
        tree_parent=_ptr(tree_parent)))


def verify_attn(desc: AttnDesc, ws=None, stream=None):
    """Runs sd_verify_attn; allocates a workspace tensor when none is given."""
    import torch
    n = sd_verify_attn_workspace_size(desc)
    if ws is None:
        ws = workspace(n, torch.device("cuda", torch.cuda.current_device()))
    sd_verify_attn(desc, _aligned(ws), ws.numel() - (_aligned(ws) - ws.data_ptr()),
                   current_stream() if stream is None else stream)
    return ws


def lm_head(H, W, logits, stream=None):
    M, hidden = H.shape
    vocab = W.shape[0]
    sd_lm_head(M, hidden, vocab, sd_dtype(H), H.data_ptr(), W.data_ptr(), logits.data_ptr(),
               current_stream() if stream is None else stream)


def accept_desc(*, logits, draft_tokens, temperature, u_accept, u_sample, num_accepted,
                out_tokens, next_token, out_offsets, packed_tokens, top_p=None,
                draft_probs=None, dev_error=None, relaxed_topk=None,
                relaxed_delta=None, tree_parent=None, accepted_nodes=None) -> AcceptDesc:
    B, Q, V = logits.shape
    return _keeping((logits, draft_tokens, temperature, u_accept, u_sample, num_accepted,
                     out_tokens, next_token, out_offsets, packed_tokens, top_p, draft_probs,
                     dev_error, relaxed_topk, relaxed_delta, tree_parent, accepted_nodes),
                    AcceptDesc(
        batch=B, K=Q - 1, vocab=V, logits_dtype=sd_dtype(logits), logits=_ptr(logits),
        draft_tokens=_ptr(draft_tokens), temperature=_ptr(temperature), top_p=_ptr(top_p),
        draft_probs=_ptr(draft_probs), u_accept=_ptr(u_accept), u_sample=_ptr(u_sample),
        num_accepted=_ptr(num_accepted), out_tokens=_ptr(out_tokens),
        next_token=_ptr(next_token), out_offsets=_ptr(out_offsets),
        packed_tokens=_ptr(packed_tokens), dev_error=_ptr(dev_error),
        relaxed_topk=_ptr(relaxed_topk), relaxed_delta=_ptr(relaxed_delta),
        tree_parent=_ptr(tree_parent), accepted_nodes=_ptr(accepted_nodes)))


def accept(desc: AcceptDesc, ws=None, stream=None):
    import torch
    n = sd_accept_workspace_size(desc)
    if ws is None:
        ws = workspace(n, torch.device("cuda", torch.cuda.current_device()))
    sd_accept(desc, _aligned(ws), ws.numel() - (_aligned(ws) - ws.data_ptr()),
              current_stream() if stream is None else stream)
    return ws


def rollback_desc(*, page_table, num_accepted, seq_lens, K, rollback_slots, rollback_offsets,
                  freed_pages, freed_offsets, poison=False, k_cache=None, v_cache=None,
                  mla=False, n_kv_heads=1, d_k=0, d_v=0, num_pages=0, dev_error=None,
                  page_size=64, accepted_nodes=None) -> RollbackDesc:
    dtype = sd_dtype(k_cache) if k_cache is not None else SD_BF16
    return _keeping((page_table, num_accepted, seq_lens, rollback_slots, rollback_offsets,
                     freed_pages, freed_offsets, k_cache, v_cache, dev_error, accepted_nodes),
                    RollbackDesc(
        batch=seq_lens.shape[0], K=K, page_size=page_size, max_pages=page_table.shape[1],
        page_table=_ptr(page_table), num_accepted=_ptr(num_accepted), seq_lens=_ptr(seq_lens),
        rollback_slots=_ptr(rollback_slots), rollback_offsets=_ptr(rollback_offsets),
        freed_pages=_ptr(freed_pages), freed_offsets=_ptr(freed_offsets),
        poison_rejected=int(poison), kind=SD_ATTN_MLA if mla else SD_ATTN_GQA, dtype=dtype,
        n_kv_heads=n_kv_heads, d_k=d_k, d_v=d_v, num_pages=num_pages, k_cache=_ptr(k_cache),
        v_cache=_ptr(v_cache), dev_error=_ptr(dev_error), accepted_nodes=_ptr(accepted_nodes)))


def kv_rollback(desc: RollbackDesc, stream=None):
    sd_kv_rollback(desc, current_stream() if stream is None else stream)


def device_error(dev_error, stream=None) -> int:
    """sd_get_device_error on an int32 device tensor."""
    return sd_get_device_error(dev_error.data_ptr(),
                               current_stream() if stream is None else stream)


from .step import VerifyStep  # noqa: E402  (uses the helpers above)

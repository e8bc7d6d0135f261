"""The C-ABI library loads, exports every symbol include/sdv.h declares, and
rejects bad arguments on the host before launching anything (CPU only: no
call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import speculative_decoding_sd_amd as sdv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "sdv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("sd_verify_attn", "sd_lm_head", "sd_accept", "sd_kv_rollback"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = sdv.lib()
    names = _declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(sdv.EXPORTS)


def test_abi_version_matches_header():
    src = open(os.path.join(ROOT, "include", "sdv.h")).read()
    ver = int(re.search(r"#define SD_ABI_VERSION (\d+)", src).group(1))
    assert sdv.lib().sd_abi_version() == ver


def test_struct_layouts_match_header():
    """Field names and order of the ctypes mirrors follow the C structs."""
    src = open(os.path.join(ROOT, "include", "sdv.h")).read()
    for struct, cls in (("sd_attn_desc", sdv.AttnDesc), ("sd_accept_desc", sdv.AcceptDesc),
                        ("sd_rollback_desc", sdv.RollbackDesc)):
        body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (struct, struct), src, re.S).group(1)
        body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
        fields = re.findall(r"(\w+)\s*;", body)
        assert fields == [f[0] for f in cls._fields_], struct


def _attn_desc(**kw):
    base = dict(batch=2, num_q=4, n_q_heads=8, n_kv_heads=2, d_qk=128, d_v=128, kind=0, dtype=1,
                page_size=64, max_pages=4, num_pages=8, max_seq_len=100, softmax_scale=0.0,
                q=256, k_new=0, v_new=0, k_cache=512, v_cache=768, page_table=1024,
                seq_lens=1280, out=1536, out_lowp=0, dev_error=0)
    base.update(kw)
    return sdv.AttnDesc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), sdv.SD_EINVAL),
    (dict(n_q_heads=7), sdv.SD_EINVAL),
    (dict(dtype=5), sdv.SD_EINVAL),
    (dict(page_size=32), sdv.SD_EUNSUPPORTED),
    (dict(d_qk=96, d_v=96), sdv.SD_EUNSUPPORTED),
    (dict(max_seq_len=1000), sdv.SD_EINVAL),            # exceeds max_pages * 64
    (dict(n_q_heads=64, n_kv_heads=2), sdv.SD_EUNSUPPORTED),  # 32 heads x 4 rows > 64
    (dict(kv_format=7), sdv.SD_EINVAL),
    (dict(kv_format=1, dtype=0), sdv.SD_EUNSUPPORTED),  # E4M3 cache with f32 q
    (dict(kv_format=1, kind=1, n_kv_heads=1, d_qk=576, d_v=512), sdv.SD_EUNSUPPORTED),  # MLA
    (dict(kv_format=1, d_qk=96, d_v=96), sdv.SD_EUNSUPPORTED),
    (dict(tree_parent=4096, kind=1, n_kv_heads=1, d_qk=576, d_v=512), sdv.SD_EUNSUPPORTED),
    (dict(tree_parent=4096, num_q=65, n_q_heads=2, n_kv_heads=2, max_pages=8),
     sdv.SD_EUNSUPPORTED),                                # a tree of more than 64 nodes
])
def test_attention_host_validation(kw, code):
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_verify_attn_workspace_size(_attn_desc(**kw))
    assert e.value.code == code
    assert sdv.last_error()


def test_attention_workspace_and_pointer_checks():
    d = _attn_desc()
    n = sdv.sd_verify_attn_workspace_size(d)
    assert n > 0 and n % 256 == 0
    with pytest.raises(sdv.SdvError) as e:      # workspace too small
        sdv.sd_verify_attn(d, 4096, n - 1, 0)
    assert e.value.code == sdv.SD_EWORKSPACE
    with pytest.raises(sdv.SdvError) as e:      # misaligned workspace
        sdv.sd_verify_attn(d, 4096 + 8, n, 0)
    assert e.value.code == sdv.SD_EINVAL
    with pytest.raises(sdv.SdvError) as e:      # misaligned tensor
        sdv.sd_verify_attn(_attn_desc(q=258), 4096, n, 0)
    assert e.value.code == sdv.SD_EINVAL
    with pytest.raises(sdv.SdvError) as e:      # NULL output
        sdv.sd_verify_attn(_attn_desc(out=0), 4096, n, 0)
    assert e.value.code == sdv.SD_EINVAL
    d8 = _attn_desc(kv_format=1, k_scale=2048, v_scale=0)
    assert sdv.sd_verify_attn_workspace_size(d8) == n  # the workspace does not depend on it
    with pytest.raises(sdv.SdvError) as e:      # E4M3 cache without v_scale
        sdv.sd_verify_attn(d8, 4096, n, 0)
    assert e.value.code == sdv.SD_EINVAL


def test_lm_head_host_validation():
    for args, code in [((0, 64, 10, 1, 16, 32, 48), sdv.SD_EINVAL),
                       ((4, 60, 10, 1, 16, 32, 48), sdv.SD_EUNSUPPORTED),
                       ((4, 64, 10, 3, 16, 32, 48), sdv.SD_EINVAL),
                       ((4, 64, 10, 1, 0, 32, 48), sdv.SD_EINVAL),
                       ((4, 64, 10, 1, 17, 32, 48), sdv.SD_EINVAL)]:
        with pytest.raises(sdv.SdvError) as e:
            sdv.sd_lm_head(*args, 0)
        assert e.value.code == code


def test_accept_and_rollback_host_validation():
    d = sdv.AcceptDesc(batch=2, K=3, vocab=100, logits_dtype=1, logits=256, draft_tokens=512,
                       temperature=768, top_p=0, draft_probs=0, u_accept=1024, u_sample=1280,
                       num_accepted=1536, out_tokens=1792, next_token=2048, out_offsets=2304,
                       packed_tokens=2560, dev_error=0)
    n = sdv.sd_accept_workspace_size(d)
    assert n >= 2 * 4 * 32
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_accept(d, 4096, n - 256, 0)
    assert e.value.code == sdv.SD_EWORKSPACE
    d.vocab = 262145                            # one id above the largest supported vocab
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_accept_workspace_size(d)
    assert e.value.code == sdv.SD_EUNSUPPORTED
    d.vocab = 262144
    assert sdv.sd_accept_workspace_size(d) % 256 == 0
    d.logits_dtype = 7
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_accept_workspace_size(d)
    assert e.value.code == sdv.SD_EINVAL
    d.logits_dtype = 1
    d.K = 64                                    # a tree of 65 nodes
    d.tree_parent = 4096
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_accept_workspace_size(d)
    assert e.value.code == sdv.SD_EUNSUPPORTED
    d.K = 63
    assert sdv.sd_accept_workspace_size(d) % 256 == 0
    r = sdv.RollbackDesc(batch=2, K=3, page_size=64, max_pages=4, page_table=0,
                         num_accepted=256, seq_lens=512, rollback_slots=768,
                         rollback_offsets=1024, freed_pages=1280, freed_offsets=1536)
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_kv_rollback(r, 0)
    assert e.value.code == sdv.SD_EINVAL
    r.page_table = 4096
    r.poison_rejected = 1
    with pytest.raises(sdv.SdvError) as e:     # poisoning without a cache description
        sdv.sd_kv_rollback(r, 0)
    assert e.value.code == sdv.SD_EINVAL


def test_descriptors_keep_their_tensors_alive():
    """A descriptor holds raw device pointers; it must also hold the tensors,
    or a temporary passed in would be freed (and its memory reused) while the
    descriptor still points at it."""
    import gc
    import weakref

    import torch

    import speculative_decoding_sd_amd as sdv

    pt = torch.zeros((2, 4), dtype=torch.int32)
    ref = weakref.ref(pt)
    d = sdv.attn_desc(q=torch.zeros((2, 4, 8, 576), dtype=torch.bfloat16),
                      k_cache=torch.zeros((3, 64, 576), dtype=torch.bfloat16), v_cache=None,
                      page_table=pt, seq_lens=torch.zeros(2, dtype=torch.int32),
                      out=torch.zeros((2, 4, 8, 512)), n_kv_heads=1, num_pages=3,
                      max_seq_len=10, mla=True)
    del pt
    gc.collect()
    assert ref() is not None and d.page_table == ref().data_ptr()
    del d
    gc.collect()
    assert ref() is None


def test_device_error_query_rejects_null_pointers():
    """sd_get_device_error checks its pointers before touching the device."""
    L = sdv.lib()
    code = ctypes.c_int32(-7)
    assert L.sd_get_device_error(None, ctypes.byref(code), None) == sdv.SD_EINVAL
    assert code.value == -7 and "NULL" in sdv.last_error()
    assert L.sd_get_device_error(ctypes.c_void_p(4096), None, None) == sdv.SD_EINVAL


def test_noalloc_accept_rejects_batches_beyond_its_scratch():
    """sd_accept_noalloc checks the batch against its fixed scratch before it
    touches the device: 70000 rows need more than the 4 MiB it holds."""
    d = sdv.AcceptDesc(batch=70000, K=0, vocab=100, logits_dtype=1, logits=256,
                       draft_tokens=0, temperature=768, top_p=0, draft_probs=0, u_accept=1024,
                       u_sample=1280, num_accepted=1536, out_tokens=1792, next_token=2048,
                       out_offsets=2304, packed_tokens=2560, dev_error=0)
    with pytest.raises(sdv.SdvError) as e:
        sdv.sd_accept_noalloc(d, 0)
    assert e.value.code == sdv.SD_EWORKSPACE and "scratch" in e.value.args[0] + sdv.last_error()
    d.out_tokens = 0
    with pytest.raises(sdv.SdvError) as e:      # pointers are checked first
        sdv.sd_accept_noalloc(d, 0)
    assert e.value.code == sdv.SD_EINVAL


def test_probe_library_rejects_bad_arguments():
    """The measurement probe bench.py --mfma-ceiling loads is built beside the
    library and checks its sizes on the host before launching."""
    from speculative_decoding_sd_amd import build as sdv_build
    assert os.path.exists(sdv_build.PROBE_LIB_PATH), "run build() first"
    P = ctypes.CDLL(sdv_build.PROBE_LIB_PATH)
    f = P.sdv_probe_mfma_bf16
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    buf = ctypes.create_string_buffer(16)
    ok_ops, ok_sink = 12 * 512 * 16, 512
    assert f(None, ok_ops, buf, ok_sink, 1, 1, None) == -1            # no operands
    assert f(buf, ok_ops, None, ok_sink, 1, 1, None) == -1            # no sink
    assert f(buf, ok_ops - 16, buf, ok_sink, 1, 1, None) == -1        # operands too small
    assert f(buf, ok_ops, buf, ok_sink - 1, 1, 1, None) == -1         # sink too small
    assert f(buf, ok_ops, buf, ok_sink, 0, 1, None) == -1             # no blocks
    assert f(buf, ok_ops, buf, ok_sink, 1, 0, None) == -1             # no iterations


def test_hbm_probe_rejects_bad_arguments():
    """The streaming-read probe bench.py --hbm-ceiling loads checks its sizes
    on the host before launching."""
    from speculative_decoding_sd_amd import build as sdv_build
    P = ctypes.CDLL(sdv_build.PROBE_LIB_PATH)
    f = P.sdv_probe_hbm_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_int, ctypes.c_void_p]
    buf = ctypes.create_string_buffer(16)
    assert f(None, 1 << 20, buf, 256, 1, None) == -1       # no source
    assert f(buf, 1 << 20, None, 256, 1, None) == -1       # no sink
    assert f(buf, 0, buf, 256, 1, None) == -1              # nothing to read
    assert f(buf, (1 << 20) + 8, buf, 256, 1, None) == -1  # not whole 16-byte words
    assert f(buf, 1 << 20, buf, 255, 1, None) == -1        # sink too small
    assert f(buf, 1 << 20, buf, 256, 0, None) == -1        # no blocks

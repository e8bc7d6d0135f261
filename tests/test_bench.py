"""Host-side logic of bench.py: the algorithmic byte and flop models behind
`roofline`, the name of the LM-head kernel whose profile supplies `traffic`,
and the refusal of a multi-GPU run.  No GPU is touched."""
import dataclasses
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import sdsynth  # noqa: E402


def _tiny_gqa(**kw):
    cfg = dataclasses.replace(sdsynth.CONFIGS[2], batch=2, K=3, n_q_heads=8, n_kv_heads=2,
                              d_qk=64, d_v=64, dtype="bf16")
    return dataclasses.replace(cfg, **kw)


def test_attention_bytes_by_hand():
    cfg = _tiny_gqa()
    L = np.array([10, 30], dtype=np.int32)
    NQ = 4
    keys = (10 + NQ) + (30 + NQ)                      # cached and new keys, each read once
    kv = keys * 2 * (64 + 64) * 2                     # 2 kv heads, K and V, bf16
    new = 2 * NQ * 2 * (64 + 64) * (2 + 2)            # new rows read (bf16), written (bf16)
    q = 2 * NQ * 8 * 64 * 2
    out = 2 * NQ * 8 * 64 * 4                         # fp32 output
    assert bench.attention_bytes(cfg, L) == kv + new + q + out
    # An E4M3 cache halves the cache bytes and the written new rows.
    e = bench.attention_bytes(dataclasses.replace(cfg, kv_cache="e4m3"), L)
    assert e == keys * 2 * 128 * 1 + 2 * NQ * 2 * 128 * (2 + 1) + q + out


def test_attention_flops_by_hand():
    cfg = _tiny_gqa()
    L = np.array([10, 30], dtype=np.int32)
    # query (i, h) of request b scores and averages L_b + i + 1 keys
    keys = sum(L[b] + i + 1 for b in range(2) for i in range(4))
    assert bench.attention_flops(cfg, L) == keys * 8 * 2 * (64 + 64)


def test_lm_head_work_by_hand():
    cfg = sdsynth.CONFIGS[5]
    M = cfg.batch * cfg.num_q
    f, b = bench.lm_head_work(cfg)
    assert f == 2.0 * M * 7168 * 129280
    assert b == (129280 * 7168 + M * 7168 + M * 129280) * 2


def test_accept_bytes_by_hand():
    cfg = sdsynth.CONFIGS[5]
    assert bench.accept_bytes(cfg) == 256 * 5 * 129280 * 2


def test_lm_head_kernel_follows_the_dispatch_rule():
    k = bench.lm_head_kernel
    assert k(1280, 7168, 129280, "bf16", 256) == "lm_head_ring"    # C5: 2525 tiles
    assert k(256, 7168, 129280, "bf16", 256) == "lm_head_ring"     # C3: 505 tiles
    assert k(192, 4096, 32000, "bf16", 256) == "lm_head_stream"    # C2: 125 tiles < 256 CUs
    assert k(192, 7168, 129280, "bf16", 256) == "lm_head_ring"     # 505 tiles
    assert k(64, 5120, 152064, "bf16", 256) == "lm_head_stream"    # C4: 64-row tiles
    assert k(300, 384, 40000, "bf16", 256) == "lm_head_ring"       # 2 x 157 tiles
    assert k(300, 384, 40000, "bf16", 512) == "lm_head_stream"     # fewer tiles than CUs
    assert k(4, 1024, 256, "f32", 256) is None                     # fp32 path
    assert k(130, 200, 333, "bf16", 256) is None                   # hidden not a multiple of 128


def test_attention_kernel_follows_the_dispatch_rule():
    k = bench.attention_kernel
    assert k(True, "bf16", "as_dtype", 128, 1, 4, 576) == "attn_mla_bf16"         # C3
    assert k(False, "bf16", "as_dtype", 40, 8, 8, 128) == "attn_gqa_stream"       # C4
    assert k(False, "bf16", "e4m3", 40, 8, 8, 128) == "attn_gqa_f8_r16"           # C4, E4M3: 40 rows
    assert k(False, "bf16", "e4m3", 32, 8, 5, 128) == "attn_gqa_stream"           # C5, E4M3: 20 rows
    assert k(False, "bf16", "e4m3", 6, 2, 11, 128) == "attn_gqa_f8_r16"           # 33 rows
    assert k(False, "bf16", "e4m3", 12, 2, 8, 128) == "attn_gqa_f8_r16"           # 48 rows
    assert k(False, "bf16", "e4m3", 8, 2, 16, 128) == "attn_gqa_stream"           # 64 rows
    assert k(False, "bf16", "e4m3", 10, 2, 8, 64) == "attn_gqa_stream"            # head dim 64
    assert k(False, "f32", "as_dtype", 4, 4, 4, 64) is None                       # C1


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_committed_profiles_match_the_sources():
    """Every committed PMC summary with machine-readable lines still hashes
    to its kernel's sources and flags (else bench.py would report null
    traffic), and the MFMA ceiling probe's figure is on record."""
    import glob
    import os
    n = 0
    for path in glob.glob(os.path.join(bench.ROOT, "profiles", "*.md")):
        name = os.path.basename(path)[:-3]
        if "source_sha256: " not in open(path).read():
            continue  # a summary without machine-readable lines (not read by bench.py)
        for kernel in bench.KERNEL_SOURCES:
            if name.startswith(kernel + "_"):
                fields = bench.profiled_fields(kernel, name[len(kernel) + 1:])
                assert fields, f"{name}: source hash is stale"
                n += 1
    assert n >= 10
    assert 1000.0 < bench.mfma_ceiling_on_record() < bench.MFMA_BF16_PEAK_TFS
    assert 3000.0 < bench.hbm_ceiling_on_record() < bench.HBM_PEAK_GBS

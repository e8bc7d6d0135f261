"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = sd_verify_attn (append + causal attention over the paged cache)
-> sd_lm_head -> sd_accept -> sd_kv_rollback, on one stream, over one batch
of seeded synthetic inputs already resident in HBM.  The steps form a decode
loop: each rollback advances seq_lens, so the next step appends after the
accepted tokens (the logits repeat because the hidden rows are fixed).

Prints one JSON line: verified positions/s (B*(K+1) per step) as `value`,
accepted (emitted) tokens/s, per-call times from HIP events on the launch
stream, the roofline fraction of the dominant call, and the CPU oracle timed
on a bounded sample of the same workload on the host cores.

Workloads (--config): 1 tiny fp32 greedy, 2 GQA bf16 sampling, 3 MLA-shaped
greedy, 4 long-context top-p, 5 ragged paged serving batch (default; the
largest configuration and the one the attention/LM-head roofline targets are
stated on).  The draft model is out of scope: drafts are synthesised from the
step's own target logits the way the workload recipe states (greedy requests
copy the target argmax for a truncated-geometric prefix, sampled requests
draw from softmax((logits + N(0, 0.5^2)) / T)).

Other modes: --graph (the step as one HIP graph), --kv-cache e4m3, --tree
binary, --flush (caches cleared before each step), --lm-operands equal (a
power diagnostic), and the two device probes --hbm-ceiling and
--mfma-ceiling, which print their own line instead of running the step.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
MFMA_F32_PEAK_TFS = 157.3

# Workload names used by the committed rocprofv3 summaries in profiles/.
WORKLOAD_NAMES = {1: "c1_tiny_fp32", 2: "c2_gqa_stochastic", 3: "c3_mla_greedy",
                  4: "c4_long_context", 5: "c5_ragged_serving"}
# Source files whose contents a kernel's PMC traffic figure is tied to.
KERNEL_SOURCES = {"lm_head_stream": "lm_head.hip", "lm_head_ring": "lm_head.hip",
                  "attn_gqa_stream": "attn_gqa.hip", "attn_gqa_f8_r16": "attn_gqa.hip",
                  "attn_mla_bf16": "attn_mla.hip", "probe_mfma_bf16": "probe_mfma.hip",
                  "probe_hbm_read": "probe_hbm.hip"}


def kernel_source_hash(kernel):
    """SHA-256 over the kernel's source file, the shared device headers and
    the hipcc flags that file is compiled with."""
    import hashlib
    from speculative_decoding_sd_amd import build as sdv_build
    h = hashlib.sha256()
    src = KERNEL_SOURCES[kernel]
    csrc = os.path.join(ROOT, "speculative_decoding_sd_amd", "csrc")
    for f in (os.path.join(csrc, src), os.path.join(csrc, "sdv_device.h"),
              os.path.join(csrc, "sdv_lds.h"), os.path.join(csrc, "sdv_internal.h")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    flags = sdv_build.HIPCC_FLAGS + sdv_build.EXTRA_FLAGS.get(src, [])
    h.update(" ".join(f for f in flags if not os.path.isabs(f)).encode())
    return h.hexdigest()


def lm_head_kernel(M, hidden, vocab, dtype, cus):
    """Name of the kernel sd_lm_head launches for this shape on a device with
    `cus` compute units (its dispatch rule: 256 x 256 tiles for more than 128
    rows while they number at least the CUs, else the streaming kernel), or
    None for the fallback paths."""
    if dtype != "bf16" or hidden % 128:
        return None
    if M > 128 and ((M + 255) // 256) * ((vocab + 255) // 256) >= cus:
        return "lm_head_ring"
    return "lm_head_stream"


def attention_kernel(mla, dtype, kv_cache, n_q_heads, n_kv_heads, num_q, d_qk):
    """Name of the attention kernel sd_verify_attn launches for this shape (its
    dispatch rule: the MLA kernel; for GQA with an E4M3 cache at head dim 128
    and 33..48 query rows per kv head the 16-row-block kernel, else the
    streaming kernel), or None for the float32 path."""
    if mla:
        return "attn_mla_bf16"
    if dtype != "bf16":
        return None
    rows = (n_q_heads // n_kv_heads) * num_q
    if kv_cache == "e4m3" and d_qk == 128 and 32 < rows <= 48:
        return "attn_gqa_f8_r16"
    return "attn_gqa_stream"


def profiled_fields(kernel, workload):
    """The machine-readable lines of the committed PMC summary of this kernel
    and workload, or {} when there is none or the kernel's sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.md")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return {}
    fields = {}
    with open(path) as fh:
        for line in fh:
            k, sep, v = line.strip().partition(": ")
            if sep:
                fields[k] = v
    if fields.get("source_sha256") != kernel_source_hash(kernel):
        return {}
    return fields


def profiled_traffic(kernel, workload):
    """HBM bytes per launch from the committed PMC summary (see
    profiled_fields), or None."""
    try:
        return float(profiled_fields(kernel, workload)["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profiled_counters(kernel, workload):
    """Shader-counter figures of the committed PMC summary: the fraction of
    the kernel's cycles the matrix pipes were busy and the clock it sustained
    (GRBM_GUI_ACTIVE per XCD over its duration), or None."""
    f = profiled_fields(kernel, workload)
    try:
        return {"mfma_busy": float(f["mfma_busy"]), "clock_ghz": float(f["clock_ghz"]),
                "source": f"profiles/{kernel}_{workload}.md"}
    except (KeyError, ValueError):
        return None


def mfma_ceiling_on_record():
    """The register-operand bf16 MFMA rate on random operands from the
    committed probe summary (bench.py --mfma-ceiling), TFLOP/s, or None."""
    f = profiled_fields("probe_mfma_bf16", "register_operands")
    try:
        return float(f["ceiling_random_tflops"])
    except (KeyError, ValueError):
        return None


def hbm_ceiling_on_record():
    """The streaming read bandwidth of the committed probe summary (bench.py
    --hbm-ceiling), GB/s, or None."""
    f = profiled_fields("probe_hbm_read", "streaming")
    try:
        return float(f["ceiling_read_gbs"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="time K replays of the step captured as one HIP graph (per-call "
                         "times still come from the eager steps before it)")
    ap.add_argument("--kv-cache", choices=("as_dtype", "e4m3"), default="as_dtype",
                    help="KV cache format: the workload's dtype (default) or FP8 E4M3 codes "
                         "with per-kv-head scales (GQA bf16 workloads)")
    ap.add_argument("--tree", choices=("binary",), default=None,
                    help="verify a tree of K+1 drafts instead of a chain (all requests "
                         "greedy; GQA workloads): the complete binary tree in "
                         "breadth-first order")
    ap.add_argument("--cpu-sample-requests", type=int, default=0,
                    help="requests timed through the CPU oracle (0: sized for about 15 s)")
    ap.add_argument("--lm-operands", choices=("random", "equal"), default="random",
                    help="diagnostic: 'equal' fills W and the LM-head input with one value "
                         "each (the same kernel on low-entropy operands, to show how its "
                         "clock depends on the data it switches; not a benchmark of the "
                         "workload)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="diagnostic: time the register-operand bf16 MFMA probe "
                         "(csrc/probe_mfma.hip) with random and with equal operands and "
                         "print its rates instead of running the verify step")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="diagnostic: time the streaming HBM read probe "
                         "(csrc/probe_hbm.hip) over a 4 GiB buffer and print its bandwidth "
                         "instead of running the verify step")
    ap.add_argument("--flush", action="store_true",
                    help="read a 1 GiB scratch buffer before every timed step, so that "
                         "neither the L2 caches nor the 256 MB MALL hold the step's inputs "
                         "(a read leaves them clean, with no write-back for the step to pay); "
                         "each step is then timed alone with HIP events")
    return ap.parse_args()


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def sampling_modes(cfg):
    """Per-request sampling modes of the workload, as a label."""
    if cfg.mixed_modes is not None:
        return f"even requests greedy, odd requests sampled at T={cfg.mixed_modes}"
    if cfg.temperature == 0:
        return "greedy"
    return f"sampled at T={cfg.temperature}"


def attention_bytes(cfg, seq_lens_before):
    """Algorithmic HBM bytes of one sd_verify_attn call: every cached and new
    key/value read once, the new rows read (q's dtype) and written once (the
    cache's element size), q read, fp32 out written."""
    es = 2 if cfg.dtype == "bf16" else 4
    es_kv = 1 if cfg.kv_cache == "e4m3" else es
    B, NQ = cfg.batch, cfg.num_q
    keys = float(np.sum(seq_lens_before.astype(np.float64) + NQ))
    if cfg.mla:
        kv = keys * cfg.d_qk * es
        new = B * NQ * cfg.d_qk * es * 2
    else:
        kv = keys * cfg.n_kv_heads * (cfg.d_qk + cfg.d_v) * es_kv
        new = B * NQ * cfg.n_kv_heads * (cfg.d_qk + cfg.d_v) * (es + es_kv)
    q = B * NQ * cfg.n_q_heads * cfg.d_qk * es
    out = B * NQ * cfg.n_q_heads * cfg.d_v * 4
    return kv + new + q + out


def attention_flops(cfg, seq_lens_before):
    """Algorithmic flops of one sd_verify_attn call: query row (i, h) of a
    request with L cached keys scores and averages L + i + 1 keys
    (2 d_qk + 2 d_v flops per key)."""
    NQ = cfg.num_q
    keys = sum(float(np.sum(seq_lens_before.astype(np.float64) + i + 1)) for i in range(NQ))
    return keys * cfg.n_q_heads * 2.0 * (cfg.d_qk + cfg.d_v)


def lm_head_work(cfg):
    es = 2 if cfg.dtype == "bf16" else 4
    M = cfg.batch * cfg.num_q
    flops = 2.0 * M * cfg.hidden * cfg.vocab
    byts = (cfg.vocab * cfg.hidden + M * cfg.hidden + M * cfg.vocab) * es
    return flops, byts


def accept_bytes(cfg):
    """Algorithmic HBM bytes of one sd_accept call, counted as its floor: every
    logits row read once (the draft-probability rows a sampled request's draw
    reads and the small per-row outputs are left out)."""
    es = 2 if cfg.dtype == "bf16" else 4
    return float(cfg.batch * cfg.num_q) * cfg.vocab * es


def synthesize_drafts(cfg, seed, logits_host_f32, temperature, top_p, tree_parent=None):
    """Draft-model stand-in from the target logits (see module docstring).
    A tree: node n copies the target token after its parent with probability
    0.6, else a token that avoids it."""
    import sdsynth
    B, Q, V = logits_host_f32.shape
    K = Q - 1
    if tree_parent is not None:
        tt = np.argmax(logits_host_f32, axis=-1)
        return (sdsynth.tree_drafts(tt, tree_parent, V, seed, p_match=1.0 - cfg.geom_p),
                np.zeros((B, K, V), np.float32))
    greedy = temperature == 0
    drafts = np.full((B, K), -1, np.int32)
    pd = np.zeros((B, K, V), np.float32)
    if greedy.any():
        tt = np.argmax(logits_host_f32, axis=-1)  # draft copies the target's top token
        dg = sdsynth.greedy_drafts(tt, K, V, seed, p=cfg.geom_p)
        drafts[greedy] = dg[greedy]
    st = np.nonzero(~greedy)[0]
    if len(st) and K > 0:
        T = float(temperature[st[0]])
        tp = float(top_p[st[0]])
        pd_st = sdsynth.draft_probs(logits_host_f32[st, :K], seed, cfg.draft_noise, T, tp)
        pd[st] = pd_st
        drafts[st] = sdsynth.sample_drafts(pd_st, seed)
    return drafts, pd


def cpu_baseline(cfg, seed, wl, host_inputs, n_req):
    """The oracle, as it stands, timed on a bounded sample of the workload:
    the first n_req requests through append + attention, LM head, accept and
    rollback.  Inputs were copied from the generator's tensors before any
    library call touched them."""
    import oracle
    import sdsynth
    t0 = time.perf_counter()
    sel = host_inputs
    timings = {}
    B = n_req
    Q = cfg.num_q
    kc, vc = sel["k_cache"], sel["v_cache"]
    s = time.perf_counter()
    tree = sel.get("tree_parent")
    tree_b = np.tile(tree, (B, 1)) if tree is not None else None
    oracle.kv_append(sel["seq_lens"], sel["page_table"], sel["num_pages"], sel["k_new"],
                     sel["v_new"], kc, vc, mla=cfg.mla, k_scale=sel["k_scale"],
                     v_scale=sel["v_scale"])
    ref_o = oracle.verify_attn(sel["q"], kc, vc, sel["page_table"], sel["seq_lens"],
                               sel["num_pages"], n_kv_heads=cfg.n_kv_heads, d_v=cfg.d_v,
                               mla=cfg.mla, k_scale=sel["k_scale"], v_scale=sel["v_scale"],
                               tree_parent=tree_b)
    timings["attention"] = time.perf_counter() - s
    H = sel["H"] if sel["H"] is not None else ref_o.reshape(B * Q, -1)
    W = sel["W"]
    if H.dtype != W.dtype:
        W = oracle.bf16_to_f64(W) if W.dtype == np.uint16 else W.astype(np.float64)
        H = H.astype(np.float64)
    s = time.perf_counter()
    exact = oracle.lm_head(H, W)
    timings["lm_head"] = time.perf_counter() - s
    logits = (oracle.round_bf16(exact) if cfg.dtype == "bf16" else exact.astype(np.float32))
    logits = logits.reshape(B, Q, cfg.vocab)
    lf = oracle.bf16_to_f64(logits) if cfg.dtype == "bf16" else logits.astype(np.float64)
    temp, top_p = wl.temperature[:B], wl.top_p[:B]
    drafts, pd = synthesize_drafts(cfg, seed, lf.astype(np.float32), temp, top_p, tree)
    s = time.perf_counter()
    acc = oracle.accept(logits, drafts, temp, top_p if (top_p < 1).any() else None, pd,
                        wl.u_accept[:B], wl.u_sample[:B], tree_parent=tree_b)
    timings["accept"] = time.perf_counter() - s
    s = time.perf_counter()
    oracle.kv_rollback(sel["page_table"], acc["num_accepted"], sel["seq_lens"], cfg.K,
                       k_cache=kc if tree is not None else None,
                       v_cache=vc if tree is not None else None, n_kv_heads=cfg.n_kv_heads,
                       d_k=cfg.d_qk, d_v=cfg.d_v, mla=cfg.mla,
                       accepted_nodes=acc["accepted_nodes"] if tree is not None else None)
    timings["rollback"] = time.perf_counter() - s
    total = sum(timings.values())
    return {"value": B * Q / total, "unit": "verified positions/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"first {B} request(s) of the same workload ({B * Q} positions) through "
                      f"append+attention, LM head, accept and rollback; per-call seconds "
                      + ", ".join(f"{k} {v:.3f}" for k, v in timings.items()),
            "wall_s": time.perf_counter() - t0}


def to_host(t):
    """Oracle-format host copy: uint16 bit patterns for bf16, float32 otherwise."""
    import torch
    import sdsynth
    if t.dtype == torch.bfloat16:
        return sdsynth.bf16_bits(t)
    return t.detach().contiguous().cpu().numpy()


def gather_sample(cfg, wl, n_req):
    """Host copies (oracle formats) of the first n_req requests' inputs, with
    their pages renumbered into a compact pool."""
    import torch
    t = wl.tensors
    Q = cfg.num_q
    pt = wl.page_table[:n_req]
    used = pt[pt >= 0]
    remap = {int(p): i for i, p in enumerate(used.tolist())}
    new_pt = np.vectorize(lambda x: remap.get(int(x), -1))(pt).astype(np.int32)
    idx = torch.tensor(used, dtype=torch.long, device=t["k_cache"].device)
    out = {"page_table": new_pt, "num_pages": len(used),
           "seq_lens": wl.seq_lens[:n_req].copy(),
           "q": to_host(t["q"][:n_req]), "k_new": to_host(t["k_new"][:n_req]),
           "v_new": to_host(t["v_new"][:n_req]) if t["v_new"] is not None else None,
           "k_cache": to_host(t["k_cache"].index_select(0, idx)),
           "v_cache": to_host(t["v_cache"].index_select(0, idx)) if t["v_cache"] is not None else None,
           "H": to_host(t["H"][: n_req * Q]) if "H" in t else None,
           "k_scale": to_host(t["k_scale"]) if "k_scale" in t else None,
           "v_scale": to_host(t["v_scale"]) if "v_scale" in t else None,
           "W": to_host(t["W"])}
    return out


def cpu_sample_size(cfg, seq_lens, budget_s=15.0):
    """Requests for the CPU-oracle sample: about budget_s of oracle work at
    the rates it reaches on 16 host cores (fp64 LM head ~50 GFLOP/s, attention
    ~24 GFLOP/s), at least one request."""
    Q = cfg.num_q
    per_req = []
    for L in seq_lens:
        lm = 2.0 * Q * cfg.hidden * cfg.vocab
        keys = sum(float(L) + i + 1 for i in range(Q))
        at = keys * cfg.n_q_heads * 2.0 * (cfg.d_qk + cfg.d_v)
        per_req.append(lm / 50e9 + at / 24e9)
    n, t = 0, 0.0
    for c in per_req:
        if n and t + c > budget_s:
            break
        n += 1
        t += c
    return n


def mfma_ceiling(warmup, steps):
    """The sustained bf16 MFMA rate of the device when only the matrix pipes
    work (csrc/probe_mfma.hip: register-resident operands, the LM head's MFMA
    order, eight waves per CU), once with random operands and once with
    equal ones.  The gap between the two is the clock the chip gives up to
    its power limit on random data; the random-operand rate is the ceiling
    any bf16 GEMM on random data meets on this device."""
    import ctypes
    import torch
    from speculative_decoding_sd_amd import build as sdv_build

    L = ctypes.CDLL(sdv_build.PROBE_LIB_PATH)
    L.sdv_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_void_p]
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 20000
    flops = blocks * 8 * iters * 16 * 32768.0
    n = 12 * 512 * 8  # bf16 operand values: 12 fragments x 512 threads x 8
    gen = torch.Generator().manual_seed(7)
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    out = {"metric": "bf16 MFMA rate, register-resident operands", "unit": "TFLOP/s",
           "peak": MFMA_BF16_PEAK_TFS, "blocks": blocks, "waves_per_cu": 8,
           "mfma_per_launch": blocks * 8 * iters * 16, "steps": steps}
    for name, host in (("random", torch.randn(n, generator=gen).to(torch.bfloat16)),
                       ("equal", torch.full((n,), 1.0, dtype=torch.bfloat16))):
        ops = host.to("cuda")

        def launch():
            rc = L.sdv_probe_mfma_bf16(ops.data_ptr(), ops.numel() * 2, sink.data_ptr(),
                                       sink.numel(), blocks, iters, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("sdv_probe_mfma_bf16 failed")

        for _ in range(warmup):
            launch()
        torch.cuda.synchronize()
        ms = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = sorted(ms)[len(ms) // 2]
        out[f"{name}_operands"] = {"tflops": flops / (t * 1e-3) / 1e12, "ms_per_launch": t,
                                   "frac_of_peak": flops / (t * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS}
    print(json.dumps(out), flush=True)


def hbm_ceiling(warmup, steps):
    """The read bandwidth a plain streaming kernel sustains from HBM
    (csrc/probe_hbm.hip: contiguous 32 KB tiles per workgroup, eight 16-byte
    loads in flight per thread, over a 4 GiB buffer that no cache holds), for
    three grid sizes;
    the best is the practical ceiling of the HBM-bound calls."""
    import ctypes
    import torch
    from speculative_decoding_sd_amd import build as sdv_build

    L = ctypes.CDLL(sdv_build.PROBE_LIB_PATH)
    L.sdv_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_bytes = 4 << 30
    buf = torch.ones(n_bytes // 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    out = {"metric": "HBM read bandwidth, streaming kernel", "unit": "GB/s",
           "peak": HBM_PEAK_GBS, "bytes_per_launch": n_bytes, "steps": steps, "grids": {}}
    best = 0.0
    for per_cu in (8, 32, 64):
        blocks = cus * per_cu
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")

        def launch():
            rc = L.sdv_probe_hbm_read(buf.data_ptr(), n_bytes, sink.data_ptr(), sink.numel(),
                                      blocks, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError("sdv_probe_hbm_read failed")

        for _ in range(warmup):
            launch()
        torch.cuda.synchronize()
        ms = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        t = sorted(ms)[len(ms) // 2]
        gbs = n_bytes / (t * 1e-3) / 1e9
        out["grids"][f"{blocks} blocks"] = {"ms_per_launch": t, "gbs": gbs}
        best = max(best, gbs)
    out["best_gbs"] = best
    out["best_frac_of_peak"] = best / HBM_PEAK_GBS
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.hbm_ceiling:
        import torch  # noqa: F401 (initialises the device for the probe)
        hbm_ceiling(args.warmup, args.steps)
        return
    if args.mfma_ceiling:
        import torch  # noqa: F401 (initialises the device for the probe)
        mfma_ceiling(args.warmup, args.steps)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the verify-step benchmark runs on one GPU only; the "
                                   "kernels shard by request, kv head or vocabulary, but "
                                   "no multi-GPU path is implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import sdsynth
    import speculative_decoding_sd_amd as sdv

    sdv.lib()  # fail loudly if the HIP library is missing
    cfg = sdsynth.CONFIGS[args.config]
    if args.kv_cache != "as_dtype":
        if cfg.mla or cfg.dtype != "bf16":
            print(json.dumps({"error": "an E4M3 KV cache needs a GQA bf16 workload",
                              "config": args.config}))
            sys.exit(2)
        cfg = dataclasses.replace(cfg, kv_cache=args.kv_cache)
    tree = None
    if args.tree:
        if cfg.mla or cfg.num_q > 64:
            print(json.dumps({"error": "a draft tree needs a GQA workload with K+1 <= 64",
                              "config": args.config}))
            sys.exit(2)
        cfg = dataclasses.replace(cfg, temperature=0.0, top_p=1.0, mixed_modes=None)
        tree = sdsynth.tree_parents(args.tree, cfg.num_q)
    seed = sdsynth.config_seed(args.config)
    workload = (WORKLOAD_NAMES[args.config] + ("_e4m3" if cfg.kv_cache == "e4m3" else "") +
                ("_tree" if tree is not None else "") +
                ("_equal_operands" if args.lm_operands == "equal" else ""))
    dev = torch.device("cuda", 0)
    extra = (args.warmup + (2 if args.graph else 1) * args.steps + 4) * cfg.num_q
    wl = sdsynth.make_workload(cfg, seed, device=dev, extra_tokens=extra)
    sample = None
    n_cpu = args.cpu_sample_requests or cpu_sample_size(cfg, wl.seq_lens)
    if not args.no_cpu_baseline:
        sample = gather_sample(cfg, wl, n_cpu)
        sample["tree_parent"] = tree
    t = wl.tensors
    if args.lm_operands == "equal":
        t["W"].fill_(0.02)
        if "H" in t:
            t["H"].fill_(1.0)
    L0 = wl.seq_lens.copy()
    seq_lens = torch.tensor(wl.seq_lens, device=dev)
    page_table = torch.tensor(wl.page_table, device=dev)
    temp = torch.tensor(wl.temperature, device=dev)
    top_p = torch.tensor(wl.top_p, device=dev) if (wl.top_p < 1).any() else None
    ua = torch.tensor(wl.u_accept, device=dev)
    us = torch.tensor(wl.u_sample, device=dev)
    drafts = torch.full((cfg.batch, cfg.K), -1, dtype=torch.int32, device=dev)
    pd = torch.zeros((cfg.batch, cfg.K, cfg.vocab), dtype=torch.float32, device=dev)
    step = sdv.VerifyStep(q=t["q"], k_cache=t["k_cache"], v_cache=t["v_cache"],
                          page_table=page_table, seq_lens=seq_lens, num_pages=wl.num_pages,
                          max_seq_len=int(L0.max()) + extra - cfg.num_q,
                          n_kv_heads=cfg.n_kv_heads, W=t["W"], drafts=drafts, temperature=temp,
                          u_accept=ua, u_sample=us, k_new=t["k_new"], v_new=t["v_new"],
                          mla=cfg.mla, d_v=cfg.d_v, H=t.get("H"), top_p=top_p,
                          draft_probs=pd if (wl.temperature > 0).any() else None,
                          k_scale=t.get("k_scale"), v_scale=t.get("v_scale"),
                          tree_parent=(torch.tensor(np.tile(tree, (cfg.batch, 1)), device=dev)
                                       if tree is not None else None))
    # Target logits of the first step -> synthetic drafts (outside the timed region).
    step.attention()
    step.lm_head()
    torch.cuda.synchronize()
    lg = step.logits.float().cpu().numpy()
    d_h, pd_h = synthesize_drafts(cfg, seed, lg, wl.temperature, wl.top_p, tree)
    drafts.copy_(torch.from_numpy(d_h))
    pd.copy_(torch.from_numpy(pd_h))
    del lg, pd_h
    seq_lens.copy_(torch.from_numpy(L0))
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    L_start = seq_lens.cpu().numpy().copy()
    names = ["attention", "lm_head", "accept", "rollback"]
    calls = [step.attention, step.lm_head, step.accept, step.rollback]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    acc_total = 0
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev) if args.flush else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if scratch is not None:
            scratch.max()             # reads 1 GiB: evicts the step's inputs from L2 and MALL
        ev[k][0].record()
        for c, fn in enumerate(calls):
            fn()
            ev[k][c + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / args.steps
    per_call = {n: float(np.mean([ev[k][c].elapsed_time(ev[k][c + 1]) for k in range(args.steps)]))
                for c, n in enumerate(names)}
    ev_step_ms = float(np.mean([ev[k][0].elapsed_time(ev[k][4]) for k in range(args.steps)]))
    if scratch is not None:
        # The flush is not part of the step: the step time is the events'.
        wall_ms = ev_step_ms
        del scratch
    L_end = seq_lens.cpu().numpy()
    emitted = int(step.out_offsets[-1].item())
    acc_total = (L_end - L_start).sum()  # j_b + 1 per request per step
    n_err = int(step.dev_error.item())
    ms = wall_ms
    eager_ms = wall_ms
    if args.graph:
        # The same step as one graph launch: capture, one untimed replay, then
        # K timed replays.  Each replay continues from the previous state.
        step.capture()
        step.replay()
        torch.cuda.synchronize()
        Lg0 = seq_lens.cpu().numpy().copy()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        acc_total = (seq_lens.cpu().numpy() - Lg0).sum()
        n_err = int(step.dev_error.item())
    B, Q = cfg.batch, cfg.num_q
    pos_per_s = B * Q / (ms * 1e-3)
    tok_per_s = acc_total / args.steps / (ms * 1e-3)
    # Rooflines per call (attention bytes at the mean lengths seen in the timed steps).
    L_mid = (L_start + L_end) / 2.0
    a_bytes = attention_bytes(cfg, L_mid)
    f, lm_bytes = lm_head_work(cfg)
    lm_bound = "mfma" if f / lm_bytes > MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
    a_flops = attention_flops(cfg, L_mid)
    attn_ms = per_call["attention"]
    # The attention's bound follows its arithmetic intensity: the MLA shape
    # (all heads share one latent row) sits above the MFMA/HBM ridge.
    if a_flops / a_bytes > MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9):
        attn_roof = {"bound": "mfma", "achieved": a_flops / (attn_ms * 1e-3) / 1e12,
                     "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "flops": a_flops,
                     "bytes": a_bytes}
    else:
        attn_roof = {"bound": "hbm", "achieved": a_bytes / (attn_ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes": a_bytes, "flops": a_flops}
    kernels = {
        "attention": attn_roof,
        "lm_head": ({"bound": "mfma", "achieved": f / (per_call["lm_head"] * 1e-3) / 1e12,
                     "peak": MFMA_BF16_PEAK_TFS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFS,
                     "unit": "TFLOP/s", "flops": f}
                    if lm_bound == "mfma" else
                    {"bound": "hbm", "achieved": lm_bytes / (per_call["lm_head"] * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes": lm_bytes}),
        "accept": {"bound": "hbm", "achieved": accept_bytes(cfg) / (per_call["accept"] * 1e-3) / 1e9,
                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes": accept_bytes(cfg)},
    }
    for k, v in kernels.items():
        v["frac"] = v["achieved"] / v["peak"]
        v["ms"] = per_call[k]
    # Whole step against its floor: every call at its own bound's peak.
    floor_ms = 0.0
    for k, v in kernels.items():
        work = v.get("flops") if v["bound"] == "mfma" else v.get("bytes")
        peak = v["peak"] * (1e12 if v["unit"] == "TFLOP/s" else 1e9)
        floor_ms += work / peak * 1e3
    step_roof = {"floor_ms": floor_ms, "ms": ev_step_ms, "frac": floor_ms / ev_step_ms,
                 "note": "sum over attention, LM head and accept of algorithmic work / peak "
                         "at each call's bound (rollback: negligible bytes), over the event "
                         "time of the four calls"}
    dom = max(("attention", "lm_head"), key=lambda k: per_call[k])
    roof = dict(kernels[dom])
    if dom == "lm_head":
        cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
        dom_kernel = lm_head_kernel(cfg.batch * cfg.num_q, cfg.hidden, cfg.vocab, cfg.dtype, cus)
    else:
        dom_kernel = attention_kernel(cfg.mla, cfg.dtype, cfg.kv_cache, cfg.n_q_heads,
                                      cfg.n_kv_heads, cfg.num_q, cfg.d_qk)
    traffic = profiled_traffic(dom_kernel, workload) if dom_kernel else None
    counters = profiled_counters(dom_kernel, workload) if dom_kernel else None
    roof = {"kernel": dom, "bound": roof["bound"], "achieved": roof["achieved"],
            "peak": roof["peak"], "unit": roof["unit"], "frac": roof["frac"], "traffic": traffic,
            "counters": counters}
    hbm_ceil = hbm_ceiling_on_record() if roof["bound"] == "hbm" else None
    if hbm_ceil is not None:
        roof["hbm_ceiling"] = {
            "achieved_frac": roof["achieved"] / hbm_ceil, "gbs": hbm_ceil,
            "what": "read bandwidth of a plain streaming kernel over a 4 GiB buffer on this "
                    "device",
            "source": "profiles/probe_hbm_read_streaming.md"}
    ceiling = mfma_ceiling_on_record() if roof["bound"] == "mfma" else None
    if ceiling is not None:
        roof["power_ceiling"] = {
            "achieved_frac": roof["achieved"] / ceiling, "tflops": ceiling,
            "what": "bf16 MFMA rate with register-resident random operands on this device "
                    "(no memory traffic; the chip's clock under its power limit)",
            "source": "profiles/probe_mfma_bf16_register_operands.md"}
    line = {
        "metric": "verified positions/sec", "value": pos_per_s, "unit": "positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"C{args.config} {cfg.name}" + (
                       ", E4M3 KV cache" if cfg.kv_cache == "e4m3" else "") + (
                       f", greedy {args.tree} draft tree" if tree is not None else ""),
                   "batch": B, "K": cfg.K,
                   "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.d_qk, "kv_len": (int(cfg.seq_len) if cfg.seq_len
                                                    else list(cfg.seq_len_range)),
                   "mean_kv_len": float(L_mid.mean()), "hidden": cfg.hidden,
                   "vocab": cfg.vocab, "sampling": sampling_modes(cfg),
                   "top_p": cfg.top_p, "page_size": cfg.page_size,
                   "l2_mall_flush": bool(args.flush),
                   "lm_operands": args.lm_operands,
                   "kv_cache": "e4m3" if cfg.kv_cache == "e4m3" else cfg.dtype,
                   "drafts": (f"{args.tree} tree of {cfg.num_q} nodes" if tree is not None
                              else f"chain of {cfg.K}")},
        "accepted_tokens_per_sec": tok_per_s,
        "mean_emitted_per_request": acc_total / args.steps / B,
        "event_ms_per_step": ev_step_ms,
        "graph": bool(args.graph),
        "eager_ms_per_step": eager_ms,
        "per_call_ms": per_call,
        "roofline": roof,
        "step_roofline": step_roof,
        "kernels": kernels,
        "device_error": n_err,
        "last_step_emitted": emitted,
    }
    if sample is not None:
        line["cpu_baseline"] = cpu_baseline(cfg, seed, wl, sample, n_cpu)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""The allocation-free acceptance entry point (sd_accept_noalloc) against
sd_accept, through the C ABI: two calls in a row on one GPU, the second on a
smaller batch (the fixed scratch keeps the first call's contents), each
compared with sd_accept on the same inputs, every output bit for bit."""
import numpy as np
import pytest
import torch

import sdsynth
import speculative_decoding_sd_amd as sdv
from parity import DEV

pytestmark = pytest.mark.gpu


def _inputs(B, K, V, seed, dtype):
    rng = np.random.default_rng(seed)
    Q = K + 1
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    lg = (torch.randn((B, Q, V), generator=torch.Generator().manual_seed(seed)) * 1.7).to(tdt)
    lg_f = lg.float().numpy()
    temp = np.where(np.arange(B) % 2 == 0, 0.0, 0.8).astype(np.float32)
    top_p = np.where(np.arange(B) % 4 == 3, 0.9, 1.0).astype(np.float32)
    pd = sdsynth.draft_probs(lg_f[:, :K], seed, 0.5, 0.8, 1.0)
    drafts = sdsynth.sample_drafts(pd, seed)
    tt = np.argmax(lg_f, axis=-1)
    greedy = sdsynth.greedy_drafts(tt, K, V, seed, p=0.4)
    drafts[temp == 0] = greedy[temp == 0]
    ua = rng.random((B, Q)).astype(np.float32)
    us = rng.random((B, Q)).astype(np.float32)
    t = lambda x: torch.tensor(x, device=DEV)
    return dict(logits=lg.to(DEV), draft_tokens=t(drafts), temperature=t(temp), top_p=t(top_p),
                draft_probs=t(pd), u_accept=t(ua), u_sample=t(us))


def _call(inp, noalloc):
    B, Q, V = inp["logits"].shape
    i32 = dict(dtype=torch.int32, device=DEV)
    out = dict(num_accepted=torch.full((B,), -7, **i32), out_tokens=torch.full((B, Q), -7, **i32),
               next_token=torch.full((B,), -7, **i32), out_offsets=torch.full((B + 1,), -7, **i32),
               packed_tokens=torch.full((B * Q,), -7, **i32))
    err = torch.zeros(1, **i32)
    d = sdv.accept_desc(dev_error=err, **inp, **out)
    stream = sdv.current_stream()
    if noalloc:
        sdv.sd_accept_noalloc(d, stream)
    else:
        sdv.accept(d)
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["dev_error"] = sdv.device_error(err, stream)
    return res


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_accept_matches_sd_accept(dtype):
    for B, K, V, seed in ((64, 5, 32000, 11), (9, 3, 5003, 12)):   # large, then smaller
        print(f"noalloc accept: B={B} K={K} V={V} {dtype}", flush=True)
        inp = _inputs(B, K, V, seed, dtype)
        ref = _call(inp, noalloc=False)
        got = _call(inp, noalloc=True)
        assert ref["dev_error"] == 0 and got["dev_error"] == 0
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (B, k)
        assert (ref["num_accepted"] >= 0).all()

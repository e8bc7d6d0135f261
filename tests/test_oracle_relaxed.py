"""Pins of the oracle's relaxed acceptance ([TRT-MTP] "寬松接受", Fig. 6):
top-N candidates of the target row, those whose softmax probability is
below (top-1 probability - delta) dropped, a draft accepted if it is a
surviving candidate; the final token stays the argmax of row j.

The hand example's probabilities are worked out in the comments from the
softmax definition; the other tests are special cases (N = 1 is the strict
rule, N = V with delta = 1 accepts every draft), monotonicity in N and
delta, the tie order at the N-th place and parameter validation."""
import numpy as np
import pytest


def _run(orc, logits, drafts, N, delta, T=None):
    B, Q, V = logits.shape
    K = Q - 1
    T = np.zeros(B, np.float32) if T is None else np.asarray(T, np.float32)
    u = np.zeros((B, Q), np.float32)
    rk = None if N is None else np.broadcast_to(np.asarray(N, np.int32), (B,)).copy()
    rd = None if delta is None else np.broadcast_to(np.asarray(delta, np.float32), (B,)).copy()
    pd = np.full((B, K, V), 1.0 / V, np.float32) if (T > 0).any() else None
    return orc.accept(logits.astype(np.float32), np.asarray(drafts, np.int32).reshape(B, K), T,
                      None, pd, u, u, relaxed_topk=rk, relaxed_delta=rd)


def _hand_logits():
    # Row 0: m = 2, e = [1, e^-1, e^-2, e^-3, e^-4] = [1, .367879, .135335, .049787,
    #   .018316], Z = 1.571317, p = [.636409, .234122, .086129, .031685, .011656].
    # Row 1: m = 3, e = [e^-3, 1, e^-.5, e^-2, e^-4] = [.049787, 1, .606531, .135335,
    #   .018316], Z = 1.809969, p = [.027507, .552496, .335106, .074772, .010119].
    # Row 2: m = 5, p_4 = 1 / (1 + 2e^-4 + 2e^-5) = .952284, p_0 = p_1 = .017442.
    # Row 3: uniform.
    return np.array([[[2, 1, 0, -1, -2], [0, 3, 2.5, 1, -1], [1, 1, 0, 0, 5],
                      [0, 0, 0, 0, 0]]], np.float32)


def test_hand_example_top3_delta045(orc):
    lg = _hand_logits()
    # delta = .45: row 0 keeps p >= .186409 -> {0, 1}: draft 1 accepted;
    # row 1 keeps p >= .102496 among top-3 {1, 2, 3} -> {1, 2}: draft 2 accepted
    # (strict would reject it: the argmax is 1); row 2 keeps p >= .502284 -> {4}:
    # draft 0 rejected.  j = 2, final token = argmax of row 2 = 4.
    out = _run(orc, lg, [[1, 2, 0]], 3, 0.45)
    assert int(out["num_accepted"][0]) == 2
    assert list(out["out_tokens"][0]) == [1, 2, 4, -1]
    assert int(out["next_token"][0]) == 4
    strict = _run(orc, lg, [[1, 2, 0]], None, None)
    assert int(strict["num_accepted"][0]) == 0
    assert list(strict["out_tokens"][0]) == [0, -1, -1, -1]


def test_hand_example_thresholds(orc):
    lg = _hand_logits()[:, [0, 3]]      # row 0 judges the single draft
    # delta = .45: threshold .186409 -> token 2 (p .086129) dropped.
    assert int(_run(orc, lg, [[2]], 3, 0.45)["num_accepted"][0]) == 0
    # delta = .6: threshold .036409 -> top-3 {0, 1, 2} all kept.
    assert int(_run(orc, lg, [[2]], 3, 0.6)["num_accepted"][0]) == 1
    # token 3 (p .031685) is rank 3: outside the top 3 whatever delta is.
    assert int(_run(orc, lg, [[3]], 3, 1.0)["num_accepted"][0]) == 0
    # N = 5, delta = .61: threshold .026409 -> token 3 kept, token 4 (.011656) dropped.
    assert int(_run(orc, lg, [[3]], 5, 0.61)["num_accepted"][0]) == 1
    assert int(_run(orc, lg, [[4]], 5, 0.61)["num_accepted"][0]) == 0
    # delta = 0: only the maximum survives, as in the strict rule.
    assert int(_run(orc, lg, [[1]], 5, 0.0)["num_accepted"][0]) == 0
    assert int(_run(orc, lg, [[0]], 5, 0.0)["num_accepted"][0]) == 1


def test_tie_at_the_nth_place_goes_by_token_id(orc):
    # Logits [3, 1, 1, 1, 0]: ranking by (logit desc, id asc) is 0, 1, 2, 3, 4.
    lg = np.array([[[3, 1, 1, 1, 0], [0, 0, 0, 0, 0]]], np.float32)
    assert int(_run(orc, lg, [[1]], 2, 1.0)["num_accepted"][0]) == 1
    assert int(_run(orc, lg, [[2]], 2, 1.0)["num_accepted"][0]) == 0
    assert int(_run(orc, lg, [[2]], 3, 1.0)["num_accepted"][0]) == 1


def _random_case(seed, B=40, K=4, V=48):
    rng = np.random.default_rng(seed)
    lg = rng.normal(0, 1.5, (B, K + 1, V)).astype(np.float32)
    order = np.argsort(-lg, axis=-1, kind="stable")
    # Drafts from each row's top 4 (so relaxed rules matter), some random.
    pick = order[:, :K, :][np.arange(B)[:, None], np.arange(K)[None, :],
                           rng.integers(0, 4, (B, K))]
    rand = rng.integers(0, V, (B, K))
    drafts = np.where(rng.random((B, K)) < 0.8, pick, rand).astype(np.int32)
    return lg, drafts


@pytest.mark.parametrize("delta", [0.0, 0.3, 1.0])
def test_top1_is_the_strict_rule(orc, delta):
    lg, drafts = _random_case(7)
    strict = _run(orc, lg, drafts, None, None)
    relaxed = _run(orc, lg, drafts, 1, delta)
    for k in ("num_accepted", "out_tokens", "next_token", "packed", "out_offsets"):
        assert np.array_equal(strict[k], relaxed[k]), k


def test_topV_delta1_accepts_every_draft(orc):
    lg, drafts = _random_case(8)
    B, Q, V = lg.shape
    drafts[3, 2] = -1                       # a negative id still ends the chain
    out = _run(orc, lg, drafts, V, 1.0)
    want = np.full(B, Q - 1)
    want[3] = 2
    assert np.array_equal(out["num_accepted"], want)
    am = np.argmax(lg, axis=-1)             # distinct maxima with continuous logits
    assert np.array_equal(out["next_token"], am[np.arange(B), want])


def test_monotone_in_topk_and_delta(orc):
    lg, drafts = _random_case(9)
    prev = _run(orc, lg, drafts, None, None)["num_accepted"]
    for N, delta in [(1, 0.0), (2, 0.1), (3, 0.3), (5, 0.3), (5, 0.6), (10, 0.6), (48, 0.9)]:
        j = _run(orc, lg, drafts, N, delta)["num_accepted"]
        assert (j >= prev).all(), (N, delta)
        prev = j
    assert prev.sum() > _run(orc, lg, drafts, None, None)["num_accepted"].sum()


def test_parameter_validation(orc):
    lg, drafts = _random_case(10, B=4)
    out = _run(orc, lg, drafts, [3, -1, 3, 0], [0.5, 0.5, np.nan, np.nan])
    assert list(out["num_accepted"][[1, 2]]) == [-1, -1]     # N < 0; bad delta
    assert out["num_accepted"][0] >= 0 and out["num_accepted"][3] >= 0   # N = 0: strict
    assert out["n_invalid"] == 2
    # Sampled requests ignore the relaxed parameters.
    T = np.array([0.8, 0.8, 0.8, 0.8], np.float32)
    a = _run(orc, lg, drafts, 3, 0.5, T=T)
    b = _run(orc, lg, drafts, None, None, T=T)
    assert np.array_equal(a["out_tokens"], b["out_tokens"])

"""Pins of the rejection-sampling rule's edge branches (CPU only).

[SD-PRACTICE] s4.4 and [VLLM-MTP] s3 stage 3 accept draft d with probability
min(1, p_t(d) / p_d(d)) and, on a rejection, draw the replacement from
norm(max(0, p_t - p_d)).  Three branches of that rule are reached only by
inputs the workload generator never produces, so they are injected here:

  * p_d(d) = 0: the ratio is +inf when p_t(d) > 0 (always accepted) and 0
    when p_t(d) = 0 as well (always rejected);
  * an all-zero residual (p_d >= p_t everywhere, which a rejection allows
    only through rounding): the replacement is drawn from p_t itself;
  * a draw whose running sum never exceeds u * S (u = 1, the one uniform at
    which no rounding is needed to get there): the largest id with positive
    weight.

Each expected value is worked out by hand from the definitions.  The same
constructions, at larger vocabularies, are the GPU parity cases of these
branches (tests/test_gpu_accept_edges.py).
"""
import numpy as np

U_MAX = np.float32(1.0) - np.float32(2.0 ** -24)  # largest float32 below 1


def _run(orc, logits, drafts, temp, top_p, pd, ua, us):
    return orc.accept(np.asarray(logits, np.float64)[None], np.asarray(drafts, np.int32)[None],
                      np.array([temp], np.float32), np.array([top_p], np.float32),
                      None if pd is None else np.asarray(pd, np.float32)[None],
                      np.asarray(ua, np.float32)[None], np.asarray(us, np.float32)[None])


def test_zero_draft_probability_with_positive_target_is_accepted(orc):
    # Row 0: p_t = softmax([0, 1, 2, 3]); the draft is token 1 with p_d(1) = 0.
    # ratio = +inf, so even u = 1 - 2^-24 accepts it.  Row 1 (draft 2 = token
    # 0, again p_d = 0) is accepted the same way, and the bonus token is drawn
    # from p_t of row 2 = softmax([5, 0, 0, 0]) with u = 0.5: token 0 (mass
    # 0.98).
    logits = [[0, 1, 2, 3], [3, 2, 1, 0], [5, 0, 0, 0]]
    pd = [[0.5, 0.0, 0.5, 0.0], [0.0, 0.2, 0.3, 0.5]]
    out = _run(orc, logits, [1, 0], 1.0, 1.0, pd, [U_MAX] * 3, [0.5] * 3)
    assert out["num_accepted"][0] == 2
    assert list(out["out_tokens"][0]) == [1, 0, 0]


def test_zero_draft_probability_with_zero_target_is_rejected(orc):
    # T = 1, top_p = 0.5 over logits [2, 1, 0, -5]: token 0 alone holds
    # e^2 / (e^2 + e + 1 + e^-5) = 0.665 >= 0.5, so p_t = [1, 0, 0, 0].  The
    # draft is token 2 with p_d(2) = 0 and p_t(2) = 0: ratio 0, rejected even
    # at u = 0.  Residual max(0, p_t - p_d) = [0.5, 0, 0, 0]: token 0 for any u.
    logits = [[2, 1, 0, -5], [0, 0, 0, 0]]
    pd = [[0.5, 0.5, 0.0, 0.0]]
    for u_s in (0.0, 0.5, float(U_MAX)):
        out = _run(orc, logits, [2], 1.0, 0.5, pd, [0.0, 0.0], [u_s, u_s])
        assert out["num_accepted"][0] == 0
        assert list(out["out_tokens"][0]) == [0, -1]
    # Without the nucleus p_t(2) = 1 / (e^2 + e + 1 + e^-5) > 0: the same
    # draft is now accepted at any u (p_d(2) = 0).
    out = _run(orc, logits, [2], 1.0, 1.0, pd, [U_MAX, 0.0], [0.0, 0.0])
    assert out["num_accepted"][0] == 1


def test_all_zero_residual_draws_from_the_target(orc):
    # Equal logits: p_t = 1/4 exactly.  p_d = the next float32 above 1/4 for
    # every token, so p_d > p_t everywhere and ratio = 1 / (1 + 2^-23) <
    # 1 - 2^-24 = u: the draft is rejected although max(0, p_t - p_d) is zero
    # everywhere.  The replacement then comes from p_t: with u = 0.3 the
    # running sums 0.25, 0.5 first exceed 0.3 at token 1 (the rejected draft
    # itself).  Drawing from p_t with the draft removed would give token 0;
    # an unguarded draw from the empty residual finds no bucket at all.
    up = np.nextafter(np.float32(0.25), np.float32(1.0))
    logits = [[0, 0, 0, 0], [0, 0, 0, 0]]
    pd = [[up] * 4]
    out = _run(orc, logits, [1], 1.0, 1.0, pd, [U_MAX, 0.0], [0.3, 0.0])
    assert out["num_accepted"][0] == 0
    assert list(out["out_tokens"][0]) == [1, -1]
    for u_s, f in ((0.0, 0), (0.2, 0), (0.6, 2), (0.9, 3)):
        out = _run(orc, logits, [1], 1.0, 1.0, pd, [U_MAX, 0.0], [u_s, 0.0])
        assert out["next_token"][0] == f, (u_s, out["next_token"])


def test_draw_without_crossing_takes_the_largest_positive_id(orc):
    # T = 1, top_p = 0.9 over [0, 3, 1, -9, -9]: masses 0.844 (token 1), then
    # 0.958 with token 2 -> the nucleus is {1, 2}.  With u = 1 the running sum
    # never exceeds u * S, and the draw takes the largest id of positive
    # weight: token 2 (not V - 1 = 4, outside the nucleus).
    logits = [[0, 3, 1, -9, -9]]
    out = _run(orc, logits, np.zeros(0, np.int32), 1.0, 0.9, None, [0.0], [1.0])
    assert out["num_accepted"][0] == 0 and out["next_token"][0] == 2
    # Just below 1 the crossing is found in the ordinary way, at the same token.
    out = _run(orc, logits, np.zeros(0, np.int32), 1.0, 0.9, None, [0.0], [U_MAX])
    assert out["next_token"][0] == 2
    # The residual of a rejected draft: the draft (token 4, one-hot p_d,
    # outside the nucleus) is rejected, the residual equals p_t, and u = 1
    # again lands on token 2.
    logits2 = [[0, 3, 1, -9, -9], [0, 0, 0, 0, 0]]
    out = _run(orc, logits2, [4], 1.0, 0.9, [[0, 0, 0, 0, 1]], [0.0, 0.0], [1.0, 0.0])
    assert out["num_accepted"][0] == 0 and out["next_token"][0] == 2

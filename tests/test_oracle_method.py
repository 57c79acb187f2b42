"""Pins of the oracle's whole verify-and-resample step (CPU only).

What the pages fix, and how each is checked:
  * acceptance sum_v min(p, q) = 0.8 on the worked example and outputs
    distributed as the target (roadtointelligence "Speculative Decoding",
    "Why the output doesn't change");
  * expected tokens per target pass (1 - a^(K+1)) / (1 - a) under i.i.d.
    acceptance, printed as 3.36 for a = 0.8, K = 4 (same page, "How much
    faster");
  * the output law of the step equals the target's (the paperlayer.ai
    summary's Theorem 1; FDE Interviews section 01): brute-force
    enumeration with exact fractions for V <= 4, K <= 2;
  * each round emits 1..K+1 tokens, accepted tokens are the draft prefix,
    the first rejection stops the round, a full acceptance adds a bonus
    (paperlayer.ai "Modified Rejection Sampling"; roadtointelligence
    "Draft, then verify");
  * greedy decoding reduces to the textbook rule: longest prefix agreeing
    with the target's argmax, then the target's argmax.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
WE = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
ET = json.load(open(os.path.join(GOLDEN, "expected_tokens.json")))
Q = np.array(WE["target_q"])
P = np.array(WE["draft_p"])


def worked_inputs(B, K=4):
    tq = np.log(Q).astype(np.float32)
    tp = np.log(P).astype(np.float32)
    target = np.broadcast_to(tq, (B, K + 1, 4)).copy()
    draft = np.broadcast_to(tp, (B, K, 4)).copy()
    toks = oracle.sample_rows(draft, seed=1001)
    return target, draft, toks.astype(np.int32)


@pytest.fixture(scope="module")
def worked_run():
    B = 1_000_000
    target, draft, toks = worked_inputs(B)
    res = oracle.verify(target, draft, toks, seed=1)
    return toks, res


def test_worked_example_acceptance_sum():
    assert np.minimum(P, Q).sum() == pytest.approx(WE["acceptance_sum_min"], abs=1e-12)
    np.testing.assert_allclose(np.minimum(P, Q), WE["acceptance_terms"], atol=1e-12)


def test_worked_example_draft_tokens_follow_p(worked_run):
    toks, _ = worked_run
    counts = np.bincount(toks.ravel(), minlength=4)
    stat, pval = stats.chisquare(counts, P * toks.size)
    assert pval > 1e-3


def test_worked_example_per_position_acceptance(worked_run):
    _, res = worked_run
    n = res["accepted"]
    for t in range(4):
        reached = np.count_nonzero(n >= t)
        acc = np.count_nonzero(n > t) / reached
        se = np.sqrt(0.8 * 0.2 / reached)
        assert abs(acc - 0.8) < 4 * se, (t, acc)


def test_worked_example_accepted_count_law(worked_run):
    _, res = worked_run
    n = res["accepted"]
    a = 0.8
    law = np.array([a**k * (1 - a) for k in range(4)] + [a**4])
    np.testing.assert_allclose(law, [0.2, 0.16, 0.128, 0.1024, 0.4096], atol=1e-12)
    counts = np.bincount(n, minlength=5)
    stat, pval = stats.chisquare(counts, law * n.size)
    assert pval > 1e-3


def test_expected_tokens_per_pass_closed_form(worked_run):
    _, res = worked_run
    a, g, c = ET["alpha"], ET["gamma"], ET["c"]
    e_tokens = (1 - a ** (g + 1)) / (1 - a)
    speedup = e_tokens / (g * c + 1)
    assert round(e_tokens, ET["printed_decimals"]["tokens_per_pass"]) == ET["printed_tokens_per_pass"]
    assert round(speedup, ET["printed_decimals"]["speedup"]) == ET["printed_speedup"]
    emitted = res["accepted"] + 1
    se = emitted.std() / np.sqrt(emitted.size)
    assert abs(emitted.mean() - e_tokens) < 4 * se


def test_worked_example_first_token_follows_target(worked_run):
    _, res = worked_run
    first = res["out_tokens"][:, 0]
    counts = np.bincount(first, minlength=4)
    stat, pval = stats.chisquare(counts, Q * first.size)
    assert stat < 11.34 or pval > 0.01


def test_worked_example_pooled_tokens_follow_target(worked_run):
    _, res = worked_run
    # Every emitted position i (given it is emitted) is marginally ~ q.
    out = res["out_tokens"]
    for i in range(5):
        col = out[:, i]
        col = col[col >= 0]
        counts = np.bincount(col, minlength=4)
        stat, pval = stats.chisquare(counts, Q * col.size)
        assert pval > 1e-3, i


def test_worked_example_every_rejection_emits_token_0(worked_run):
    _, res = worked_run
    n = res["accepted"]
    rej = n < 4
    y = res["out_tokens"][np.arange(n.size), n]
    # (q - p)+ = [0.2, 0, 0, 0]: the residual has a single token
    assert np.all(y[rej] == 0)


def test_emission_invariants(worked_run):
    toks, res = worked_run
    n = res["accepted"]
    out = res["out_tokens"]
    assert n.min() >= 0 and n.max() <= 4
    idx = np.arange(5)[None, :]
    assert np.all(out[idx > n[:, None]] == -1)
    assert np.all(out[idx <= n[:, None]] >= 0)
    prefix = idx[:, :4] < n[:, None]
    assert np.all(out[:, :4][prefix] == toks[prefix])
    assert np.all(res["row_status"] == 0)


def _exact_law(qs, ps):
    """P(n = k, emitted tokens = seq) for fixed per-position distributions.

    Accepting d_t at position t has probability p_t(d_t) * min(1, q_t/p_t) =
    min(p_t(d_t), q_t(d_t)); a rejection at k then emits v with probability
    (q_k - p_k)+(v); after K acceptances the bonus is v ~ q_K.
    """
    K = len(ps)
    V = len(qs[0])
    law = {}
    for k in range(K + 1):
        for prefix in itertools.product(range(V), repeat=k):
            pr = Fraction(1)
            for t, d in enumerate(prefix):
                pr *= min(ps[t][d], qs[t][d])
            for v in range(V):
                r = max(Fraction(0), qs[k][v] - ps[k][v]) if k < K else qs[K][v]
                if pr * r > 0:
                    law[(k,) + prefix + (v,)] = pr * r
    return law


ENUM_CASES = [
    # (target rows q_0..q_K, draft rows p_0..p_{K-1}) as exact fractions
    ([[Fraction(1, 2), Fraction(1, 4), Fraction(1, 8), Fraction(1, 8)],
      [Fraction(1, 10), Fraction(2, 10), Fraction(3, 10), Fraction(4, 10)],
      [Fraction(1, 4)] * 4],
     [[Fraction(1, 8), Fraction(1, 8), Fraction(1, 4), Fraction(1, 2)],
      [Fraction(3, 10), Fraction(3, 10), Fraction(2, 10), Fraction(2, 10)]]),
    ([[Fraction(2, 3), Fraction(1, 3), Fraction(0)],
      [Fraction(1, 5), Fraction(1, 5), Fraction(3, 5)]],
     [[Fraction(0), Fraction(1, 2), Fraction(1, 2)]]),
]


@pytest.mark.parametrize("case", range(len(ENUM_CASES)))
def test_output_law_matches_exact_enumeration(case):
    qs, ps = ENUM_CASES[case]
    K, V = len(ps), len(qs[0])
    law = _exact_law(qs, ps)
    assert sum(law.values()) == 1
    # Theorem 1: the first emitted token is distributed as q_0.
    for v in range(V):
        assert sum(pr for key, pr in law.items() if key[1] == v) == qs[0][v]

    def logits(rows):
        with np.errstate(divide="ignore"):
            return np.log(np.array([[float(x) for x in r] for r in rows])).astype(np.float32)

    B = 400_000
    target = np.broadcast_to(logits(qs), (B, K + 1, V)).copy()
    draft = np.broadcast_to(logits(ps), (B, K, V)).copy()
    toks = oracle.sample_rows(draft, seed=77 + case).astype(np.int32)
    res = oracle.verify(target, draft, toks, seed=5 + case)
    assert np.all(res["row_status"] & oracle.ST_ERRORS == 0)
    keys = list(law.keys())
    index = {k: i for i, k in enumerate(keys)}
    counts = np.zeros(len(keys))
    for b in range(B):
        n = int(res["accepted"][b])
        key = (n,) + tuple(int(x) for x in res["out_tokens"][b, :n + 1])
        counts[index[key]] += 1  # a KeyError means an outcome of probability 0
    expected = np.array([float(law[k]) for k in keys]) * B
    stat, pval = stats.chisquare(counts, expected)
    assert pval > 1e-3, (stat, pval)


def test_non_iid_expected_tokens_per_round():
    # Fresh logits per round (target N(0, 3^2), draft = target + N(0, 1)):
    # E[n + 1 | logits] = sum_k P(n >= k), P(n >= k) = prod_{t<k} alpha_t,
    # alpha_t = sum_v min(p_t(v), q_t(v)); alpha from torch's softmax.
    rng = np.random.default_rng(21)
    B, K, V = 20000, 4, 64
    t32 = (rng.standard_normal((B, K + 1, V)) * 3).astype(np.float32)
    d32 = (t32[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    toks = oracle.sample_rows(d32, seed=99).astype(np.int32)
    res = oracle.verify(t32, d32, toks, seed=3)
    q = torch.softmax(torch.from_numpy(t32[:, :K].astype(np.float64)), -1)
    p = torch.softmax(torch.from_numpy(d32.astype(np.float64)), -1)
    alpha = torch.minimum(p, q).sum(-1).numpy()  # [B][K]
    reach = np.concatenate([np.ones((B, 1)), np.cumprod(alpha, axis=1)], axis=1)  # P(n >= k)
    pmf = reach[:, :K] - reach[:, 1:]
    pmf = np.concatenate([pmf, reach[:, K:]], axis=1)
    ks = np.arange(K + 1)
    mean = (pmf * (ks + 1)).sum(1)
    var = (pmf * (ks + 1) ** 2).sum(1) - mean ** 2
    z = ((res["accepted"] + 1) - mean).sum() / np.sqrt(var.sum())
    assert abs(z) < 4
    # the first emitted token follows q_0 (the paperlayer.ai summary's
    # Theorem 1): its randomised PIT F(y - 1) + U q(y) is U(0, 1)
    q0 = q[:, 0].numpy()
    y0 = res["out_tokens"][:, 0].astype(np.int64)
    qy = q0[np.arange(B), y0]
    below = np.cumsum(q0, axis=1)[np.arange(B), y0] - qy
    pit = np.clip(below + rng.random(B) * qy, 0.0, 1.0)
    assert stats.kstest(pit, "uniform").pvalue > 1e-3
    # the accept loop saw exactly these probabilities
    np.testing.assert_allclose(res["diag"][:, :, 0],
                               np.take_along_axis(q.numpy(), toks[..., None], -1)[..., 0], rtol=1e-12)
    np.testing.assert_allclose(res["diag"][:, :, 1],
                               np.take_along_axis(p.numpy(), toks[..., None], -1)[..., 0], rtol=1e-12)


def test_bonus_with_k0_is_inverse_cdf_of_target():
    rng = np.random.default_rng(31)
    B, V = 300, 50
    x = (rng.standard_normal((B, 1, V)) * 2).astype(np.float32)
    res = oracle.verify(x, np.zeros((B, 0, V), np.float32), np.zeros((B, 0), np.int32),
                        seed=8, row_offset=1000)
    q = torch.softmax(torch.from_numpy(x[:, 0].astype(np.float64)), -1).numpy()
    for b in range(B):
        u = oracle.uniform(8, 1000 + b, 0, oracle.PURPOSE_BONUS)
        c = np.cumsum(q[b])
        want = int(np.searchsorted(c, u * c[-1], side="right"))
        assert res["out_tokens"][b, 0] == want
        assert res["accepted"][b] == 0


def test_identical_models_never_reject():
    rng = np.random.default_rng(41)
    B, K, V = 2000, 5, 30
    x = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    for mode, kw in [(oracle.PLAIN, {}), (oracle.TOPK, {"default_top_k": 5}),
                     (oracle.TOPP, {"default_top_p": 0.6}), (oracle.GREEDY, {})]:
        toks = oracle.sample_rows(x[:, :K].copy(), default_mode=mode, seed=4, **kw).astype(np.int32)
        res = oracle.verify(x, x[:, :K].copy(), toks, default_mode=mode, seed=2, **kw)
        # q == p: u * p(d) < q(d) holds for every u < 1 and every d drawn from p
        assert np.all(res["accepted"] == K), mode
        assert np.all(res["diag"][..., 0] == res["diag"][..., 1])


def test_disjoint_supports_always_reject_and_resample_from_q():
    B, K, V = 500, 3, 6
    tq = np.array([0, 0, 0, -np.inf, -np.inf, -np.inf], np.float32) + np.float32(0)
    tq[:3] = [0.3, -0.2, 1.0]
    tp = np.array([-np.inf, -np.inf, -np.inf, 0.5, 0.1, -0.4], np.float32)
    target = np.broadcast_to(tq, (B, K + 1, V)).copy()
    draft = np.broadcast_to(tp, (B, K, V)).copy()
    toks = oracle.sample_rows(draft, seed=6).astype(np.int32)
    res = oracle.verify(target, draft, toks, seed=12)
    assert np.all(res["accepted"] == 0)
    q = torch.softmax(torch.from_numpy(tq.astype(np.float64)), 0).numpy()
    c = np.cumsum(q)
    for b in range(B):
        u = oracle.uniform(12, b, 0, oracle.PURPOSE_RESAMPLE)
        assert res["out_tokens"][b, 0] == int(np.searchsorted(c, u * c[-1], side="right"))


def test_greedy_reduces_to_longest_matching_prefix():
    rng = np.random.default_rng(51)
    B, K, V = 3000, 4, 12
    target = rng.integers(-3, 3, (B, K + 1, V)).astype(np.float32)  # frequent ties
    draft = rng.integers(-3, 3, (B, K, V)).astype(np.float32)
    am = np.argmax(target, -1)  # first (lowest-index) maximum
    toks = np.where(rng.random((B, K)) < 0.7, am[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    res = oracle.verify(target, draft, toks, default_mode=oracle.GREEDY, default_temperature=0.0,
                        seed=17)
    for b in range(B):
        n = 0
        while n < K and toks[b, n] == am[b, n]:
            n += 1
        assert res["accepted"][b] == n
        assert res["out_tokens"][b, n] == am[b, n]
        assert res["flags"][b] & oracle.FL_TOPP == 0


def test_ragged_rows_never_read_padding():
    rng = np.random.default_rng(61)
    B, K, V = 200, 6, 40
    target = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    draft = (target[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    kpr = rng.integers(0, K + 1, B).astype(np.int32)
    toks = oracle.sample_rows(draft, seed=3).astype(np.int32)
    ref = oracle.verify(target, draft, toks, k_per_row=kpr, seed=9)
    t2, d2 = target.copy(), draft.copy()
    for b in range(B):
        t2[b, kpr[b] + 1:] = np.nan
        d2[b, kpr[b]:] = np.nan
    got = oracle.verify(t2, d2, toks, k_per_row=kpr, seed=9)
    for k in ("accepted", "out_tokens", "row_status"):
        np.testing.assert_array_equal(got[k], ref[k])
    assert np.all(ref["accepted"] <= kpr)
    assert np.all(np.isnan(ref["diag"][np.arange(K)[None, :] >= kpr[:, None]]))


def test_error_rows():
    B, K, V = 6, 2, 8
    target = np.zeros((B, K + 1, V), np.float32)
    draft = np.zeros((B, K, V), np.float32)
    toks = np.zeros((B, K), np.int32)
    target[0, 1, 3] = np.nan          # used row: error
    toks[1, 1] = V                    # token out of range
    draft[2, 0, :] = -np.inf          # empty row
    target[3, 0, 0] = np.inf          # +inf
    temp = np.ones(B, np.float32)
    temp[4] = 0.0                     # invalid temperature
    kpr = np.full(B, K, np.int32)
    kpr[5] = 3                        # K_b > K_max
    res = oracle.verify(target, draft, toks, temperature=temp, k_per_row=kpr, seed=1)
    want = [oracle.ST_NONFINITE, oracle.ST_TOKEN, oracle.ST_EMPTY, oracle.ST_NONFINITE,
            oracle.ST_PARAM, oracle.ST_PARAM]
    for b in range(B):
        assert res["row_status"][b] & oracle.ST_ERRORS == want[b], b
        assert res["accepted"][b] == -1
        assert np.all(res["out_tokens"][b] == -1)


def test_row_offset_equals_global_row():
    rng = np.random.default_rng(71)
    B, K, V = 64, 3, 20
    target = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    draft = (target[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    toks = oracle.sample_rows(draft, seed=1).astype(np.int32)
    whole = oracle.verify(target, draft, toks, seed=4, row_offset=100)
    lo = oracle.verify(target[:20], draft[:20], toks[:20], seed=4, row_offset=100)
    hi = oracle.verify(target[20:], draft[20:], toks[20:], seed=4, row_offset=120)
    np.testing.assert_array_equal(whole["out_tokens"], np.concatenate([lo["out_tokens"], hi["out_tokens"]]))

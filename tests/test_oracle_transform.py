"""Pins of the oracle's per-row transform (CPU only).

The transform turns raw logits into the "adjusted distribution" sampled by
the step: temperature, then plain / top-k / nucleus / greedy, applied before
the rejection step (paperlayer.ai summary of arXiv 2302.01318, "Modified
Rejection Sampling"; FDE Interviews breakdown, section 01).  Each mode is
checked against something other than the oracle's own code: torch's softmax
and topk, numpy's sort / cumsum / searchsorted, closed forms and hand cases.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
WE = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
Q = np.array(WE["target_q"])
P = np.array(WE["draft_p"])


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_plain_worked_example_recovers_target():
    x = np.log(Q).astype(np.float32)
    pi, st, margin, nk = oracle.row_probs(x, oracle.PLAIN, 1.0)
    assert st == 0 and nk == 4 and margin == np.inf
    np.testing.assert_allclose(pi, Q, rtol=0, atol=2e-7)


@pytest.mark.parametrize("tau", [1.0, 0.7, 1.9])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_plain_matches_torch_softmax(tau, dtype):
    rng = np.random.default_rng(1)
    for _ in range(5):
        x32 = (rng.standard_normal(1000) * 3).astype(np.float32)
        x32[rng.integers(0, 1000, 7)] = -np.inf
        row = x32 if dtype == "f32" else bf16_bits(x32)
        vals = x32.astype(np.float64) if dtype == "f32" else bf16_values(row)
        want = torch.softmax(torch.from_numpy(vals) / np.float64(np.float32(tau)), 0).numpy()
        pi, st, _, _ = oracle.row_probs(row, oracle.PLAIN, tau)
        assert st == 0
        np.testing.assert_allclose(pi, want, rtol=1e-12, atol=1e-300)


def test_plain_shift_invariance():
    rng = np.random.default_rng(2)
    x = rng.integers(-20, 20, 300).astype(np.float32)
    a, _, _, _ = oracle.row_probs(x, oracle.PLAIN, 0.9)
    b, _, _, _ = oracle.row_probs(x + np.float32(64), oracle.PLAIN, 0.9)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=0)


@pytest.mark.parametrize("k", [1, 2, 7, 40, 999, 1000])
def test_topk_matches_torch_topk(k):
    rng = np.random.default_rng(3 + k)
    tau = 0.7
    for _ in range(4):
        x32 = (rng.standard_normal(1000) * 3).astype(np.float32)
        bits = bf16_bits(x32)  # bf16 rounding creates ties
        vals = bf16_values(bits)
        t = torch.from_numpy(vals)
        kth = torch.topk(t, k).values[-1]
        masked = torch.where(t >= kth, t / np.float64(np.float32(tau)), torch.tensor(-np.inf, dtype=torch.float64))
        want = torch.softmax(masked, 0).numpy()
        pi, st, _, nk = oracle.row_probs(bits, oracle.TOPK, tau, top_k=k)
        assert st == 0
        assert nk == int((t >= kth).sum())
        assert nk >= k
        np.testing.assert_allclose(pi, want, rtol=1e-12, atol=1e-300)


def test_topk_keeps_all_ties_at_the_boundary():
    x = np.array([3, 1, 2, 2, 2, 0], np.float32)
    pi, _, _, nk = oracle.row_probs(x, oracle.TOPK, 1.0, top_k=2)
    assert nk == 4
    assert pi[1] == 0 and pi[5] == 0
    np.testing.assert_allclose(pi[[0, 2, 3, 4]].sum(), 1.0, rtol=1e-15)
    assert pi[2] == pi[3] == pi[4]


# Hand cases on the worked example's target [0.5, 0.25, 0.15, 0.10]: the
# masses before each token (descending) are 0, 0.5, 0.75, 0.9.
@pytest.mark.parametrize("top_p,kept", [
    (0.3, [0]), (0.7, [0, 1]), (0.8, [0, 1, 2]), (0.85, [0, 1, 2]), (0.95, [0, 1, 2, 3]),
])
def test_topp_hand_cases(top_p, kept):
    x = np.log(Q).astype(np.float32)
    pi, st, margin, nk = oracle.row_probs(x, oracle.TOPP, 1.0, top_p=top_p)
    assert st == 0 and nk == len(kept)
    want = np.zeros(4)
    want[kept] = Q[kept] / Q[kept].sum()
    np.testing.assert_allclose(pi, want, atol=3e-7)
    assert margin > 1e-3


@pytest.mark.parametrize("top_p", [0.5, 0.75, 0.9])
def test_topp_boundary_is_flagged(top_p):
    # the cumulative mass lands on top_p (up to fp32 rounding of the logits)
    x = np.log(Q).astype(np.float32)
    _, _, margin, _ = oracle.row_probs(x, oracle.TOPP, 1.0, top_p=top_p)
    assert margin < 1e-6


def test_topp_matches_smallest_prefix_definition():
    # Without ties, "keep a token iff the mass before it is < top_p" is the
    # classic nucleus: the shortest descending prefix whose mass reaches top_p.
    rng = np.random.default_rng(4)
    for trial in range(60):
        V = int(rng.integers(2, 400))
        x = (rng.standard_normal(V) * rng.uniform(0.5, 4)).astype(np.float32)
        tau = float(rng.uniform(0.3, 2.0))
        top_p = float(rng.uniform(0.05, 0.99))
        s = torch.softmax(torch.from_numpy(x.astype(np.float64)) / np.float64(np.float32(tau)), 0).numpy()
        if len(np.unique(x)) != V:
            continue
        order = np.argsort(-x, kind="stable")
        cum = np.cumsum(s[order])
        n_keep = min(V, 1 + int(np.searchsorted(cum, np.float32(top_p), side="left")))
        pi, st, margin, nk = oracle.row_probs(x, oracle.TOPP, tau, top_p=top_p)
        if margin < 1e-9:
            continue
        assert nk == n_keep, trial
        kept = order[:n_keep]
        want = np.zeros(V)
        want[kept] = s[kept] / s[kept].sum()
        np.testing.assert_allclose(pi, want, rtol=1e-10, atol=1e-300)


def test_topp_groups_ties():
    # target 0.4 / 0.2 / 0.2 / 0.2: the three tied tokens form one group
    x = np.log(np.array([0.4, 0.2, 0.2, 0.2])).astype(np.float32)
    pi, _, _, nk = oracle.row_probs(x, oracle.TOPP, 1.0, top_p=0.5)
    assert nk == 4  # mass before the tied group is 0.4 < 0.5: all three kept
    pi, _, _, nk = oracle.row_probs(x, oracle.TOPP, 1.0, top_p=0.3)
    assert nk == 1 and pi[0] == 1.0


def test_topp_one_is_plain():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(500) * 3).astype(np.float32)
    a, _, ma, _ = oracle.row_probs(x, oracle.TOPP, 0.8, top_p=1.0)
    b, _, _, _ = oracle.row_probs(x, oracle.PLAIN, 0.8)
    np.testing.assert_array_equal(a, b)
    assert ma == np.inf


def test_greedy_is_lowest_index_argmax():
    rng = np.random.default_rng(9)
    for _ in range(50):
        x = rng.integers(-3, 4, 40).astype(np.float32)  # many ties
        pi, st, _, nk = oracle.row_probs(x, oracle.GREEDY, 0.0)
        assert st == 0 and nk == 1
        assert pi[int(np.argmax(x))] == 1.0 and pi.sum() == 1.0


def test_row_errors():
    x = np.zeros(8, np.float32)
    x[3] = np.nan
    assert oracle.row_probs(x, oracle.PLAIN, 1.0)[1] == oracle.ST_NONFINITE
    x[3] = np.inf
    assert oracle.row_probs(x, oracle.TOPK, 1.0, top_k=2)[1] == oracle.ST_NONFINITE
    y = np.full(8, -np.inf, np.float32)
    assert oracle.row_probs(y, oracle.GREEDY, 1.0)[1] == oracle.ST_EMPTY
    y[5] = -1e30
    pi, st, _, _ = oracle.row_probs(y, oracle.PLAIN, 1.0)
    assert st == 0 and pi[5] == 1.0

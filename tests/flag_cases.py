"""Inputs that put one floating-point decision of the step at a chosen
distance from its boundary, for pinning the oracle's boundary flags.

The parity rule excuses a row from exact comparison only when one of its
decisions lies within 1e-6 of the value it is compared with: an accept test
|u - q/p| < 1e-6 (FDE Interviews breakdown, section 01: keep d with
probability min(1, q/p)), an inverse-CDF draw whose uniform is within 1e-6
of a step of the cumulative distribution (paperlayer.ai summary,
"Modified Rejection Sampling": resample from normalize((q - p)+)), or a
nucleus cut whose preceding mass is within 1e-6 of top_p.  Each case below
sets that distance deliberately, to 4e-7 (inside the window) or 2.5e-6
(outside), on either side of the boundary.  The distance the inputs really
give is recomputed from the fp32 logits with torch.softmax in float64 (a
library routine, not the oracle), and every case asserts that it landed
where it was aimed: inside means |d| < 8e-7, outside |d| > 1.5e-6.

The uniforms come from the library of the oracle under test (its Philox is
pinned separately to the published known-answer vectors); rows are matched
to them by their global row id g.
"""
import numpy as np
import torch

import oracle

SEED = 20240
INSIDE, OUTSIDE = 4e-7, 2.5e-6
DELTAS = (INSIDE, -INSIDE, OUTSIDE, -OUTSIDE)


def softmax64(x32):
    """Probabilities of fp32 logits, in float64 (torch)."""
    return torch.softmax(torch.from_numpy(np.asarray(x32, np.float32).astype(np.float64)), -1).numpy()


def check_aim(dist, delta):
    if abs(delta) == INSIDE:
        assert abs(dist) < 8e-7, dist
    else:
        assert abs(dist) > 1.5e-6, dist
    assert np.sign(dist) == np.sign(delta), (dist, delta)


def uniforms(purpose, n, t=0, lib=None):
    """The 24-bit integers k (u = k 2^-24) of rows g = 0..n-1."""
    g = np.arange(n, dtype=np.uint64)
    return oracle.philox_words(SEED, g, t, purpose, lib=lib) >> 8


def find_rows(purpose, pred, n=1 << 23, t=0, lib=None, count=1):
    k = uniforms(purpose, n, t, lib)
    hits = np.nonzero(pred(k))[0][:count]
    assert hits.size == count, "no row id with such a uniform"
    return [int(h) for h in hits]


def _logit2(a):
    """fp32 logits of a two-token row with probabilities (a, 1 - a)."""
    return np.array([np.log(a), np.log1p(-a)], np.float32)


def accept_rows(lib=None):
    """K = 1, V = 2, fp32, plain at tau = 1.  Draft logits [0, 0] (p = 1/2,
    1/2), draft token 0, target q(0) = (u + delta) / 2, so q/p - u = delta.
    Returns (target, draft, tokens, expected flag, expected accept, dist)."""
    B = len(DELTAS)
    u = np.array([oracle.uniform(SEED, b, 0, oracle.PURPOSE_ACCEPT, lib=lib) for b in range(B)])
    target = np.zeros((B, 2, 2), np.float32)
    draft = np.zeros((B, 1, 2), np.float32)
    tokens = np.zeros((B, 1), np.int32)
    dist = np.zeros(B)
    for b, d in enumerate(DELTAS):
        assert 0.01 < u[b] < 0.99
        target[b, 0] = _logit2((u[b] + d) / 2.0)
        target[b, 1] = [0.0, 0.0]
        ratio = softmax64(target[b, 0])[0] / softmax64(draft[b, 0])[0]
        dist[b] = ratio - u[b]
        check_aim(dist[b], d)
    flag = np.abs(dist) < 1e-6
    accept = dist > 0          # u p < q  <=>  u < q / p
    return target, draft, tokens, flag, accept, dist


def accept_at_one(lib=None):
    """q = p (identical logits): the ratio is exactly 1, and a uniform within
    1e-6 below it is a decision at its boundary.  Returns (row id, target,
    draft, tokens)."""
    (g,) = find_rows(oracle.PURPOSE_ACCEPT, lambda k: k >= (1 << 24) - 12, lib=lib)
    x = np.array([0.3, -0.2, 1.1], np.float32)
    target = np.stack([x, x])[None]
    draft = x[None, None].copy()
    tokens = np.array([[2]], np.int32)
    return g, target, draft, tokens


def bonus_rows(lib=None):
    """K = 0, V = 2, fp32, plain: the bonus draw from q = (a, 1 - a) with
    a = u + delta, so the CDF step a lies delta above the target u.  Returns
    (target, expected y, expected flag, dist)."""
    B = len(DELTAS)
    u = np.array([oracle.uniform(SEED, b, 0, oracle.PURPOSE_BONUS, lib=lib) for b in range(B)])
    target = np.zeros((B, 1, 2), np.float32)
    dist = np.zeros(B)
    for b, d in enumerate(DELTAS):
        assert 0.01 < u[b] < 0.99
        target[b, 0] = _logit2(u[b] + d)
        dist[b] = softmax64(target[b, 0])[0] - u[b]
        check_aim(dist[b], d)
    y = np.where(dist > 0, 0, 1)
    flag = np.abs(dist) < 1e-6
    return target, y, flag, dist


def bonus_at_ends(lib=None):
    """Uniforms within 1e-6 of 0 and of 1 under q = (1/2, 1/2): the draw then
    sits next to the CDF's ends, which are not boundaries between tokens of
    non-zero weight, so no flag.  Returns [(row id, expected y)]."""
    (g0,) = find_rows(oracle.PURPOSE_BONUS, lambda k: k < 12, lib=lib)
    (g1,) = find_rows(oracle.PURPOSE_BONUS, lambda k: k >= (1 << 24) - 12, lib=lib)
    return [(g0, 0), (g1, 1)]


def resample_rows(lib=None):
    """K = 1, V = 3, fp32, plain: draft p ~ (1/2, 1/4, 1/4), draft token 0,
    target q(0) = 1/5, so the test u p(0) < q(0) rejects whenever the accept
    uniform is above 2/5 (rows are picked so).  The residual (q - p)+ is
    (0, q1 - p1, q2 - p2); q1 is set so that its CDF step lies delta above
    the resample uniform.  Returns (row ids, target, draft, tokens, expected
    y, expected flag, dist)."""
    ka = uniforms(oracle.PURPOSE_ACCEPT, 4096, lib=lib)
    kr = uniforms(oracle.PURPOSE_RESAMPLE, 4096, lib=lib)
    ok = (ka > int(0.45 * 2 ** 24)) & (kr > int(0.05 * 2 ** 24)) & (kr < int(0.95 * 2 ** 24))
    rows = [int(g) for g in np.nonzero(ok)[0][:len(DELTAS)]]
    B = len(rows)
    draft = np.tile(np.log(np.array([0.5, 0.25, 0.25])).astype(np.float32), (B, 1, 1))
    p = softmax64(draft[0, 0])
    target = np.zeros((B, 2, 3), np.float32)
    dist = np.zeros(B)
    for i, (g, d) in enumerate(zip(rows, DELTAS)):
        u = kr[g] / 2.0 ** 24
        # residual masses r1 = q1 - p1, r2 = q2 - p2 with q0 = 1/5: the step
        # r1 / (r1 + r2) placed at u + d
        free = 0.8 - p[1] - p[2]
        q1 = p[1] + free * (u + d)
        target[i, 0] = np.log(np.array([0.2, q1, 0.8 - q1])).astype(np.float32)
        target[i, 1] = [0.0, 0.0, 0.0]
        q = softmax64(target[i, 0])
        assert q[0] / p[0] < 0.44          # rejected: u_accept > 0.45
        r = np.maximum(q - p, 0.0)
        dist[i] = r[1] / r.sum() - u
        check_aim(dist[i], d)
    y = np.where(dist > 0, 1, 2)
    flag = np.abs(dist) < 1e-6
    tokens = np.zeros((B, 1), np.int32)
    return rows, target, draft, tokens, y, flag, dist


def topp_rows(lib=None):
    """K = 1, V = 4, fp32, nucleus at tau = 1.  The draft row is the worked
    example's target (0.5, 0.25, 0.15, 0.10) (roadtointelligence.com
    "Speculative Decoding", "Why the output doesn't change"), whose mass
    before its third token is 0.75; top_p = 0.75 + delta puts the draft's cut
    delta from top_p.  The target rows keep every cut far from top_p, so a
    flag can only come from the draft row.  Returns (target, draft, tokens,
    top_p per row, expected flag, dist)."""
    B = len(DELTAS)
    wx = np.log(np.array([0.5, 0.25, 0.15, 0.10])).astype(np.float32)
    s = softmax64(wx)
    c = s[0] + s[1]
    draft = np.tile(wx, (B, 1, 1))
    tx = np.log(np.array([0.6, 0.3, 0.06, 0.04])).astype(np.float32)  # masses before: 0, .6, .9, .96
    target = np.tile(tx, (B, 2, 1))
    st = np.cumsum(softmax64(tx))
    top_p = np.zeros(B, np.float32)
    dist = np.zeros(B)
    for b, d in enumerate(DELTAS):
        top_p[b] = np.float32(c + d)
        dist[b] = float(top_p[b]) - c
        check_aim(dist[b], d)
        assert np.min(np.abs(np.concatenate([[0.0], st[:-1]]) - float(top_p[b]))) > 1e-3
    tokens = np.zeros((B, 1), np.int32)
    flag = np.abs(dist) < 1e-6
    return target, draft, tokens, top_p, flag, dist

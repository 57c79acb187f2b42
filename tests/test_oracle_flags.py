"""Pins of the oracle's boundary flags (CPU only).

A row is excused from exact GPU-vs-oracle comparison only when the oracle
flags it: a decision it used lies within 1e-6 of its boundary.  These tests
put each kind of decision 4e-7 and 2.5e-6 from its boundary, on both sides,
and check that the flag is set exactly in the first case, and that the
decision itself (accept, token) is the one the definition gives.  The
distances are computed with torch.softmax in float64 from the same fp32
logits (tests/flag_cases.py), not by the oracle.

Decisions and their boundaries:
  * accept test u p < q (FDE Interviews breakdown, section 01): |u - q/p|;
  * inverse-CDF draw of the bonus token and of the resample from
    normalize((q - p)+) (paperlayer.ai summary, "Modified Rejection
    Sampling"): the distance from u to the nearest step of the cumulative
    weight between tokens of non-zero weight;
  * nucleus cut: the distance from top_p to the mass before a group, on the
    target and on the draft rows.
"""
import numpy as np

import flag_cases as fc
import oracle


def _verify(target, draft, tokens, **kw):
    return oracle.verify(target, draft, tokens, seed=fc.SEED, **kw)


def test_accept_flag_set_inside_and_clear_outside_the_window():
    target, draft, tokens, flag, accept, dist = fc.accept_rows()
    res = _verify(target, draft, tokens)
    got = (res["flags"] & oracle.FL_ACCEPT) != 0
    assert list(got) == list(flag), (dist, res["flags"])
    assert list(res["accepted"] == 1) == list(accept)
    # the CDF flag is about the draw, not the accept test
    assert np.all((res["flags"] & oracle.FL_TOPP) == 0)


def test_accept_flag_at_ratio_one():
    g, target, draft, tokens = fc.accept_at_one()
    res = _verify(target, draft, tokens, row_offset=g)
    assert res["accepted"][0] == 1                    # u < 1 = q/p
    assert res["flags"][0] & oracle.FL_ACCEPT


def test_accept_flag_needs_the_test_to_be_reached():
    # K = 2: position 1's accept test sits 4e-7 from its boundary (its own
    # uniform, t = 1).  Behind a position that always accepts (q = p) the
    # walk reaches it and the row is flagged; behind one that always rejects
    # (q(d) ~ 1e-30, p(d) = 1/2) the walk stops first and the test is unused.
    rows = []
    for g in range(64):
        u1 = oracle.uniform(fc.SEED, g, 1, oracle.PURPOSE_ACCEPT)
        u0 = oracle.uniform(fc.SEED, g, 0, oracle.PURPOSE_ACCEPT)
        if 0.01 < u1 < 0.99 and 1e-3 < u0 < 0.99:
            rows.append((g, u1))
        if len(rows) == 2:
            break
    out = {}
    for (g, u1), first in zip(rows, ("accept", "reject")):
        near = np.array([np.log((u1 + fc.INSIDE) / 2.0), np.log1p(-(u1 + fc.INSIDE) / 2.0)], np.float32)
        ratio = fc.softmax64(near)[0] / 0.5
        assert 0 < ratio - u1 < 8e-7
        t0 = np.zeros(2, np.float32) if first == "accept" else np.log(np.array([1e-30, 1.0])).astype(np.float32)
        target = np.stack([t0, near, np.zeros(2, np.float32)])[None]
        draft = np.zeros((1, 2, 2), np.float32)
        tokens = np.zeros((1, 2), np.int32)
        out[first] = _verify(target, draft, tokens, row_offset=g)
    assert out["accept"]["accepted"][0] == 2
    assert out["accept"]["flags"][0] & oracle.FL_ACCEPT
    assert out["reject"]["accepted"][0] == 0
    assert out["reject"]["flags"][0] & oracle.FL_ACCEPT == 0


def test_bonus_cdf_flag():
    target, y, flag, dist = fc.bonus_rows()
    res = _verify(target, np.zeros((len(y), 0, 2), np.float32), np.zeros((len(y), 0), np.int32))
    assert list(res["out_tokens"][:, 0]) == list(y), dist
    assert list((res["flags"] & oracle.FL_CDF) != 0) == list(flag), (dist, res["flags"])


def test_cdf_ends_are_not_boundaries():
    for g, y in fc.bonus_at_ends():
        res = _verify(np.zeros((1, 1, 2), np.float32), np.zeros((1, 0, 2), np.float32),
                      np.zeros((1, 0), np.int32), row_offset=g)
        assert res["out_tokens"][0, 0] == y
        assert res["flags"][0] == 0, g


def test_resample_cdf_flag():
    rows, target, draft, tokens, y, flag, dist = fc.resample_rows()
    for i, g in enumerate(rows):
        res = _verify(target[i:i + 1], draft[i:i + 1], tokens[i:i + 1], row_offset=g)
        assert res["accepted"][0] == 0, g
        assert res["out_tokens"][0, 0] == y[i], (g, dist[i])
        assert bool(res["flags"][0] & oracle.FL_CDF) == bool(flag[i]), (g, dist[i])
        assert res["flags"][0] & oracle.FL_ACCEPT == 0


def test_nucleus_flag_comes_from_the_draft_row_too():
    target, draft, tokens, top_p, flag, dist = fc.topp_rows()
    res = _verify(target, draft, tokens, default_mode=oracle.TOPP, top_p=top_p)
    assert list((res["flags"] & oracle.FL_TOPP) != 0) == list(flag), (dist, res["flags"])
    # and the same cut on the row alone
    for b in range(len(flag)):
        _, _, margin, _ = oracle.row_probs(draft[b, 0], oracle.TOPP, 1.0, top_p=float(top_p[b]))
        assert (margin < 1e-6) == flag[b]
        np.testing.assert_allclose(margin, abs(dist[b]), rtol=1e-6)

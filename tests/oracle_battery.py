"""A fast battery of the oracle's pins, runnable against any build of it.

Used by the planted-mistake test: each mutant of the oracle is compiled into
its own library and this battery runs in a subprocess against it; a mutant
is caught when any check fails, raises or the process dies.  The checks are
condensed forms of the pins in test_oracle_*.py (same external references:
published Philox vectors, torch's softmax / topk, numpy searchsorted, exact
enumeration of the output law, the worked example).

Usage: python oracle_battery.py /path/to/liboracle.so   (exit 0 = all pass)
"""
import itertools
import os
import sys
from fractions import Fraction

import numpy as np
import torch
from scipy import stats

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)
import oracle  # noqa: E402

Q = np.array([0.5, 0.25, 0.15, 0.10])
P = np.array([0.3, 0.4, 0.2, 0.1])


def check_kat(lib):
    got = oracle.philox([0, 0, 0, 0], [0, 0], lib=lib)
    want = [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]
    assert [int(x) for x in got] == want
    got = oracle.philox([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344],
                        [0xa4093822, 0x299f31d0], lib=lib)
    assert [int(x) for x in got] == [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]


def check_counter_layout(lib):
    for seed, g, t, p in [(5, 7, 3, 1), (2**40 + 3, 2**33 + 9, 17, 2)]:
        w = oracle.philox([g & 0xFFFFFFFF, t, p, g >> 32], [seed & 0xFFFFFFFF, seed >> 32], lib=lib)
        assert oracle.uniform(seed, g, t, p, lib=lib) == (int(w[0]) >> 8) / 2.0**24


def check_plain(lib):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(500) * 3).astype(np.float32)
    want = torch.softmax(torch.from_numpy(x.astype(np.float64)) / np.float64(np.float32(0.7)), 0).numpy()
    pi, st, _, _ = oracle.row_probs(x, oracle.PLAIN, 0.7, lib=lib)
    assert st == 0
    np.testing.assert_allclose(pi, want, rtol=1e-10)


def check_topk(lib):
    rng = np.random.default_rng(2)
    xs = [(rng.standard_normal(300) * 4).astype(np.float32),            # distinct values
          np.round(rng.standard_normal(300) * 4).astype(np.float32)]  # many ties
    for x, k in itertools.product(xs, (1, 5, 37)):
        t = torch.from_numpy(x.astype(np.float64))
        kth = torch.topk(t, k).values[-1]
        m = torch.where(t >= kth, t / np.float64(np.float32(0.8)), torch.tensor(-np.inf, dtype=torch.float64))
        want = torch.softmax(m, 0).numpy()
        pi, _, _, _ = oracle.row_probs(x, oracle.TOPK, 0.8, top_k=k, lib=lib)
        np.testing.assert_allclose(pi, want, rtol=1e-10, atol=1e-300)


def check_topp(lib):
    x = np.log(Q).astype(np.float32)
    for top_p, kept in [(0.3, [0]), (0.7, [0, 1]), (0.8, [0, 1, 2]), (0.95, [0, 1, 2, 3])]:
        pi, _, _, _ = oracle.row_probs(x, oracle.TOPP, 1.0, top_p=top_p, lib=lib)
        want = np.zeros(4)
        want[kept] = Q[kept] / Q[kept].sum()
        np.testing.assert_allclose(pi, want, atol=3e-7)
    rng = np.random.default_rng(3)
    for _ in range(20):
        V = 200
        x = (rng.standard_normal(V) * 2).astype(np.float32)
        top_p = float(rng.uniform(0.1, 0.95))
        s = torch.softmax(torch.from_numpy(x.astype(np.float64)) / np.float64(np.float32(0.9)), 0).numpy()
        order = np.argsort(-x, kind="stable")
        n_keep = min(V, 1 + int(np.searchsorted(np.cumsum(s[order]), np.float32(top_p), side="left")))
        _, _, margin, nk = oracle.row_probs(x, oracle.TOPP, 0.9, top_p=top_p, lib=lib)
        if margin > 1e-9:
            assert nk == n_keep


def check_greedy(lib):
    rng = np.random.default_rng(4)
    B, K, V = 400, 3, 9
    target = rng.integers(-2, 2, (B, K + 1, V)).astype(np.float32)
    draft = rng.integers(-2, 2, (B, K, V)).astype(np.float32)
    am = np.argmax(target, -1)
    toks = np.where(rng.random((B, K)) < 0.7, am[:, :K], rng.integers(0, V, (B, K))).astype(np.int32)
    res = oracle.verify(target, draft, toks, default_mode=oracle.GREEDY, seed=3, lib=lib)
    for b in range(B):
        n = 0
        while n < K and toks[b, n] == am[b, n]:
            n += 1
        assert res["accepted"][b] == n and res["out_tokens"][b, n] == am[b, n]


def _worked(lib, B=200_000):
    tq = np.log(Q).astype(np.float32)
    tp = np.log(P).astype(np.float32)
    target = np.broadcast_to(tq, (B, 5, 4)).copy()
    draft = np.broadcast_to(tp, (B, 4, 4)).copy()
    toks = oracle.sample_rows(draft, seed=1001, lib=lib).astype(np.int32)
    return toks, oracle.verify(target, draft, toks, seed=1, lib=lib)


def check_worked_example(lib):
    toks, res = _worked(lib)
    n = res["accepted"]
    assert stats.chisquare(np.bincount(toks.ravel(), minlength=4), P * toks.size)[1] > 1e-4
    law = np.array([0.2, 0.16, 0.128, 0.1024, 0.4096])
    assert stats.chisquare(np.bincount(n, minlength=5), law * n.size)[1] > 1e-4
    out = res["out_tokens"]
    assert stats.chisquare(np.bincount(out[:, 0], minlength=4), Q * n.size)[1] > 1e-4
    assert np.all(out[np.arange(n.size), n][n < 4] == 0)
    idx = np.arange(4)[None, :]
    prefix = idx < n[:, None]
    assert np.all(out[:, :4][prefix] == toks[prefix])
    np.testing.assert_allclose(res["diag"][0, 0], [Q[toks[0, 0]], P[toks[0, 0]]], atol=1e-6)


def check_enumeration(lib):
    qs = [[Fraction(1, 2), Fraction(1, 4), Fraction(1, 8), Fraction(1, 8)],
          [Fraction(1, 10), Fraction(2, 10), Fraction(3, 10), Fraction(4, 10)],
          [Fraction(1, 4)] * 4]
    ps = [[Fraction(1, 8), Fraction(1, 8), Fraction(1, 4), Fraction(1, 2)],
          [Fraction(3, 10), Fraction(3, 10), Fraction(2, 10), Fraction(2, 10)]]
    K, V = 2, 4
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
    B = 150_000
    tl = np.log(np.array([[float(x) for x in r] for r in qs])).astype(np.float32)
    dl = np.log(np.array([[float(x) for x in r] for r in ps])).astype(np.float32)
    target = np.broadcast_to(tl, (B, K + 1, V)).copy()
    draft = np.broadcast_to(dl, (B, K, V)).copy()
    toks = oracle.sample_rows(draft, seed=77, lib=lib).astype(np.int32)
    res = oracle.verify(target, draft, toks, seed=5, lib=lib)
    keys = list(law)
    index = {k: i for i, k in enumerate(keys)}
    counts = np.zeros(len(keys))
    for b in range(B):
        n = int(res["accepted"][b])
        counts[index[(n,) + tuple(int(x) for x in res["out_tokens"][b, :n + 1])]] += 1
    assert stats.chisquare(counts, np.array([float(law[k]) for k in keys]) * B)[1] > 1e-4


def check_bonus(lib):
    rng = np.random.default_rng(5)
    B, V = 100, 30
    x = (rng.standard_normal((B, 1, V)) * 2).astype(np.float32)
    res = oracle.verify(x, np.zeros((B, 0, V), np.float32), np.zeros((B, 0), np.int32),
                        seed=8, row_offset=50, lib=lib)
    q = torch.softmax(torch.from_numpy(x[:, 0].astype(np.float64)), -1).numpy()
    for b in range(B):
        u = oracle.uniform(8, 50 + b, 0, oracle.PURPOSE_BONUS, lib=lib)
        c = np.cumsum(q[b])
        assert res["out_tokens"][b, 0] == int(np.searchsorted(c, u * c[-1], side="right"))


def check_errors_and_ragged(lib):
    B, K, V = 4, 2, 8
    target = np.zeros((B, K + 1, V), np.float32)
    draft = np.zeros((B, K, V), np.float32)
    toks = np.zeros((B, K), np.int32)
    target[0, 1, 3] = np.nan
    toks[1, 1] = V
    draft[2, 0, :] = -np.inf
    kpr = np.array([2, 2, 2, 1], np.int32)
    draft[3, 1, :] = np.nan     # padding of a ragged row
    target[3, 2, :] = np.nan
    res = oracle.verify(target, draft, toks, k_per_row=kpr, seed=1, lib=lib)
    assert [int(x) for x in res["row_status"][:3] & oracle.ST_ERRORS] == \
        [oracle.ST_NONFINITE, oracle.ST_TOKEN, oracle.ST_EMPTY]
    assert list(res["accepted"][:3]) == [-1, -1, -1]
    assert res["accepted"][3] in (0, 1) and res["row_status"][3] == 0


def check_nonuniform_positions(lib):
    rng = np.random.default_rng(6)
    B, K, V = 4000, 3, 16
    t32 = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    d32 = (t32[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    toks = oracle.sample_rows(d32, seed=9, lib=lib).astype(np.int32)
    res = oracle.verify(t32, d32, toks, seed=3, lib=lib)
    q = torch.softmax(torch.from_numpy(t32[:, :K].astype(np.float64)), -1).numpy()
    p = torch.softmax(torch.from_numpy(d32.astype(np.float64)), -1).numpy()
    np.testing.assert_allclose(res["diag"][..., 0], np.take_along_axis(q, toks[..., None], -1)[..., 0],
                               rtol=1e-10)
    np.testing.assert_allclose(res["diag"][..., 1], np.take_along_axis(p, toks[..., None], -1)[..., 0],
                               rtol=1e-10)
    alpha = np.minimum(p, q).sum(-1)
    reach = np.concatenate([np.ones((B, 1)), np.cumprod(alpha, 1)], 1)
    pmf = np.concatenate([reach[:, :K] - reach[:, 1:], reach[:, K:]], 1)
    ks = np.arange(K + 1) + 1
    mean = (pmf * ks).sum(1)
    var = (pmf * ks ** 2).sum(1) - mean ** 2
    z = ((res["accepted"] + 1) - mean).sum() / np.sqrt(var.sum())
    assert abs(z) < 5


def check_flags(lib):
    """Boundary flags at 4e-7 (set) and 2.5e-6 (clear) from each kind of
    boundary (tests/flag_cases.py)."""
    import flag_cases as fc

    def ver(t, d, k, **kw):
        return oracle.verify(t, d, k, seed=fc.SEED, lib=lib, **kw)

    t, d, k, flag, accept, _ = fc.accept_rows(lib)
    r = ver(t, d, k)
    assert list((r["flags"] & oracle.FL_ACCEPT) != 0) == list(flag)
    assert list(r["accepted"] == 1) == list(accept)
    g, t, d, k = fc.accept_at_one(lib)
    assert ver(t, d, k, row_offset=g)["flags"][0] & oracle.FL_ACCEPT
    t, y, flag, _ = fc.bonus_rows(lib)
    r = ver(t, np.zeros((len(y), 0, 2), np.float32), np.zeros((len(y), 0), np.int32))
    assert list(r["out_tokens"][:, 0]) == list(y)
    assert list((r["flags"] & oracle.FL_CDF) != 0) == list(flag)
    for g, y0 in fc.bonus_at_ends(lib):
        r = ver(np.zeros((1, 1, 2), np.float32), np.zeros((1, 0, 2), np.float32), np.zeros((1, 0), np.int32),
                row_offset=g)
        assert r["out_tokens"][0, 0] == y0 and r["flags"][0] == 0
    rows, t, d, k, y, flag, _ = fc.resample_rows(lib)
    for i, g in enumerate(rows):
        r = ver(t[i:i + 1], d[i:i + 1], k[i:i + 1], row_offset=g)
        assert r["out_tokens"][0, 0] == y[i] and bool(r["flags"][0] & oracle.FL_CDF) == bool(flag[i])
    t, d, k, top_p, flag, _ = fc.topp_rows(lib)
    r = ver(t, d, k, default_mode=oracle.TOPP, top_p=top_p)
    assert list((r["flags"] & oracle.FL_TOPP) != 0) == list(flag)


CHECKS = [check_kat, check_counter_layout, check_plain, check_topk, check_topp, check_greedy,
          check_bonus, check_errors_and_ragged, check_nonuniform_positions,
          check_flags, check_worked_example, check_enumeration]


def run(path):
    lib = oracle.load(path)
    failed = []
    for chk in CHECKS:
        try:
            chk(lib)
        except Exception as e:  # noqa: BLE001 - any failure counts
            failed.append(f"{chk.__name__}: {type(e).__name__}")
    return failed


if __name__ == "__main__":
    failed = run(sys.argv[1])
    print("FAILED " + "; ".join(failed) if failed else "ALL PASSED")
    sys.exit(1 if failed else 0)

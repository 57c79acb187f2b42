"""Loop-level model of speculative sampling, and acceptance monitoring.

Host-only arithmetic around the verify step (no GPU, no oracle):

* The law of the number of tokens one round emits, its mean and the
  speed-up over plain decoding under i.i.d. acceptance (roadtointelligence.com
  "Speculative Decoding", section "How much faster": tokens per target pass
  (1 - a^(K+1)) / (1 - a) and speed-up (1 - a^(K+1)) / ((1 - a)(K c + 1)),
  with c the cost of a draft step relative to a target step).
* The same with a separate acceptance rate per draft position
  (E[tokens] = 1 + sum_k prod_{t<k} a_t), for drafts whose acceptance is
  not identically distributed.
* Milliseconds per token and the spread of a whole response's time from the
  model-call times plus the measured verify time (fdeinterviews.com,
  "Accelerating Large Language Model Decoding with Speculative Sampling",
  figure "The idea, visually": latency against K at acceptance 0.75, flat
  from K = 3 to 5, response-time spread rising with K).  The spread is exact:
  the number of rounds a response of N tokens needs is computed from the
  per-round law by dynamic programming over the tokens still to emit.
* AcceptanceMonitor: per-position acceptance rates estimated from the
  accepted counts the verify step returns (ai-trend.me "Speculative
  decoding", "Limitations and open issues": acceptance is worth monitoring,
  since crafted inputs can lower it and slow decoding below plain sampling).

A round: the draft proposes K tokens (K draft calls), the target scores the
K + 1 positions in one call, the verify step accepts n of the drafts and
emits n + 1 tokens (fdeinterviews.com, section 01 and the figure "The idea,
visually"; paperlayer.ai, "Speculative Sampling").
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "tokens_law", "expected_tokens", "tokens_variance", "speedup", "round_ms", "ms_per_token",
    "best_k", "rounds_moments", "response_time", "AcceptanceMonitor",
]


def _alphas(alpha, K: Optional[int]) -> np.ndarray:
    """Per-position acceptance rates: a scalar repeated K times, or a sequence."""
    if np.ndim(alpha) == 0:
        if K is None or K < 0:
            raise ValueError("a scalar acceptance rate needs K >= 0")
        a = np.full(int(K), float(alpha))
    else:
        a = np.asarray(alpha, dtype=np.float64).ravel()
        if K is not None and len(a) != K:
            raise ValueError(f"{len(a)} acceptance rates for K = {K}")
    if np.any(a < 0.0) or np.any(a > 1.0) or np.any(~np.isfinite(a)):
        raise ValueError("acceptance rates must lie in [0, 1]")
    return a


def tokens_law(alpha, K: Optional[int] = None) -> np.ndarray:
    """P(a round emits j tokens) for j = 1 .. K + 1.

    The round stops at the first rejected draft position n (then n accepted
    drafts plus one resampled token: n + 1 tokens) or after all K drafts are
    accepted (K drafts plus the bonus token: K + 1).  Position t is accepted
    with probability alpha[t], independently given the logits.
    """
    a = _alphas(alpha, K)
    reach = np.concatenate([[1.0], np.cumprod(a)])  # P(first t drafts all accepted), t = 0..K
    law = np.empty(len(a) + 1)
    law[:-1] = reach[:-1] * (1.0 - a)
    law[-1] = reach[-1]
    return law


def expected_tokens(alpha, K: Optional[int] = None) -> float:
    """Mean tokens per round: 1 + sum_{k=1..K} prod_{t<k} alpha_t; with one
    rate a this is (1 - a^(K+1)) / (1 - a) (K + 1 when a = 1)."""
    a = _alphas(alpha, K)
    return float(1.0 + np.sum(np.cumprod(a)))


def tokens_variance(alpha, K: Optional[int] = None) -> float:
    law = tokens_law(alpha, K)
    j = np.arange(1, len(law) + 1, dtype=np.float64)
    m = float(np.dot(law, j))
    return float(np.dot(law, j * j) - m * m)


def speedup(alpha, K: int, c: float) -> float:
    """Speed-up over plain decoding when a draft step costs c target steps
    and verification is free: E[tokens] / (K c + 1)."""
    if c < 0:
        raise ValueError("c must be >= 0")
    return expected_tokens(alpha, K) / (K * c + 1.0)


def round_ms(K: int, t_target_ms: float, t_draft_ms: float, t_verify_ms: float = 0.0) -> float:
    """Wall time of one round: K draft calls, one target call over K + 1
    positions (taken to cost one target step), one verify step."""
    return K * t_draft_ms + t_target_ms + t_verify_ms


def ms_per_token(alpha, K: int, t_target_ms: float, t_draft_ms: float, t_verify_ms: float = 0.0) -> float:
    return round_ms(K, t_target_ms, t_draft_ms, t_verify_ms) / expected_tokens(alpha, K)


def best_k(alpha: float, t_target_ms: float, t_draft_ms: float, t_verify_ms: float = 0.0,
           k_max: int = 8) -> int:
    """The K in 1..k_max with the lowest ms per token (ties: the smaller K)."""
    costs = [ms_per_token(alpha, k, t_target_ms, t_draft_ms, t_verify_ms) for k in range(1, k_max + 1)]
    return 1 + int(np.argmin(costs))


def rounds_moments(alpha, K: Optional[int], n_tokens: int) -> tuple:
    """Mean and standard deviation of the number of rounds until a response
    has at least n_tokens tokens.  R(m), the rounds needed with m tokens
    still to emit, satisfies R(m) = 1 + R(max(m - J, 0)) with J drawn from
    the per-round law and R(0) = 0; its first two moments follow exactly."""
    if n_tokens < 0:
        raise ValueError("n_tokens must be >= 0")
    law = tokens_law(alpha, K)
    er = np.zeros(n_tokens + 1)
    er2 = np.zeros(n_tokens + 1)
    for m in range(1, n_tokens + 1):
        e1 = 0.0
        e2 = 0.0
        for j, pj in enumerate(law, start=1):
            r = m - j if m > j else 0
            e1 += pj * er[r]
            e2 += pj * (er2[r] + 2.0 * er[r])
        er[m] = 1.0 + e1
        er2[m] = 1.0 + e2
    mean = float(er[n_tokens])
    return mean, math.sqrt(max(float(er2[n_tokens]) - mean * mean, 0.0))


def response_time(alpha, K: int, n_tokens: int, t_target_ms: float, t_draft_ms: float,
                  t_verify_ms: float = 0.0) -> tuple:
    """Mean and standard deviation (ms) of the time to emit n_tokens."""
    mean_r, sd_r = rounds_moments(alpha, K, n_tokens)
    t = round_ms(K, t_target_ms, t_draft_ms, t_verify_ms)
    return mean_r * t, sd_r * t


@dataclass
class _Window:
    reached: np.ndarray
    accepted: np.ndarray
    rounds: int = 0
    tokens: int = 0
    errors: int = 0


class AcceptanceMonitor:
    """Running per-position acceptance rates from the verify step's outputs.

    update() takes one call's accepted counts n_b (-1 marks an error row,
    which is skipped) and the per-row draft lengths K_b.  Position t of row
    b was reached when t < K_b and n_b >= t; it was accepted when n_b > t.
    The estimate of alpha_t is accepted / reached, pooled over every call
    seen (all-time) and, separately, with exponential forgetting of past
    calls (decay per call), which is what alarm() compares to its floor.
    """

    def __init__(self, k_max: int, decay: float = 0.99):
        if k_max < 0:
            raise ValueError("k_max must be >= 0")
        if not 0.0 < decay <= 1.0:
            raise ValueError("decay must be in (0, 1]")
        self.k_max = int(k_max)
        self.decay = float(decay)
        self.total = _Window(np.zeros(self.k_max), np.zeros(self.k_max))
        self._ew_reached = np.zeros(self.k_max)
        self._ew_accepted = np.zeros(self.k_max)

    def update(self, accepted, k_per_row=None) -> None:
        n = np.asarray(accepted, dtype=np.int64).ravel()
        if k_per_row is None:
            kb = np.full(n.shape, self.k_max, dtype=np.int64)
        else:
            kb = np.asarray(k_per_row, dtype=np.int64).ravel()
            if kb.shape != n.shape:
                raise ValueError("accepted and k_per_row differ in length")
        if np.any(kb < 0) or np.any(kb > self.k_max):
            raise ValueError("k_per_row outside [0, k_max]")
        ok = n >= 0
        if np.any(n[ok] > kb[ok]):
            raise ValueError("an accepted count exceeds its row's draft length")
        n, kb = n[ok], kb[ok]
        t = np.arange(self.k_max)[None, :]
        reached = ((t < kb[:, None]) & (n[:, None] >= t)).sum(axis=0).astype(np.float64)
        acc = ((t < kb[:, None]) & (n[:, None] > t)).sum(axis=0).astype(np.float64)
        self.total.reached += reached
        self.total.accepted += acc
        self.total.rounds += int(n.size)
        self.total.tokens += int(np.sum(n + 1))
        self.total.errors += int(np.count_nonzero(~ok))
        self._ew_reached = self.decay * self._ew_reached + reached
        self._ew_accepted = self.decay * self._ew_accepted + acc

    @staticmethod
    def _ratio(num: np.ndarray, den: np.ndarray) -> np.ndarray:
        out = np.full(num.shape, np.nan)
        np.divide(num, den, out=out, where=den > 0)
        return out

    def alpha(self) -> np.ndarray:
        """All-time acceptance rate per position (NaN where never reached)."""
        return self._ratio(self.total.accepted, self.total.reached)

    def alpha_recent(self) -> np.ndarray:
        """Acceptance rate per position with exponential forgetting."""
        return self._ratio(self._ew_accepted, self._ew_reached)

    def alpha_pooled(self) -> float:
        """Accepted drafts / reached draft positions, over all positions."""
        den = float(self.total.reached.sum())
        return float(self.total.accepted.sum()) / den if den > 0 else float("nan")

    def stderr(self) -> np.ndarray:
        a = self.alpha()
        out = np.full(a.shape, np.nan)
        np.divide(np.sqrt(a * (1.0 - a)), np.sqrt(self.total.reached), out=out, where=self.total.reached > 0)
        return out

    def tokens_per_round(self) -> float:
        """Observed mean tokens emitted per round (n + 1)."""
        return self.total.tokens / self.total.rounds if self.total.rounds else float("nan")

    def predicted_tokens_per_round(self) -> float:
        """E[tokens] from the per-position estimates (all rows at K = k_max)."""
        a = self.alpha()
        if np.any(np.isnan(a)):
            return float("nan")
        return expected_tokens(a, self.k_max)

    def alarm(self, floor: float) -> bool:
        """True when the recent pooled acceptance rate has fallen below floor."""
        den = float(self._ew_reached.sum())
        return den > 0 and float(self._ew_accepted.sum()) / den < floor

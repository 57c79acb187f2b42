"""GPU statistics on the pages' worked example: 10^6 sequences of K = 4 draft
tokens over a four-word vocabulary, target q = [0.5, 0.25, 0.15, 0.10] and
draft p = [0.3, 0.4, 0.2, 0.1] at every position (roadtointelligence.com
"Speculative Decoding", section "Why the output doesn't change"; the
letters are swapped there).

What the pages fix, checked on the library's own outputs:
  * acceptance sum_v min(p, q) = 0.8 per position;
  * the accepted count follows a^k (1 - a), and E[tokens per pass] =
    (1 - a^(K+1)) / (1 - a) = 3.3616 (same page, "How much faster");
  * every emitted token is distributed as the target (the paperlayer.ai
    summary's Theorem 1);
  * a rejection resamples from normalize((q - p)+) = [1, 0, 0, 0].

The draft tokens come from the library's own K = 0 step (a draw from the
filtered draft). The first 20,000 sequences are also compared with the oracle
element by element.
"""
import numpy as np
import pytest
import torch
from scipy import stats

from helpers import compare, run_gpu, run_oracle
from speculative_sampling_amd import workloads
from speculative_sampling_amd.binding import ST_ERRORS, Verifier

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

Q = np.array([0.5, 0.25, 0.15, 0.10])
P = np.array([0.3, 0.4, 0.2, 0.1])
A = 0.8


@pytest.fixture(scope="module")
def run():
    dev = torch.device("cuda", 0)
    B, K = 1_000_000, 4
    w = workloads.worked_example(B, K, device=dev, seed=1, draft_seed=1001)
    print(f"[worked_example_gpu] B={B} K={K}: drawing drafts", flush=True)
    sampler = Verifier(B * K, 0, 4, torch.float32)
    toks, st = sampler.sample(w.draft.reshape(-1, 4), seed=w.draft_seed)
    torch.cuda.synchronize()
    sampler.close()
    assert int(((st & ST_ERRORS) != 0).sum()) == 0
    w.draft_tokens = toks.reshape(B, K).to(torch.int32).contiguous()
    print("[worked_example_gpu] verifying", flush=True)
    out = run_gpu(w)
    return w, out


def test_draft_tokens_follow_p(run):
    w, _ = run
    toks = w.draft_tokens.cpu().numpy().ravel()
    counts = np.bincount(toks, minlength=4)
    _, pval = stats.chisquare(counts, P * toks.size)
    print(f"[worked_example_gpu] draft tokens: chi-square p = {pval:.3f}", flush=True)
    assert pval > 0.01


def test_per_position_acceptance(run):
    _, out = run
    n = out["accepted"]
    for t in range(4):
        reached = np.count_nonzero(n >= t)
        acc = np.count_nonzero(n > t) / reached
        assert abs(acc - A) < 4 * np.sqrt(A * (1 - A) / reached), (t, acc)


def test_accepted_count_law(run):
    _, out = run
    n = out["accepted"]
    law = np.array([A ** k * (1 - A) for k in range(4)] + [A ** 4])
    _, pval = stats.chisquare(np.bincount(n, minlength=5), law * n.size)
    print(f"[worked_example_gpu] accepted counts: chi-square p = {pval:.3f}", flush=True)
    assert pval > 0.01


def test_expected_tokens_per_pass(run):
    _, out = run
    emitted = out["accepted"] + 1
    e_tokens = (1 - A ** 5) / (1 - A)
    assert round(e_tokens, 4) == 3.3616
    assert abs(emitted.mean() - e_tokens) < 4 * emitted.std() / np.sqrt(emitted.size)


def test_emitted_tokens_follow_target(run):
    """Chi-square over the 10^6 sequences, p > 0.01, for the tokens emitted at
    each output position and pooled over all of them (each emitted token is
    distributed as the target: roadtointelligence.com "Speculative
    Decoding", "Why the output doesn't change")."""
    _, out = run
    toks = out["out_tokens"]
    for i in range(5):
        col = toks[:, i]
        col = col[col >= 0]
        _, pval = stats.chisquare(np.bincount(col, minlength=4), Q * col.size)
        print(f"[worked_example_gpu] position {i}: chi-square p = {pval:.3f}", flush=True)
        assert pval > 0.01, i
    # Pooled over every emitted token.  Tokens of one sequence are dependent
    # (a long accepted run leans towards min(p, q) / a), so a plain
    # chi-square over the pooled counts would be miscalibrated.  Sequences
    # are i.i.d., and each emitted token is q-distributed, so the residual
    # r_b = c_b - (n_b + 1) q (c_b: sequence b's token counts) has mean 0:
    # the Wald statistic of sum_b r_b with the empirical covariance is
    # chi-square with 3 degrees of freedom (the 4 counts sum to n_b + 1).
    c = np.stack([(toks == v).sum(1) for v in range(4)], 1).astype(np.float64)
    r = (c - c.sum(1, keepdims=True) * Q[None, :])[:, :3]
    R = r.sum(0)
    W = float(R @ np.linalg.solve(np.cov(r, rowvar=False) * r.shape[0], R))
    pval = stats.chi2.sf(W, 3)
    print(f"[worked_example_gpu] pooled: Wald chi-square p = {pval:.3f}", flush=True)
    assert pval > 0.01


def test_every_rejection_emits_token_0(run):
    _, out = run
    n = out["accepted"]
    y = out["out_tokens"][np.arange(n.size), n]
    assert np.all(y[n < 4] == 0)


def test_emission_invariants(run):
    w, out = run
    n = out["accepted"]
    toks = out["out_tokens"]
    drafts = w.draft_tokens.cpu().numpy()
    idx = np.arange(5)[None, :]
    assert n.min() >= 0 and n.max() <= 4
    assert np.all(toks[idx > n[:, None]] == -1) and np.all(toks[idx <= n[:, None]] >= 0)
    prefix = idx[:, :4] < n[:, None]
    assert np.all(toks[:, :4][prefix] == drafts[prefix])
    assert np.all(out["row_status"] & ST_ERRORS == 0)


def test_first_sequences_match_oracle(run):
    w, out = run
    m = 20_000
    sub = workloads.Workload(w.name, m, w.K_max, w.V, w.dtype, w.target[:m], w.draft[:m], w.draft_tokens[:m],
                             default_mode=w.default_mode, default_temperature=w.default_temperature,
                             seed=w.seed)
    ref = run_oracle(sub)
    compare({k: v[:m] for k, v in out.items()}, ref, "f32", "worked_example_gpu_first")


def test_monitor_on_library_outputs(run):
    """The acceptance monitor fed with the library's accepted counts gives
    0.8 at every position and the loop model's 3.3616 tokens per round."""
    from speculative_sampling_amd import loop_model

    _, out = run
    mon = loop_model.AcceptanceMonitor(4)
    mon.update(out["accepted"])
    assert mon.total.errors == 0
    assert np.all(np.abs(mon.alpha() - A) < 4 * mon.stderr())
    pred = loop_model.expected_tokens(A, 4)
    assert mon.tokens_per_round() == pytest.approx(pred, abs=4 * np.sqrt(loop_model.tokens_variance(A, 4) / 1e6))


def test_non_iid_rounds_expected_tokens_and_first_token_law():
    """100,000 rounds shaped like batch-1 serving (K = 4, V = 32000 bf16,
    target N(0, 3^2), draft = target + N(0, 1), plain sampling at
    temperature 1), batched 10,000 rounds per call.  The acceptance rate
    differs from round to round, so:
      * given the logits, a round emits n + 1 tokens with
        E = 1 + sum_k prod_{t<k} a_t, a_t = sum_v min(p_t(v), q_t(v))
        (roadtointelligence.com "How much faster", per position), and the
        law of n + 1 gives its variance: sum(n + 1 - E) is tested as a
        normal z-score;
      * the first emitted token follows q_0 whatever happens at position 0
        (the paperlayer.ai summary's Theorem 1): its randomised PIT
        F(y - 1) + V q(y), V ~ U(0, 1), is uniform (Kolmogorov-Smirnov).
    The expectations are computed in fp64 from the same bf16 logits."""
    from speculative_sampling_amd import loop_model

    dev = torch.device("cuda", 0)
    B, K, V, batches = 10_000, 4, 32000, 10
    gen_v = torch.Generator(device=dev).manual_seed(2468)
    dev_sum, var_sum = 0.0, 0.0
    pits = []
    for i in range(batches):
        print(f"[non_iid_rounds] batch {i}", flush=True)
        w = workloads.iid_normal(B, K, V, sigma_t=3.0, sigma_d=1.0, gen_seed=3000 + i, seed=4000 + i,
                                 device=dev)
        sampler = Verifier(B * K, 0, V, torch.bfloat16)
        toks, st = sampler.sample(w.draft.reshape(-1, V), seed=w.draft_seed)
        torch.cuda.synchronize()
        sampler.close()
        assert int(((st & ST_ERRORS) != 0).sum()) == 0
        w.draft_tokens = toks.reshape(B, K).to(torch.int32).contiguous()
        out = run_gpu(w)
        assert int(((out["row_status"] & ST_ERRORS) != 0).sum()) == 0
        # per-round acceptance rates in fp64
        alpha = torch.empty(B, K, dtype=torch.float64, device=dev)
        for t in range(K):
            q = torch.softmax(w.target[:, t].double(), dim=-1)
            p = torch.softmax(w.draft[:, t].double(), dim=-1)
            alpha[:, t] = torch.minimum(p, q).sum(-1)
            del p
            if t == 0:
                y0 = torch.from_numpy(out["out_tokens"][:, 0]).to(dev).long()
                qy = q.gather(1, y0[:, None])[:, 0]
                before = q.cumsum(-1).gather(1, y0[:, None])[:, 0] - qy
                u = before + torch.rand(B, generator=gen_v, device=dev, dtype=torch.float64) * qy
                pits.append(u.clamp(0.0, 1.0).cpu().numpy())
            del q
        a = alpha.cpu().numpy()
        n1 = out["accepted"].astype(np.float64) + 1.0
        exp = np.array([loop_model.expected_tokens(a[b]) for b in range(B)])
        var = np.array([loop_model.tokens_variance(a[b]) for b in range(B)])
        dev_sum += float(np.sum(n1 - exp))
        var_sum += float(np.sum(var))
    z = dev_sum / np.sqrt(var_sum)
    assert abs(z) < 4.5, f"z = {z:.2f}"
    ks = stats.kstest(np.concatenate(pits), "uniform")
    assert ks.pvalue > 1e-3, f"KS p = {ks.pvalue:.2e}"
    print(f"[non_iid_rounds] z = {z:.2f}, KS p = {ks.pvalue:.3f}", flush=True)

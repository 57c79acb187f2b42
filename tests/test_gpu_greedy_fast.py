"""Greedy verification without the draft's logits: the HIP library against
the oracle.

Under greedy decoding a draft token is kept exactly when it is the target's
argmax at its position, and the token emitted at the first rejection, or
the bonus token, is the target's argmax there (FDE Interviews breakdown of
Chen et al., the greedy row of the figure "The idea, visually";
roadtointelligence "Speculative Decoding", "How it works": the rule becomes
sampling from a one-hot distribution).  So the draft's logits are not
needed: with draft_logits = NULL the library streams only the K_b + 1 target
rows of a sequence and draws no uniforms.

The oracle runs the same inputs with the draft's logits (its GREEDY mode).
Accepted counts, tokens and q_t(d_t) must agree exactly.  Without the draft
the library cannot give p_t(d_t) (NaN in diag) or the status bits that need
the draft's argmax (zero residual, p(d) = 0); those are left out of the
comparison.  Greedy decisions are comparisons of logits, with no boundary
window, so no row may differ.
"""
import numpy as np
import pytest
import torch

from helpers import run_gpu, run_oracle, with_oracle_drafts
from speculative_sampling_amd import workloads
from speculative_sampling_amd.binding import ST_ERRORS, SV_GREEDY, Verifier

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_without_draft(w, device=0):
    dev = torch.device("cuda", device)
    v = Verifier(w.B, w.K_max, w.V, w.target.dtype, device)

    def d(x):
        return None if x is None else x.to(dev)
    acc, toks, st, diag = v(d(w.target), None, d(w.draft_tokens), k_per_row=d(w.k_per_row),
                            default_mode=SV_GREEDY, seed=w.seed)
    torch.cuda.synchronize()
    out = {"accepted": acc.cpu().numpy(), "out_tokens": toks.cpu().numpy(),
           "row_status": st.cpu().numpy().view(np.uint32), "diag": diag.cpu().numpy()}
    v.close()
    return out


def check_greedy(w, label):
    ref = run_oracle(w)
    print(f"[{label}] B={w.B} K={w.K_max} V={w.V} {w.dtype}: without the draft's logits", flush=True)
    gpu = run_without_draft(w)
    assert np.array_equal(gpu["accepted"], ref["accepted"]), label
    assert np.array_equal(gpu["out_tokens"], ref["out_tokens"]), label
    assert np.array_equal(gpu["row_status"] & ST_ERRORS, ref["row_status"].astype(np.uint32) & ST_ERRORS), label
    # q_t(d_t) is 1 or 0; p_t(d_t) needs the draft
    q_gpu, q_ref = gpu["diag"][..., 0], ref["diag"][..., 0]
    assert np.array_equal(np.isnan(q_gpu), np.isnan(q_ref)), label
    assert np.array_equal(np.nan_to_num(q_gpu, nan=-1), np.nan_to_num(q_ref.astype(np.float32), nan=-1)), label
    assert np.all(np.isnan(gpu["diag"][..., 1])), label
    # the same call with the draft's logits gives the same tokens
    print(f"[{label}] with the draft's logits", flush=True)
    full = run_gpu(w)
    assert np.array_equal(full["accepted"], gpu["accepted"]), label
    assert np.array_equal(full["out_tokens"], gpu["out_tokens"]), label
    return gpu, ref


def test_greedy_without_draft_at_config4_shape():
    """B=256, K=8, V=32000 fp32, target N(0, 3^2), draft = target + N(0, 1)."""
    w = with_oracle_drafts(workloads.iid_normal(256, 8, 32000, sigma_t=3.0, sigma_d=1.0, dtype="f32",
                                                mode=SV_GREEDY, temperature=0.7, gen_seed=41, seed=40))
    gpu, _ = check_greedy(w, "greedy_nodraft_f32")
    # drafts drawn from the draft's argmax agree with the target's often
    assert 0 < gpu["accepted"].mean() < w.K_max


def test_greedy_without_draft_bf16_ragged():
    w = workloads.zipf_ragged(24, 8, 64000, gen_seed=43, seed=42)
    w.mode = None
    w.default_mode = SV_GREEDY
    w = with_oracle_drafts(w)
    check_greedy(w, "greedy_nodraft_bf16_ragged")


def test_greedy_ties_take_the_lowest_index():
    """Rows whose maximum is held by several tokens: the argmax is the lowest
    of them; a draft token at a higher tied index is rejected and the lowest
    is emitted, a draft token at the lowest is kept."""
    B, K, V = 16, 3, 5000
    g = torch.Generator().manual_seed(44)
    target = torch.randn(B, K + 1, V, generator=g) * 2.0
    tied = torch.zeros(B, K + 1, 3, dtype=torch.long)
    for b in range(B):
        for t in range(K + 1):
            idx = torch.randperm(V, generator=g)[:3].sort().values
            target[b, t, idx] = 12.0   # three tokens share the maximum
            tied[b, t] = idx
    target = target.to(torch.bfloat16)
    draft = target[:, :K].clone()
    tokens = torch.empty(B, K, dtype=torch.int32)
    for b in range(B):
        for t in range(K):
            # even sequences: the lowest tied index (kept); odd: another tied index (rejected)
            tokens[b, t] = int(tied[b, t, 0]) if b % 2 == 0 else int(tied[b, t, 1 + (t % 2)])
    w = workloads.Workload("ties", B, K, V, "bf16", target.contiguous(), draft.contiguous(), tokens,
                           default_mode=SV_GREEDY, seed=45)
    gpu, ref = check_greedy(w, "greedy_ties")
    for b in range(B):
        if b % 2 == 0:
            assert gpu["accepted"][b] == K and gpu["out_tokens"][b, K] == int(tied[b, K, 0])
        else:
            assert gpu["accepted"][b] == 0 and gpu["out_tokens"][b, 0] == int(tied[b, 0, 0])

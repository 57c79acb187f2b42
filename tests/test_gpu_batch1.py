"""Batch-1 serving, call by call: one sequence per call, K = 4 draft tokens,
V = 32000 bf16 logits (target N(0, 3^2), draft = target + N(0, 1^2)), plain
sampling at temperature 1, and the round index r as the Philox seed of
round r (sequence id 0 in every call).  This is the serving setting of the
pages (FDE Interviews breakdown, "The problem": one token at a time at
batch 1; paperlayer.ai summary, "Results").  Every round's call is compared
with the oracle's on the same inputs: accepted count, tokens, status bits
and the probabilities of the draft tokens.
"""
import numpy as np
import pytest
import torch

from helpers import compare, run_oracle, with_oracle_drafts
from speculative_sampling_amd import workloads
from speculative_sampling_amd.binding import Verifier

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ROUNDS = 2000


def test_batch1_rounds_match_oracle_call_by_call():
    dev = torch.device("cuda", 0)
    K, V = 4, 32000
    w = with_oracle_drafts(workloads.iid_normal(ROUNDS, K, V, sigma_t=3.0, sigma_d=1.0, gen_seed=606,
                                                seed=0))
    tgt, drf, tok = w.target.to(dev), w.draft.to(dev), w.draft_tokens.to(dev)
    v = Verifier(1, K, V, torch.bfloat16)
    acc = torch.empty(ROUNDS, dtype=torch.int32, device=dev)
    out = torch.empty(ROUNDS, K + 1, dtype=torch.int32, device=dev)
    st = torch.empty(ROUNDS, dtype=torch.int32, device=dev)
    diag = torch.empty(ROUNDS, K, 2, dtype=torch.float32, device=dev)
    print(f"[batch1] {ROUNDS} calls of B=1 K={K} V={V} bf16 plain", flush=True)
    for r in range(ROUNDS):
        v(tgt[r:r + 1], drf[r:r + 1], tok[r:r + 1], seed=r,
          out=(acc[r:r + 1], out[r:r + 1], st[r:r + 1], diag[r:r + 1]))
    torch.cuda.synchronize()
    v.close()
    gpu = {"accepted": acc.cpu().numpy(), "out_tokens": out.cpu().numpy(),
           "row_status": st.cpu().numpy().view(np.uint32), "diag": diag.cpu().numpy()}
    print("[batch1] oracle", flush=True)
    keys = ("accepted", "out_tokens", "row_status", "diag", "flags")
    ref = {k: [] for k in keys}
    for r in range(ROUNDS):
        sub = workloads.Workload(w.name, 1, K, V, w.dtype, w.target[r:r + 1], w.draft[r:r + 1],
                                 w.draft_tokens[r:r + 1], default_mode=w.default_mode,
                                 default_temperature=w.default_temperature, seed=r)
        o = run_oracle(sub)
        for k in keys:
            ref[k].append(o[k])
    ref = {k: np.concatenate(x) for k, x in ref.items()}
    n_flag, err = compare(gpu, ref, "bf16", "batch1_rounds")
    print(f"[batch1] flagged={n_flag} max|diag err|={err:.2e} mean accepted="
          f"{gpu['accepted'].mean():.3f}", flush=True)

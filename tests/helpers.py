"""Shared test plumbing: run a workload through the oracle and the GPU
library and compare them element by element.

Parity rule (both sides take the same seeded inputs):
  * rows the oracle flags (a decision within 1e-6 of its boundary) are
    excluded from exact comparison; there may be at most
    max(1, ceil(1e-4 * B)) of them;
  * on every other row the accepted count, every emitted token, the error
    bits and the discrete info bits (zero residual, p(d) = 0) are equal;
  * diag (q_t(d_t), p_t(d_t)) agrees within DIAG_TOL absolute.
"""
import math

import numpy as np
import torch

import oracle
from speculative_sampling_amd import workloads
from speculative_sampling_amd.binding import (ST_ERRORS, ST_PZERO, ST_ZERO_RESIDUAL, Verifier)

# fp32 and bf16 probability tolerances; the fp32-accumulating kernels are
# expected to be far inside both (the tests report the actual maximum).
DIAG_TOL = {"f32": 1e-5, "bf16": 2e-3}


def oracle_sampler(rows, mode, temperature, top_k, top_p, dmode, dtemp, dtopk, dtopp, seed):
    def np_(x):
        return None if x is None else x.cpu().numpy()
    toks = oracle.sample_rows(workloads.host_array(rows), mode=np_(mode), temperature=np_(temperature),
                              top_k=np_(top_k), top_p=np_(top_p), default_mode=dmode,
                              default_temperature=dtemp, default_top_k=dtopk, default_top_p=dtopp,
                              seed=seed)
    return torch.from_numpy(toks.astype(np.int32))


def run_oracle(w: workloads.Workload, rows=None, row_offset: int = 0):
    """Oracle outputs for sequences `rows` (default: all) of w."""
    sel = slice(None) if rows is None else rows

    def np_(x):
        return None if x is None else x[sel].cpu().numpy()
    tgt = workloads.host_array(w.target[sel])
    drf = workloads.host_array(w.draft[sel])
    return oracle.verify(tgt, drf, w.draft_tokens[sel].cpu().numpy(), k_per_row=np_(w.k_per_row),
                         mode=np_(w.mode), temperature=np_(w.temperature), top_k=np_(w.top_k),
                         top_p=np_(w.top_p), default_mode=w.default_mode,
                         default_temperature=w.default_temperature, default_top_k=w.default_top_k,
                         default_top_p=w.default_top_p, seed=w.seed, row_offset=row_offset)


def run_gpu(w: workloads.Workload, verifier: Verifier = None, row_offset: int = 0, device=0):
    dev = torch.device("cuda", device)
    own = verifier is None
    if own:
        verifier = Verifier(w.B, w.K_max, w.V, w.target.dtype, device)

    def d(x):
        return None if x is None else x.to(dev)
    acc, toks, st, diag = verifier(d(w.target), d(w.draft), d(w.draft_tokens), k_per_row=d(w.k_per_row),
                                   mode=d(w.mode), temperature=d(w.temperature), top_k=d(w.top_k),
                                   top_p=d(w.top_p), default_mode=w.default_mode,
                                   default_temperature=w.default_temperature,
                                   default_top_k=w.default_top_k, default_top_p=w.default_top_p,
                                   seed=w.seed, row_offset=row_offset)
    torch.cuda.synchronize()
    out = {"accepted": acc.cpu().numpy(), "out_tokens": toks.cpu().numpy(),
           "row_status": st.cpu().numpy().view(np.uint32), "diag": diag.cpu().numpy()}
    if own:
        verifier.close()
    return out


def compare(gpu: dict, ref: dict, dtype: str, label: str = "", rate_bound: bool = True):
    """Asserts parity; returns (n_flagged, max_diag_err).  rate_bound=False
    drops the flagged-row rate bound for parameters chosen to sit on a
    boundary (flagged rows are still excluded from exact comparison)."""
    B = ref["accepted"].shape[0]
    flagged = ref["flags"] != 0
    n_flag = int(flagged.sum())
    if rate_bound:
        assert n_flag <= max(1, math.ceil(1e-4 * B)), f"{label}: {n_flag} flagged rows of {B}"
    ok = ~flagged
    acc_g, acc_r = gpu["accepted"][ok], ref["accepted"][ok]
    bad = np.nonzero(acc_g != acc_r)[0]
    assert bad.size == 0, f"{label}: accepted differs on rows {np.nonzero(ok)[0][bad][:10]}"
    tg, tr = gpu["out_tokens"][ok], ref["out_tokens"][ok]
    bad = np.nonzero((tg != tr).any(axis=1))[0]
    assert bad.size == 0, (f"{label}: tokens differ on rows {np.nonzero(ok)[0][bad][:10]}: "
                           f"gpu {tg[bad[:3]].tolist()} oracle {tr[bad[:3]].tolist()}")
    bits = ST_ERRORS | ST_ZERO_RESIDUAL | ST_PZERO
    sg = gpu["row_status"][ok] & bits
    sr = ref["row_status"][ok].astype(np.uint32) & bits
    bad = np.nonzero(sg != sr)[0]
    assert bad.size == 0, f"{label}: status differs on rows {np.nonzero(ok)[0][bad][:10]}: {sg[bad[:5]]} vs {sr[bad[:5]]}"
    dg = gpu["diag"].astype(np.float64)
    dr = ref["diag"]
    both_nan = np.isnan(dg) & np.isnan(dr)
    assert np.array_equal(np.isnan(dg), np.isnan(dr)), f"{label}: diag NaN pattern differs"
    err = np.abs(np.where(both_nan, 0.0, dg - dr))
    max_err = float(err.max()) if err.size else 0.0
    assert max_err <= DIAG_TOL[dtype], f"{label}: diag error {max_err}"
    return n_flag, max_err


def with_oracle_drafts(w: workloads.Workload) -> workloads.Workload:
    return workloads.draw_draft_tokens(w, oracle_sampler)


def gpu_sampler(rows, mode, temperature, top_k, top_p, dmode, dtemp, dtopk, dtopp, seed):
    """The library's K = 0 step as a draft sampler (rows on the GPU)."""
    dev = rows.device

    def d(x):
        return None if x is None else x.to(dev)
    v = Verifier(rows.shape[0], 0, rows.shape[-1], rows.dtype, dev.index or 0)
    toks, _ = v.sample(rows, seed=seed, mode=d(mode), temperature=d(temperature), top_k=d(top_k),
                       top_p=d(top_p), default_mode=dmode, default_temperature=dtemp,
                       default_top_k=dtopk, default_top_p=dtopp)
    torch.cuda.synchronize()
    v.close()
    return toks.reshape(-1).to(torch.int32)

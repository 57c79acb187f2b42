"""Shared test plumbing: run a workload through the oracle and the GPU
library and compare them element by element.

Parity rule (both sides take the same seeded inputs):
  * the oracle flags a row when a decision it used lies within 1e-6 of its
    boundary (an accept ratio, a CDF step, a nucleus cut); only flagged rows
    may differ;
  * every row is compared: a row whose accepted count, tokens or discrete
    status bits (errors, zero residual, p(d) = 0) differ must be flagged,
    and such differing rows may be at most 1e-4 of the rows compared.  Each
    comparison adds its rows, flagged rows and differing rows to
    FLAG_TALLY; the last GPU test module checks the session's totals.  A
    single comparison may differ on at most max(1, ceil(1e-4 * B)) rows;
  * diag (q_t(d_t), p_t(d_t)) agrees within DIAG_TOL absolute on every row.

How many rows are flagged depends on the inputs, not on the GPU: plain
sampling over 32000 near-uniform tokens puts a uniform within 1e-6 of a CDF
step in about 2.5% of rows, since most tokens' intervals are only a few
1e-6 wide; a peaked nucleus flags about 1e-5 of rows.
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

# rows compared, rows flagged and rows that differ, over the session
FLAG_TALLY = {"rows": 0, "flagged": 0, "differ": 0}


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


def compare(gpu: dict, ref: dict, dtype: str, label: str = "", diag_only: bool = False):
    """Asserts parity; returns (n_flagged, max_diag_err).  diag_only=True is
    for parameters chosen to put every row on a boundary: the rows must all
    be flagged, only diag is compared, and the comparison stays out of the
    tally."""
    B = ref["accepted"].shape[0]
    flagged = ref["flags"] != 0
    n_flag = int(flagged.sum())
    if diag_only:
        assert n_flag == B, f"{label}: a diag-only case must flag every row ({n_flag} of {B})"
    else:
        bits = ST_ERRORS | ST_ZERO_RESIDUAL | ST_PZERO
        differ = (gpu["accepted"] != ref["accepted"]) | (gpu["out_tokens"] != ref["out_tokens"]).any(axis=1) | \
                 ((gpu["row_status"] & bits) != (ref["row_status"].astype(np.uint32) & bits))
        bad = np.nonzero(differ & ~flagged)[0]
        assert bad.size == 0, (
            f"{label}: unflagged rows differ: {bad[:10].tolist()}: accepted gpu "
            f"{gpu['accepted'][bad[:3]].tolist()} oracle {ref['accepted'][bad[:3]].tolist()}, tokens gpu "
            f"{gpu['out_tokens'][bad[:3]].tolist()} oracle {ref['out_tokens'][bad[:3]].tolist()}, status gpu "
            f"{gpu['row_status'][bad[:3]].tolist()} oracle {ref['row_status'][bad[:3]].tolist()}")
        n_diff = int(differ.sum())
        assert n_diff <= max(1, math.ceil(1e-4 * B)), f"{label}: {n_diff} flagged rows of {B} differ"
        FLAG_TALLY["rows"] += B
        FLAG_TALLY["flagged"] += n_flag
        FLAG_TALLY["differ"] += n_diff
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

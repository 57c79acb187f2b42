"""Rows streamed in parts, against the oracle on every row.

A call of between 1 and 3 rows per CU, not a whole number of them (257..767
rows of at least 8 chunks, one filter of plain, nucleus or greedy), streams
its first 256 or 512 rows whole and splits every further row into 2 to 4
parts, one work-group each, so that every CU streams about the same bytes;
the last part of a row to
arrive merges the parts' softmax records and candidate lists and finishes
the row.  The merged row must give the same filtered distributions as one
work-group over the whole row (FDE Interviews breakdown of Chen et al.,
section 01; paperlayer.ai summary of arXiv 2302.01318, "Modified Rejection
Sampling"): these cases put split rows under every filter the split serves,
under ragged K_b, error rows and nucleus lists that need narrower windows.
"""
import numpy as np
import pytest
import torch

from helpers import compare, run_gpu, run_oracle, with_oracle_drafts
from speculative_sampling_amd import workloads
from speculative_sampling_amd.binding import (ST_EMPTY, ST_ERRORS, ST_FULLSELECT, ST_NONFINITE, SV_GREEDY,
                                              SV_PLAIN, SV_TOPP)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

CUS, MAX_PARTS, ROW_WAVES = 256, 4, 4


def split_plan(rows, V, dtype):
    """(rows streamed whole, parts per further row) as the library plans a
    launch (the same rule as its row_split)."""
    S = -(-V // (4096 if dtype == "bf16" else 2048))
    if rows <= CUS or rows >= 3 * CUS or rows % CUS == 0:
        return rows, 1
    whole = rows // CUS * CUS
    p = min(CUS // (rows - whole), MAX_PARTS, S // ROW_WAVES)
    return (whole, p) if p >= 2 else (rows, 1)


def check(w, label):
    full, parts = split_plan(w.B * (2 * w.K_max + 1), w.V, w.dtype)
    assert parts > 1, "the case must split rows"
    w = with_oracle_drafts(w)
    ref = run_oracle(w)
    print(f"[{label}] B={w.B} K={w.K_max} V={w.V} {w.dtype}: {w.B * (2 * w.K_max + 1) - full} rows in {parts} parts",
          flush=True)
    gpu = run_gpu(w)
    n_flag, err = compare(gpu, ref, w.dtype, label)
    print(f"[{label}] flagged={n_flag} max|diag err|={err:.2e}", flush=True)
    return w, gpu, ref


def test_split_nucleus_bf16():
    # 540 rows: 28 rows in 2 parts
    w, gpu, _ = check(workloads.peaked(60, 4, 40000, gen_seed=81, seed=80), "split_nucleus")
    assert not np.any(gpu["row_status"] & ST_FULLSELECT)   # the merged lists served every row


def test_split_nucleus_four_parts():
    # 531 rows of 16 chunks: 19 rows in 4 parts
    check(workloads.peaked(59, 4, 65536, gen_seed=83, seed=82), "split_nucleus_4")


def test_split_plain_fp32():
    # 525 rows of 10 chunks
    check(workloads.iid_normal(35, 7, 20000, sigma_t=3.0, sigma_d=1.0, dtype="f32", temperature=1.2,
                               gen_seed=85, seed=84), "split_plain_f32")


def test_split_greedy_bf16():
    check(workloads.iid_normal(60, 4, 40000, sigma_t=3.0, sigma_d=1.0, mode=SV_GREEDY, gen_seed=87, seed=86),
          "split_greedy")


def test_split_nucleus_wide_lists():
    """A flat nucleus (top-p 0.95 over logits of sd 1): each part's waves
    list thousands of vectors and narrow their windows; the merge then
    narrows the row's window or hands the row to the whole-row selection."""
    check(workloads.iid_normal(58, 4, 40000, sigma_t=1.0, sigma_d=0.3, mode=SV_TOPP, temperature=1.0,
                               top_p=0.95, gen_seed=89, seed=88), "split_nucleus_wide")


def test_split_one_row_per_cu_and_parts():
    # 288 rows: 256 whole, 32 in 2 parts; and 270 plain rows, 14 in 4 parts
    check(workloads.peaked(32, 4, 40000, gen_seed=97, seed=96), "split_nucleus_256")
    check(workloads.iid_normal(30, 4, 70000, sigma_t=3.0, sigma_d=1.0, gen_seed=99, seed=98), "split_plain_256")


def test_split_greedy_without_draft_logits():
    # without the draft's logits only the target rows are launched: 60
    # sequences x 5 = 300 rows, 256 whole and 44 in 2 parts
    w = workloads.iid_normal(60, 4, 40000, sigma_t=3.0, sigma_d=1.0, mode=SV_GREEDY, gen_seed=101, seed=100)
    w = with_oracle_drafts(w)
    ref = run_oracle(w)
    w.draft = None
    full, parts = split_plan(60 * 5, 40000, "bf16")
    assert parts > 1
    print(f"[split_greedy_nodraft] 300 target rows: {300 - full} in {parts} parts", flush=True)
    gpu = run_gpu(w)
    assert np.array_equal(gpu["accepted"], ref["accepted"])
    assert np.array_equal(gpu["out_tokens"], ref["out_tokens"])


def test_split_rows_with_errors_and_ragged_k():
    """Ragged K_b (padding rows return before streaming, in every part) and
    error rows among the split ones: a NaN in one part only, +inf in
    another, an empty row."""
    B, K, V = 60, 4, 40000
    w = workloads.peaked(B, K, V, gen_seed=91, seed=90)
    w = with_oracle_drafts(w)
    g = torch.Generator().manual_seed(92)
    w.k_per_row = torch.randint(1, K + 1, (B,), generator=g).to(torch.int32)
    w.k_per_row[57:] = K                           # the split rows are those of the last sequences
    tgt, drf = w.target.float(), w.draft.float()
    tgt[57, 4, V - 5] = float("nan")               # the last part of a split row
    drf[58, 1, 3] = float("inf")                   # the first part of another
    tgt[59, 0, :] = float("-inf")                  # an empty split row
    w.target, w.draft = tgt.to(torch.bfloat16).contiguous(), drf.to(torch.bfloat16).contiguous()
    full, parts = split_plan(B * (2 * K + 1), V, "bf16")
    assert parts > 1 and full // (2 * K + 1) < 57
    ref = run_oracle(w)
    gpu = run_gpu(w)
    compare(gpu, ref, "bf16", "split_errors")
    for b, bit in {57: ST_NONFINITE, 58: ST_NONFINITE, 59: ST_EMPTY}.items():
        assert gpu["row_status"][b] & ST_ERRORS == bit, b
        assert gpu["accepted"][b] == -1
    assert np.all(gpu["row_status"][:57] & ST_ERRORS == 0)


def test_split_twice_in_a_row():
    # the per-row arrival counters are left at zero: a second call, and a
    # call of another split shape after it, give the same results
    w = with_oracle_drafts(workloads.peaked(60, 4, 40000, gen_seed=93, seed=92))
    a = run_gpu(w)
    b = run_gpu(w)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    w2 = workloads.iid_normal(58, 4, 40000, sigma_t=3.0, sigma_d=1.0, mode=SV_PLAIN, gen_seed=95, seed=94)
    check(w2, "split_after_split")

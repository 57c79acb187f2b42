"""The workloads at their full sizes, in the launch configuration of the
benchmark (one call over the whole batch), checked against the oracle on
sampled sequences: the oracle recomputes a sequence from its own inputs
with row_offset set to its index, so its random numbers are those the GPU
used for that sequence.

  * B=256, K=8, V=32000 fp32, top-k 40 at temperature 0.7, draft noise
    sigma 0.3, 1.0 and 2.0, and the greedy variant at sigma 1.0;
  * B=512, ragged K_b ~ U{1..8}, V=256000 bf16, Zipf-shaped logits with a
    per-row vocabulary permutation, modes cycling plain / top-k 50 /
    top-p 0.9 at temperature 0.7;
  * B=100,000, K=4, V=32000 bf16, plain at temperature 1 (the batch-1
    serving rounds in one call);
  * the headline B=64, K=4, V=128256 bf16 shape in plain mode; its nucleus
    form is checked on sampled sequences in test_gpu_parity.py.

Draft tokens come from the library's own K = 0 step on the draft rows; the
GPU sampler is compared with the oracle's in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

from helpers import compare, gpu_sampler, run_gpu, run_oracle
from speculative_sampling_amd import workloads
from speculative_sampling_amd.binding import ST_ERRORS

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def check_sampled(w, picks, label):
    print(f"[{label}] B={w.B} K={w.K_max} V={w.V} {w.dtype}: drafts", flush=True)
    workloads.draw_draft_tokens(w, gpu_sampler)
    print(f"[{label}] verify", flush=True)
    gpu = run_gpu(w)
    for b in picks:
        ref = run_oracle(w, rows=slice(b, b + 1), row_offset=b)
        compare({k: v[b:b + 1] for k, v in gpu.items()}, ref, w.dtype, f"{label}_b{b}")
    print(f"[{label}] ok", flush=True)
    return gpu


@pytest.mark.parametrize("sigma", ["0.3", "1.0", "2.0"])
def test_topk_fp32_full(sigma):
    # draft noise sigma 0.3 / 1.0 / 2.0: acceptance from high to low
    dev = torch.device("cuda", 0)
    w = workloads.config(f"topk_f32_s{sigma}", device=dev, gen_seed=31, seed=3)
    gpu = check_sampled(w, (0, 97, 255), f"topk_f32_s{sigma}_full")
    assert np.all(gpu["row_status"] & ST_ERRORS == 0)
    del w
    torch.cuda.empty_cache()


def test_greedy_fp32_full():
    dev = torch.device("cuda", 0)
    w = workloads.config("topk_f32_greedy_s1.0", device=dev, gen_seed=32, seed=4)
    check_sampled(w, (0, 128, 255), "greedy_f32_full")


def test_zipf_ragged_full():
    dev = torch.device("cuda", 0)
    w = workloads.config("zipf_ragged", device=dev, gen_seed=33, seed=5)
    gpu = check_sampled(w, (0, 1, 2, 256, 510, 511), "zipf_ragged_full")
    kb = w.k_per_row.cpu().numpy()
    assert np.all(gpu["accepted"] >= 0) and np.all(gpu["accepted"] <= kb)
    del w
    torch.cuda.empty_cache()


def test_plain_b100000_full():
    dev = torch.device("cuda", 0)
    w = workloads.config("latency_b1", device=dev, B=100000, gen_seed=34, seed=6)
    gpu = check_sampled(w, (0, 1, 4097, 50000, 99998, 99999), "plain_b100000_full")
    assert np.all(gpu["row_status"] & ST_ERRORS == 0)
    del w
    torch.cuda.empty_cache()


def test_plain_headline_shape_full():
    dev = torch.device("cuda", 0)
    w = workloads.config("plain_b64", device=dev, gen_seed=35, seed=7)
    gpu = check_sampled(w, (0, 21, 42, 63), "plain_b64_full")
    assert np.all(gpu["row_status"] & ST_ERRORS == 0)
    del w
    torch.cuda.empty_cache()

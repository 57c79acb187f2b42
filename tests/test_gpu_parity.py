"""GPU parity: the HIP library against the oracle, element by element, on
the same seeded inputs (draft tokens drawn by the oracle's own sampler from
the filtered draft distribution).  Shapes follow the workloads of the
method at sizes the oracle finishes in seconds, spanning several chunks and
a ragged tail; the full-size headline shape is checked on sampled rows.
"""
import numpy as np
import pytest
import torch

from helpers import DIAG_TOL, compare, run_gpu, run_oracle, with_oracle_drafts
from speculative_sampling_amd import workloads
from speculative_sampling_amd.binding import (ST_ERRORS, ST_FULLSELECT, ST_NONFINITE, ST_PARAM,
                                              ST_REREAD, ST_TOKEN, ST_EMPTY, SV_GREEDY, SV_PLAIN,
                                              SV_TOPK, SV_TOPP, Verifier)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def check(w, label, diag_only=False):
    w = with_oracle_drafts(w)
    ref = run_oracle(w)
    print(f"[{label}] B={w.B} K={w.K_max} V={w.V} {w.dtype}", flush=True)
    gpu = run_gpu(w)
    n_flag, err = compare(gpu, ref, w.dtype, label, diag_only)
    print(f"[{label}] flagged={n_flag} max|diag err|={err:.2e}", flush=True)
    return w, gpu, ref


def test_worked_example_parity():
    check(workloads.worked_example(20000), "worked_example")


def test_plain_bf16_parity():
    _, gpu, _ = check(workloads.iid_normal(48, 4, 32000, sigma_t=3.0, sigma_d=1.0, gen_seed=5, seed=3),
                      "plain_bf16")
    # plain draws read the rows again (every token kept: no threshold test)
    assert np.all(gpu["row_status"] & ST_REREAD)


def test_plain_fp32_parity():
    check(workloads.iid_normal(24, 3, 20000, dtype="f32", temperature=1.3, gen_seed=6, seed=4),
          "plain_f32")


def test_nucleus_parity():
    w, gpu, _ = check(workloads.peaked(8, 4, 128256, gen_seed=7, seed=5), "nucleus_bf16")
    assert not np.any(gpu["row_status"] & ST_FULLSELECT)   # the candidate path served every row


@pytest.mark.parametrize("sigma", [0.3, 1.0, 2.0])
def test_topk_fp32_parity(sigma):
    check(workloads.iid_normal(24, 8, 32000, sigma_t=3.0, sigma_d=sigma, dtype="f32", mode=SV_TOPK,
                               temperature=0.7, top_k=40, gen_seed=8, seed=6), f"topk_f32_s{sigma}")


@pytest.mark.parametrize("k", [1, 50, 300])
def test_topk_bf16_parity(k):
    """bf16 top-k at the headline's vocabulary.  The streaming pass searches
    the cut on the vectors' maxima; bf16 logits often tie at the cut (ties
    are kept).  k = 300 exceeds a chunk's list capacity (256 vectors), so
    every row takes the full-row selection."""
    w, gpu, _ = check(workloads.peaked(6, 4, 128256, mode=SV_TOPK, top_k=k, gen_seed=40 + k, seed=9),
                      f"topk_bf16_k{k}")
    if k == 300:
        assert np.all(gpu["row_status"][gpu["accepted"] >= 0] & ST_FULLSELECT)


@pytest.mark.parametrize("V,dtype", [(20000, "f32"), (40000, "bf16")])
def test_topk_rows_across_work_groups(V, dtype):
    """Five chunks per row: work-groups of four chunks hold chunks of two
    rows, and only chunks of the same row share a top-k cut."""
    w = workloads.iid_normal(5, 3, V, sigma_t=3.0, sigma_d=1.0, dtype=dtype, mode=SV_TOPK,
                             temperature=0.7, top_k=30, gen_seed=70, seed=13)
    check(w, f"topk_span_{dtype}_V{V}")


def test_greedy_fp32_parity():
    check(workloads.iid_normal(32, 8, 32000, sigma_t=3.0, sigma_d=1.0, dtype="f32", mode=SV_GREEDY,
                               temperature=0.7, gen_seed=9, seed=7), "greedy_f32")


def test_mixed_ragged_parity():
    w, gpu, ref = check(workloads.zipf_ragged(12, 8, 64000, gen_seed=10, seed=8), "zipf_ragged")
    assert np.all(gpu["accepted"] <= w.k_per_row.numpy())


@pytest.mark.parametrize("V,dtype", [(40000, "bf16"), (20000, "f32")])
def test_every_mode_in_one_call(V, dtype):
    """A mode per sequence runs one streaming instance holding every path:
    greedy, top-k, nucleus and plain rows, and rows whose top-k covers the
    vocabulary or whose top-p is 1 (plain), side by side in one call, with
    per-row temperatures and ragged K."""
    B, K = 18, 4
    w = workloads.iid_normal(B, K, V, sigma_t=3.0, sigma_d=1.0, dtype=dtype, gen_seed=90, seed=15)
    g = torch.Generator().manual_seed(91)
    w.mode = torch.tensor([SV_GREEDY, SV_TOPK, SV_TOPP, SV_PLAIN, SV_TOPK, SV_TOPP] * 3, dtype=torch.uint8)
    w.top_k = torch.tensor([1, 40, 1, 1, V, 1] * 3, dtype=torch.int32)
    w.top_p = torch.tensor([1.0, 1.0, 0.8, 1.0, 1.0, 1.0] * 3, dtype=torch.float32)
    w.temperature = (0.5 + torch.rand(B, generator=g)).to(torch.float32)
    w.k_per_row = torch.randint(0, K + 1, (B,), generator=g).to(torch.int32)
    _, gpu, _ = check(w, f"every_mode_{dtype}")
    assert np.all(gpu["accepted"] <= w.k_per_row.numpy())


@pytest.mark.parametrize("V,dtype", [(1001, "bf16"), (999, "f32"), (1, "bf16"), (7, "f32")])
def test_unaligned_vocab_parity(V, dtype):
    # rows that are not a multiple of 16 bytes take the element-wise load path
    check(workloads.iid_normal(16, 3, V, dtype=dtype, gen_seed=11, seed=9), f"plain_V{V}")
    check(workloads.iid_normal(16, 3, V, dtype=dtype, mode=SV_TOPP, temperature=0.9, top_p=0.7,
                               gen_seed=12, seed=10), f"topp_V{V}")
    check(workloads.iid_normal(16, 3, V, dtype=dtype, mode=SV_TOPK, top_k=min(5, V), gen_seed=13,
                               seed=11), f"topk_V{V}")


@pytest.mark.parametrize("mode", [SV_PLAIN, SV_TOPP, SV_TOPK])
def test_maximum_draft_length(mode):
    # K = 64, the largest the library accepts: 129 rows per sequence, several
    # rows per wave of the sequence kernel, kept sets in global memory
    check(workloads.iid_normal(3, 64, 3000, sigma_d=0.3, mode=mode, temperature=0.9, top_p=0.8,
                               top_k=20, gen_seed=40, seed=41), f"k64_{mode}")
    # identical models accept all 64 drafts and draw the bonus from q_64
    w, gpu, _ = check(workloads.iid_normal(3, 64, 3000, sigma_d=0.0, mode=mode, temperature=0.9,
                                           top_p=0.8, top_k=20, gen_seed=46, seed=47), f"k64_same_{mode}")
    assert np.all(gpu["accepted"] == 64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_maximum_vocab(dtype):
    # V = 2^22, the largest the library accepts: 512 (bf16) or 1024 (fp32)
    # chunks per row, tile sums beyond the LDS cache in the row draw
    V = 1 << 22
    check(workloads.iid_normal(2, 2, V, dtype=dtype, gen_seed=42, seed=43), f"vmax_plain_{dtype}")
    check(workloads.iid_normal(2, 2, V, dtype=dtype, mode=SV_TOPP, temperature=0.5, top_p=0.9,
                               gen_seed=42, seed=43), f"vmax_topp_{dtype}")
    check(workloads.iid_normal(2, 2, V, dtype=dtype, mode=SV_TOPK, temperature=0.7, top_k=50,
                               gen_seed=42, seed=43), f"vmax_topk_{dtype}")


def test_empty_batch():
    # B = 0 launches nothing and returns success
    dev = torch.device("cuda", 0)
    v = Verifier(4, 3, 1000, torch.bfloat16)
    tgt = torch.zeros(0, 4, 1000, dtype=torch.bfloat16, device=dev)
    drf = torch.zeros(0, 3, 1000, dtype=torch.bfloat16, device=dev)
    toks = torch.zeros(0, 3, dtype=torch.int32, device=dev)
    acc, out, st, _ = v(tgt, drf, toks, seed=1)
    torch.cuda.synchronize()
    v.close()
    assert acc.numel() == 0 and out.shape == (0, 4) and st.numel() == 0


def test_k0_is_a_single_draw():
    w = workloads.iid_normal(64, 0, 5000, gen_seed=14, seed=12)
    check(w, "k0")


def test_edge_parameters():
    # top-p = 1 and top-k = V are plain sampling; k above the candidate list
    # capacity and all-equal logits take the full-row selection
    B, K, V = 8, 3, 3000
    base = workloads.iid_normal(B, K, V, gen_seed=15, seed=13)
    for mode, kw in [(SV_TOPP, {"default_top_p": 1.0}), (SV_TOPK, {"default_top_k": V}),
                     (SV_TOPK, {"default_top_k": 700}), (SV_TOPP, {"default_top_p": 0.97}),
                     (SV_TOPP, {"default_top_p": 0.999})]:
        w = workloads.Workload("edge", B, K, V, "bf16", base.target.clone(), base.draft.clone(),
                               default_mode=mode, default_temperature=0.9, seed=13, draft_seed=99, **kw)
        # at top_p = 0.999 the tail tokens' masses are far below 1e-6, so the
        # cut always lies within 1e-6 of top_p: every row is flagged, and
        # only the probabilities are compared (test_nucleus_near_one compares
        # tokens at a top_p this close to 1)
        _, gpu, _ = check(w, f"edge_{mode}_{kw}", diag_only=kw.get("default_top_p") == 0.999)
        if kw.get("default_top_k") == 700:
            # kept sets beyond the 512-entry list: drawn from the re-read rows
            # with the kept-set threshold applied per token
            assert np.any(gpu["row_status"] & ST_REREAD)
    flat = torch.zeros(B, K + 1, V, dtype=torch.bfloat16)
    flat[:, :, ::7] = 1.0   # big tied groups
    w = workloads.Workload("ties", B, K, V, "bf16", flat, flat[:, :K].clone(), default_mode=SV_TOPP,
                           default_top_p=0.5, default_temperature=1.0, seed=14, draft_seed=98)
    _, gpu, _ = check(w, "ties_topp")
    assert np.all(gpu["row_status"] & ST_FULLSELECT)


def test_nucleus_near_one():
    """Nucleus with top_p just below 1, token for token.  Tail tokens have
    masses far below 1e-6 here, so top_p = 0.999 lands within 1e-6 of a cut
    on almost every row.  Each sequence instead gets the first top_p of
    0.990, 0.991, ..., 0.999 (per-row top_p, its draft tokens drawn from the
    draft filtered at that top_p) at which the oracle flags none of its
    decisions, so every cut lies more than 1e-6 from its top_p."""
    import oracle
    B, K, V = 12, 3, 20000
    w = workloads.iid_normal(B, K, V, sigma_t=1.5, sigma_d=0.5, mode=SV_TOPP, temperature=0.9,
                             top_p=0.995, gen_seed=23, seed=21)
    chosen = np.full(B, np.nan, np.float32)
    toks = torch.zeros(B, K, dtype=torch.int32)
    for c in np.round(np.arange(0.990, 0.9995, 0.001), 3).astype(np.float32):
        w.top_p = torch.full((B,), float(c), dtype=torch.float32)
        w = with_oracle_drafts(w)
        ref = run_oracle(w)
        free = torch.from_numpy(np.isnan(chosen) & (ref["flags"] == 0))
        chosen[free.numpy()] = c
        toks[free] = w.draft_tokens[free]
    assert not np.any(np.isnan(chosen)), "no top_p in [0.990, 0.999] leaves some sequence unflagged"
    w.top_p = torch.from_numpy(chosen)
    w.draft_tokens = toks
    ref = run_oracle(w)
    assert np.all(ref["flags"] == 0)
    print(f"[nucleus_near_one] top_p per row {chosen.tolist()}", flush=True)
    gpu = run_gpu(w)
    compare(gpu, ref, "bf16", "nucleus_near_one")
    kept = [oracle.row_probs(workloads.host_array(w.target[b, 0]), oracle.TOPP, 0.9,
                             top_p=float(chosen[b]))[3] for b in range(B)]
    assert min(kept) > 2048     # more tokens than a chunk's candidate list holds


def test_large_logits_take_the_exact_exponent_path():
    w = workloads.iid_normal(8, 3, 8000, gen_seed=16, seed=15, temperature=0.5)
    w.target = (w.target.float() + 3000.0).to(torch.bfloat16)
    w.draft = (w.draft.float() + 3000.0).to(torch.bfloat16)
    check(w, "large_logits")


@pytest.mark.parametrize("dtype,mode", [("bf16", SV_PLAIN), ("f32", SV_PLAIN), ("bf16", SV_TOPP)])
def test_one_dominant_token_at_low_temperature(dtype, mode):
    """One token per row sits 40 logits above the rest, at tau = 0.5: the
    row's terms span about 2^-115 .. 1, and the dominant token lies far above
    the largest logit of most lanes' first vectors, so the sums are taken
    with an exponent offset that the row's own maximum must raise (the chunk
    holding the token is redone from its exact maximum).  q(d) near 1 and
    the tail's tiny masses must both match the oracle."""
    B, K, V = 16, 4, 40000
    w = workloads.iid_normal(B, K, V, sigma_t=1.0, sigma_d=0.5, dtype=dtype, mode=mode, temperature=0.5,
                             top_p=0.9, gen_seed=61, seed=60)
    g = torch.Generator().manual_seed(62)
    tgt, drf = w.target.float(), w.draft.float()
    for b in range(B):
        for t in range(K + 1):
            i = int(torch.randint(0, V, (1,), generator=g))
            tgt[b, t, i] += 40.0
            if t < K:
                drf[b, t, i] += 40.0 if b % 2 == 0 else 0.0   # odd sequences: the draft misses it
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    w.target, w.draft = tgt.to(dt).contiguous(), drf.to(dt).contiguous()
    check(w, f"dominant_{dtype}_{mode}")


def test_error_rows():
    B, K, V = 10, 3, 4096
    w = workloads.iid_normal(B, K, V, gen_seed=17, seed=16)
    w = with_oracle_drafts(w)
    w.target[0, 1, 100] = float("nan")           # NaN in a used row
    w.draft[1, 2, 5] = float("inf")               # +inf in a used row
    w.target[2, 0, :] = float("-inf")             # empty row
    w.draft_tokens[3, 1] = V                      # token out of range
    w.draft_tokens[4, 0] = -5
    w.k_per_row = torch.full((B,), K, dtype=torch.int32)
    w.k_per_row[5] = K + 1                        # K_b > K_max
    w.k_per_row[6] = 1
    w.target[6, 2:, :] = float("nan")             # NaN only in padding: fine
    w.draft[6, 1:, :] = float("nan")
    w.temperature = torch.full((B,), 1.0)
    w.temperature[7] = 0.0                        # invalid temperature
    w.target[8, 3, 17] = float("-inf")            # -inf is a valid logit
    ref = run_oracle(w)
    gpu = run_gpu(w)
    compare(gpu, ref, "bf16", "errors")
    want = {0: ST_NONFINITE, 1: ST_NONFINITE, 2: ST_EMPTY, 3: ST_TOKEN, 4: ST_TOKEN, 5: ST_PARAM,
            7: ST_PARAM}
    for b, bit in want.items():
        assert gpu["row_status"][b] & ST_ERRORS == bit, b
        assert gpu["accepted"][b] == -1 and np.all(gpu["out_tokens"][b] == -1)
    for b in (6, 8, 9):
        assert gpu["row_status"][b] & ST_ERRORS == 0


def test_invalid_mode_value():
    w = with_oracle_drafts(workloads.iid_normal(6, 2, 2048, gen_seed=18, seed=17))
    w.mode = torch.tensor([0, 1, 2, 3, 9, 0], dtype=torch.uint8)
    w.top_k = torch.full((6,), 5, dtype=torch.int32)
    w.top_p = torch.full((6,), 0.8)
    gpu = run_gpu(w)
    ref = run_oracle(w)
    compare(gpu, ref, "bf16", "modes")
    assert gpu["row_status"][4] & ST_PARAM and gpu["accepted"][4] == -1


def test_deterministic_and_row_offset_split():
    w = with_oracle_drafts(workloads.peaked(6, 4, 50000, gen_seed=19, seed=18))
    a = run_gpu(w)
    b = run_gpu(w)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    # two calls over halves with row_offset give the same result as one call
    v = Verifier(6, 4, 50000, torch.bfloat16)
    lo = workloads.Workload(w.name, 3, 4, w.V, w.dtype, w.target[:3], w.draft[:3], w.draft_tokens[:3],
                            default_mode=w.default_mode, default_temperature=w.default_temperature,
                            default_top_p=w.default_top_p, seed=w.seed)
    hi = workloads.Workload(w.name, 3, 4, w.V, w.dtype, w.target[3:], w.draft[3:], w.draft_tokens[3:],
                            default_mode=w.default_mode, default_temperature=w.default_temperature,
                            default_top_p=w.default_top_p, seed=w.seed)
    glo = run_gpu(lo, v, row_offset=0)
    ghi = run_gpu(hi, v, row_offset=3)
    v.close()
    assert np.array_equal(np.concatenate([glo["out_tokens"], ghi["out_tokens"]]), a["out_tokens"])


def test_gpu_sampler_matches_oracle_sampler():
    import oracle
    w = workloads.zipf_ragged(6, 4, 20000, gen_seed=20, seed=19)
    md, tmp, tk, tp = w.row_params()
    rows = w.draft.reshape(-1, w.V)
    v = Verifier(rows.shape[0], 0, w.V, torch.bfloat16)
    dev = torch.device("cuda", 0)
    ok = ~torch.isnan(rows.float()).any(dim=1)
    g_toks, st = v.sample(rows.to(dev), seed=77, mode=md.to(dev), temperature=tmp.to(dev),
                          top_k=tk.to(dev), top_p=tp.to(dev))
    torch.cuda.synchronize()
    v.close()
    o_toks = oracle.sample_rows(workloads.host_array(rows), mode=md.numpy(), temperature=tmp.numpy(),
                                top_k=tk.numpy(), top_p=tp.numpy(), seed=77)
    g = g_toks.cpu().numpy()
    assert np.array_equal(g[ok.numpy()], o_toks[ok.numpy()])


def test_sampler_over_several_launches():
    """6,000,000 single-row draws (K = 0, V = 4, fp32): more sequences than
    one launch of the sequence kernel takes (2^22, so that its grid stays
    below 2^32 work-items), so the call is split in two.  Rows on both sides
    of the split and at the ends match the oracle's sampler exactly."""
    import oracle
    dev = torch.device("cuda", 0)
    n, V = 6_000_000, 4
    g = torch.Generator().manual_seed(404)
    rows = torch.randn(n, V, generator=g) * 2.0
    v = Verifier(n, 0, V, torch.float32)
    print(f"[sampler_split] rows={n} V={V}", flush=True)
    toks, st = v.sample(rows.to(dev), seed=55)
    torch.cuda.synchronize()
    v.close()
    toks, st = toks.cpu().numpy(), st.cpu().numpy()
    assert int(((st & ST_ERRORS) != 0).sum()) == 0
    assert toks.min() >= 0 and toks.max() < V
    x = rows.numpy()
    split = 1 << 22
    for lo, hi in ((0, 300), (split - 300, split + 300), (n - 300, n)):
        ref = oracle.sample_rows(x[lo:hi], seed=55, row_offset=lo)
        assert np.array_equal(toks[lo:hi], ref), (lo, hi)


def test_headline_shape_sampled_rows():
    # B=64, K=4, V=128256 bf16 nucleus: whole batch on the GPU, the oracle on
    # a sample of sequences (same global row ids via row_offset)
    w = workloads.peaked(64, 4, 128256, gen_seed=21, seed=20)
    w = with_oracle_drafts(w)
    gpu = run_gpu(w)
    for b in (0, 17, 33, 63):
        ref = run_oracle(w, rows=slice(b, b + 1), row_offset=b)
        sub = {k: v[b:b + 1] for k, v in gpu.items()}
        compare(sub, ref, "bf16", f"headline_b{b}")
    assert np.all(gpu["row_status"] & ST_ERRORS == 0)

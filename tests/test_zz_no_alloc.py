"""spec_verify_run_static, the entry point that allocates nothing (for
callers that cannot call hipMalloc), against spec_verify_run on the same
inputs.  They share every kernel, so every output must be equal bit for bit.
Two static calls in a row, the second smaller than the first, since all
calls on a device share one static buffer that keeps the previous call's
contents."""
import numpy as np
import pytest
import torch

from helpers import with_oracle_drafts
from speculative_sampling_amd import binding, workloads
from speculative_sampling_amd.binding import SV_TOPK, SV_TOPP, SV_PLAIN, SV_GREEDY, Verifier

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _kw(w, dev):
    def d(x):
        return None if x is None else x.to(dev)
    return dict(k_per_row=d(w.k_per_row), mode=d(w.mode), temperature=d(w.temperature), top_k=d(w.top_k),
                top_p=d(w.top_p), default_mode=w.default_mode, default_temperature=w.default_temperature,
                default_top_k=w.default_top_k, default_top_p=w.default_top_p, seed=w.seed)


def _outs(B, K, dev):
    return (torch.full((B,), -7, dtype=torch.int32, device=dev),
            torch.full((B, K + 1), -7, dtype=torch.int32, device=dev),
            torch.full((B,), -7, dtype=torch.int32, device=dev),
            torch.full((B, K, 2), -7.0, dtype=torch.float32, device=dev))


def _both(w, label):
    dev = torch.device("cuda", 0)
    dt = w.target.dtype
    tgt, drf, tok = w.target.to(dev), w.draft.to(dev), w.draft_tokens.to(dev)
    kw = _kw(w, dev)
    v = Verifier(w.B, w.K_max, w.V, dt)
    ref = v(tgt, drf, tok, **kw)
    torch.cuda.synchronize()
    v.close()
    out = _outs(w.B, w.K_max, dev)
    args = binding.make_args(tgt, drf, tok, accepted=out[0], out_tokens=out[1], row_status=out[2],
                             diag=out[3], **kw)
    print(f"[no_alloc] {label}: B={w.B} K={w.K_max} V={w.V} {w.dtype}", flush=True)
    binding.spec_verify_run_static(w.V, dt, args)
    torch.cuda.synchronize()
    for name, a, b in zip(("accepted", "out_tokens", "row_status", "diag"), out, ref):
        assert torch.equal(torch.isnan(a), torch.isnan(b)) if a.is_floating_point() else True, name
        a_, b_ = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(a_, b_, equal_nan=True), f"{label}: {name} differs"
    assert int(out[0].min().item()) >= 0


def test_static_entry_matches_handle_entry_on_two_calls():
    big = with_oracle_drafts(workloads.peaked(8, 4, 128256, gen_seed=501, seed=502))
    _both(big, "first call (nucleus)")
    small = workloads.iid_normal(5, 3, 40000, sigma_t=3.0, sigma_d=1.0, gen_seed=503, seed=504)
    g = torch.Generator().manual_seed(505)
    small.mode = torch.tensor([SV_PLAIN, SV_TOPK, SV_TOPP, SV_GREEDY, SV_TOPP], dtype=torch.uint8)
    small.top_k = torch.full((5,), 30, dtype=torch.int32)
    small.top_p = torch.full((5,), 0.85, dtype=torch.float32)
    small.temperature = (0.6 + torch.rand(5, generator=g)).to(torch.float32)
    small.k_per_row = torch.tensor([3, 1, 2, 3, 0], dtype=torch.int32)
    _both(with_oracle_drafts(small), "second call (smaller, mixed modes, ragged K)")


def test_static_entry_with_rows_streamed_in_parts():
    # 540 rows: the rows beyond two per CU are streamed in parts, whose
    # arrival counters sit in the static buffer and must be left at zero
    split = with_oracle_drafts(workloads.peaked(60, 4, 40000, gen_seed=507, seed=508))
    _both(split, "rows in parts")
    _both(split, "rows in parts, again")
    plain = workloads.iid_normal(58, 4, 40000, sigma_t=3.0, sigma_d=1.0, mode=SV_PLAIN, gen_seed=509, seed=510)
    _both(with_oracle_drafts(plain), "rows in parts, plain, smaller")


def test_static_entry_refuses_a_call_beyond_its_buffer():
    dev = torch.device("cuda", 0)
    B, K, V = 4096, 8, 256000
    assert binding.spec_verify_workspace_bytes(B, K, V, torch.bfloat16) > binding.SV_STATIC_SCRATCH_BYTES
    tgt = torch.zeros(1, dtype=torch.bfloat16, device=dev)  # never read: refused on the host
    args = binding.SvArgs()
    args.B, args.K_max = B, K
    args.target_logits = args.draft_logits = tgt.data_ptr()
    args.draft_tokens = args.accepted = args.out_tokens = tgt.data_ptr()
    args.default_temperature = 1.0
    with pytest.raises(binding.SpecVerifyError, match="static scratch"):
        binding.spec_verify_run_static(V, torch.bfloat16, args)

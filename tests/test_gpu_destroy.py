"""spec_verify_destroy waits for the handle's runs (GPU).

The library records no event per run, so destroy cannot tell which streams
a handle's runs used; it waits for the whole device instead, as the header
states.  A run enqueued on a stream of its own and followed at once by
destroy, with no synchronisation by the caller, must have finished when
destroy returns, with its outputs equal to those of a run that was waited
for normally.
"""
import numpy as np
import pytest
import torch

from speculative_sampling_amd import binding, workloads
from speculative_sampling_amd.binding import SV_TOPP

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _call(v, w, out, stream):
    args = binding.make_args(w.target, w.draft, w.draft_tokens, accepted=out[0], out_tokens=out[1],
                             row_status=out[2], diag=out[3], default_mode=SV_TOPP,
                             default_temperature=0.8, default_top_p=0.8, seed=11)
    binding.spec_verify_run(v.handle, args, stream.cuda_stream)


def test_destroy_waits_for_runs_on_other_streams():
    dev = torch.device("cuda", 0)
    w = workloads.peaked(64, 4, 128256, gen_seed=50, seed=1, device=dev)
    w.draft_tokens = torch.argmax(w.draft.float(), dim=-1).to(torch.int32).contiguous()
    # reference: a run that is waited for
    ref_v = binding.Verifier(64, 4, 128256, torch.bfloat16)
    ref_out = ref_v.outputs(64, 4)
    _call(ref_v, w, ref_out, torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.cpu().numpy() for t in ref_out]
    ref_v.close()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    v1 = binding.Verifier(64, 4, 128256, torch.bfloat16)
    v2 = binding.Verifier(64, 4, 128256, torch.bfloat16)
    out1, out2 = v1.outputs(64, 4), v2.outputs(64, 4)
    torch.cuda.synchronize()   # the outputs' allocation is done before the runs
    for _ in range(3):          # a few queued runs, so that destroy finds work in flight
        _call(v1, w, out1, s1)
        _call(v2, w, out2, s2)
    binding.spec_verify_destroy(v1.handle)
    v1.handle = 0
    # v1's runs are finished, and so is every other stream's work (device-wide)
    assert s1.query() and s2.query()
    got = [t.cpu().numpy() for t in out1]
    for a, b in zip(got, ref):
        assert np.array_equal(a, b, equal_nan=a.dtype.kind == 'f')
    v2.close()

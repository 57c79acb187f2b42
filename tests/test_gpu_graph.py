"""The verify call captured into a HIP graph (stream capture through
torch.cuda.graph).  The graph's kernels read the buffers given at capture,
so each replay runs on the data then in them: three ragged, mixed-mode
batches are copied in turn into the captured buffers, replayed, and each
replay must equal an eager call on the same batch bit for bit (the same
kernels, seed and sequence ids).  Eager calls run between the replays."""
import numpy as np
import pytest
import torch

from helpers import gpu_sampler
from speculative_sampling_amd import binding, workloads
from speculative_sampling_amd.binding import ST_ERRORS, Verifier

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _args(w, bufs, out):
    return binding.make_args(bufs["target"], bufs["draft"], bufs["draft_tokens"], accepted=out[0],
                             out_tokens=out[1], row_status=out[2], diag=out[3],
                             k_per_row=bufs["k_per_row"], mode=bufs["mode"],
                             temperature=bufs["temperature"], top_k=bufs["top_k"], top_p=bufs["top_p"],
                             default_mode=w.default_mode, default_temperature=w.default_temperature,
                             default_top_k=w.default_top_k, default_top_p=w.default_top_p, seed=77)


def _host(out):
    return [x.cpu().numpy() for x in out]


def test_graph_replays_match_eager():
    dev = torch.device("cuda", 0)
    B, K, V = 12, 8, 20000
    names = ("target", "draft", "draft_tokens", "k_per_row", "mode", "temperature", "top_k", "top_p")
    ws = []
    for i in range(3):
        w = workloads.zipf_ragged(B, K, V, gen_seed=60 + i, seed=77, device=dev)
        workloads.draw_draft_tokens(w, gpu_sampler)
        ws.append(w)
    static = {n: getattr(ws[0], n).clone() for n in names}
    v = Verifier(B, K, V, torch.bfloat16)
    out = v.outputs(B, K)
    args = _args(ws[0], static, out)
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        binding.spec_verify_run(v.handle, args, side)  # eager warm-up before capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("[graph] capture", flush=True)
    binding.spec_verify_profile_begin(v.handle, 4)  # stage events are not recorded under capture
    with torch.cuda.graph(g):
        binding.spec_verify_run(v.handle, args)
    torch.cuda.synchronize()
    calls, _ = binding.spec_verify_profile_end(v.handle)
    assert calls == 0
    ref_v = Verifier(B, K, V, torch.bfloat16)
    for rep in range(2):
        for i, w in enumerate(ws):
            print(f"[graph] replay {rep} batch {i}", flush=True)
            for n in names:
                static[n].copy_(getattr(w, n))
            g.replay()
            torch.cuda.synchronize()
            got = _host(out)
            ref_out = ref_v.outputs(B, K)
            ref_v(*(getattr(w, n) for n in names[:3]), out=ref_out, k_per_row=w.k_per_row, mode=w.mode,
                  temperature=w.temperature, top_k=w.top_k, top_p=w.top_p, default_mode=w.default_mode,
                  default_temperature=w.default_temperature, default_top_k=w.default_top_k,
                  default_top_p=w.default_top_p, seed=77)
            torch.cuda.synchronize()
            ref = _host(ref_out)
            assert int(((ref[2] & ST_ERRORS) != 0).sum()) == 0
            for a, b in zip(got[:3], ref[:3]):
                assert np.array_equal(a, b), (rep, i)
            assert np.array_equal(got[3], ref[3], equal_nan=True), (rep, i)
    del g
    torch.cuda.synchronize()
    ref_v.close()
    v.close()

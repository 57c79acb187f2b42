"""The streaming-ceiling probes (measurement helpers, not part of the
method): they read whole blocks of a device buffer (8 KB for the fixed
probe; 64 x 4, 8 or 16 vectors of 16 bytes for the sweep) and return
without error, including a partial last block (ignored), an empty range and
fewer blocks than the persistent grid has waves."""
import pytest
import torch

from speculative_sampling_amd import binding

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("nbytes", [0, 8192, 8192 * 37 + 1000, 147750912])
def test_stream_probe_reads_whole_blocks(nbytes):
    dev = torch.device("cuda", 0)
    print(f"[stream_probe] bytes={nbytes}", flush=True)
    buf = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    binding.spec_verify_stream_probe(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    # an all-zero buffer folds to 0, never the value that writes the sink
    assert int(sink.item()) == 0


@pytest.mark.parametrize("loads,waves", [(4, 1), (8, 3), (16, 8), (8, 32)])
@pytest.mark.parametrize("nbytes", [0, 4096, 16384 * 37 + 1000, 147750912])
def test_stream_probe_sweep_reads_whole_blocks(loads, waves, nbytes):
    dev = torch.device("cuda", 0)
    print(f"[stream_probe_sweep] loads={loads} waves={waves} bytes={nbytes}", flush=True)
    buf = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    binding.spec_verify_stream_probe_sweep(buf.data_ptr(), nbytes, loads, waves, sink.data_ptr(),
                                           stream.cuda_stream)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_stream_probe_sweep_rejects_bad_parameters():
    dev = torch.device("cuda", 0)
    buf = torch.zeros(4096, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for loads, waves in [(2, 4), (12, 4), (8, 0), (8, 33), (32, 4)]:
        with pytest.raises(binding.SpecVerifyError):
            binding.spec_verify_stream_probe_sweep(buf.data_ptr(), 4096, loads, waves, sink.data_ptr(), 0)

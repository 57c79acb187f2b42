"""The streaming-ceiling probe (a measurement helper, not part of the
method): it reads whole 16 KB blocks of a device buffer and returns without
error, including a partial last block (ignored) and an empty range."""
import pytest
import torch

from speculative_sampling_amd import binding

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("nbytes", [0, 16384, 16384 * 37 + 1000, 147750912])
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

"""The device's random numbers against the oracle's own Philox4x32-10, word
for word.  The step draws every uniform from word 0 of Philox4x32-10
(Salmon, Moraes, Dror and Shaw, SC'11; keyed by the seed, counter = the
sequence's global index, position and purpose) as (word >> 8) / 2^24; the
oracle's generator is written independently and pinned to the published
known-answer vectors (test_oracle_philox.py).  Here the library's device
generator is compared with it on more than 10^6 counters, random and at
the edges of every counter word."""
import numpy as np
import pytest
import torch

import oracle
from speculative_sampling_amd import binding

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def device_words(seed, g, t, p):
    dev = torch.device("cuda", 0)
    gd = torch.from_numpy(g.view(np.int64)).to(dev)
    td = torch.from_numpy(t.view(np.int32)).to(dev)
    pd = torch.from_numpy(p.view(np.int32)).to(dev)
    out = torch.zeros(g.size, dtype=torch.int32, device=dev)
    binding.spec_verify_philox_words(seed, gd.data_ptr(), td.data_ptr(), pd.data_ptr(), g.size, out.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("seed", [0, 1, 0xDEADBEEFCAFEF00D, 2**64 - 1])
def test_device_philox_words_equal_the_oracles(seed):
    rng = np.random.default_rng(seed % 2**32 + 7)
    n = 1 << 20
    g = rng.integers(0, 2**64, n, dtype=np.uint64)
    t = rng.integers(0, 65, n, dtype=np.uint32)
    p = rng.integers(0, 3, n, dtype=np.uint32)
    # the edges of each counter word
    edge_g = np.array([0, 1, 2**32 - 1, 2**32, 2**63, 2**64 - 1], dtype=np.uint64)
    edge_t = np.array([0, 1, 63, 64, 2**31, 2**32 - 1], dtype=np.uint32)
    eg, et, ep = np.meshgrid(edge_g, edge_t, np.array([0, 1, 2, 2**32 - 1], dtype=np.uint32), indexing="ij")
    g = np.concatenate([g, eg.ravel()])
    t = np.concatenate([t, et.ravel()])
    p = np.concatenate([p, ep.ravel()])
    dev = device_words(seed, g, t, p)
    ref = oracle.philox_words(seed, g, t, p)
    bad = np.nonzero(dev != ref)[0]
    print(f"[philox] seed={seed:#x}: {g.size} counters, {bad.size} differ", flush=True)
    assert bad.size == 0, f"first differing counter {bad[:3]}: device {dev[bad[:3]]} oracle {ref[bad[:3]]}"
    # the uniforms the step takes from them, and their range
    u = (dev >> 8).astype(np.float64) / 2**24
    assert u.min() >= 0.0 and u.max() < 1.0
    for i in (0, 1, n - 1, n):
        assert u[i] == oracle.uniform(seed, int(g[i]), int(t[i]), int(p[i]))

"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/spec_verify.h declares, and its host-side validation
rejects bad arguments before anything is launched.  Also checks that the
oracle and the library share no code."""
import ctypes
import os
import re

import pytest
import torch

from speculative_sampling_amd import binding
from speculative_sampling_amd.binding import (SV_BF16, SV_ECAPACITY, SV_EDTYPE, SV_EINVAL, SV_F32,
                                              SV_GREEDY, SV_OK, SV_PLAIN, SV_TOPK, SV_TOPP, SvArgs)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

needs_lib = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                               reason="libspec_verify.so not built (run __graft_entry__.build())")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", text)))


def test_binding_lists_every_header_function():
    assert sorted(binding.EXPORTS) == header_functions()


@needs_lib
def test_library_exports_every_header_function():
    lib = ctypes.CDLL(binding.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def _args(**kw):
    # fake, never dereferenced device addresses: validation is host-only
    a = SvArgs()
    a.B, a.K_max = kw.get("B", 4), kw.get("K_max", 2)
    a.target_logits = kw.get("target", 0x10000)
    a.draft_logits = kw.get("draft", 0x20000)
    a.draft_tokens = kw.get("tokens", 0x30000)
    a.accepted = kw.get("accepted", 0x40000)
    a.out_tokens = kw.get("out_tokens", 0x50000)
    a.mode = kw.get("mode", None)
    a.temperature = kw.get("temperature", None)
    a.top_k = kw.get("top_k_arr", None)
    a.top_p = kw.get("top_p_arr", None)
    a.default_mode = kw.get("default_mode", SV_PLAIN)
    a.default_temperature = kw.get("tau", 1.0)
    a.default_top_k = kw.get("top_k", 1)
    a.default_top_p = kw.get("top_p", 1.0)
    return a


def validate(args, max_batch=8, max_k=4, vocab=100, dtype=SV_BF16):
    return binding.spec_verify_validate(max_batch, max_k, vocab, dtype, args)


@needs_lib
def test_validate_accepts_good_arguments():
    assert validate(_args()) == SV_OK
    assert validate(_args(B=0, target=None, accepted=None)) == SV_OK
    assert validate(_args(K_max=0, draft=None, tokens=None)) == SV_OK


@needs_lib
def test_greedy_calls_may_leave_out_the_draft_logits():
    # the greedy rule needs only the target's argmax: without a mode array
    # and with greedy as the default, draft_logits may be NULL
    assert validate(_args(draft=None, default_mode=SV_GREEDY)) == SV_OK
    # any other default, or a mode array (which may name other modes), needs them
    assert validate(_args(draft=None, default_mode=SV_TOPK)) == SV_EINVAL
    assert validate(_args(draft=None, default_mode=SV_GREEDY, mode=0x60000)) == SV_EINVAL
    # the binding refuses the same calls before anything is launched
    t = torch.zeros(2, 3, 100)
    toks = torch.zeros(2, 2, dtype=torch.int32)
    out = dict(accepted=torch.zeros(2, dtype=torch.int32), out_tokens=torch.zeros(2, 3, dtype=torch.int32))
    with pytest.raises(ValueError):
        binding.make_args(t, None, toks, default_mode=SV_TOPP, **out)
    with pytest.raises(ValueError):
        binding.make_args(t, None, toks, default_mode=SV_GREEDY, mode=torch.zeros(2, dtype=torch.uint8), **out)


@needs_lib
@pytest.mark.parametrize("kw,code", [
    ({"target": None}, SV_EINVAL),
    ({"draft": None}, SV_EINVAL),
    ({"tokens": None}, SV_EINVAL),
    ({"accepted": None}, SV_EINVAL),
    ({"out_tokens": None}, SV_EINVAL),
    ({"B": 9}, SV_ECAPACITY),
    ({"K_max": 5}, SV_ECAPACITY),
    ({"B": -1}, SV_EINVAL),
    ({"default_mode": 7}, SV_EINVAL),
    ({"tau": 0.0}, SV_EINVAL),
    ({"tau": float("nan")}, SV_EINVAL),
    ({"default_mode": SV_TOPK, "top_k": 0}, SV_EINVAL),
    ({"default_mode": SV_TOPK, "top_k": 101}, SV_EINVAL),
    ({"default_mode": SV_TOPP, "top_p": 0.0}, SV_EINVAL),
    ({"default_mode": SV_TOPP, "top_p": 1.5}, SV_EINVAL),
    ({"mode": 0x60000, "top_p": 0.0}, SV_EINVAL),  # some row may use the default
])
def test_validate_rejects(kw, code):
    assert validate(_args(**kw)) == code
    assert binding.spec_verify_last_error() != ""


@needs_lib
def test_validate_refuses_long_rows_that_are_not_whole_vectors():
    # rows of more than one chunk (4096 bf16 / 2048 fp32 logits) are streamed
    # as 16-byte vectors only: V * element size a multiple of 16 and the
    # logit buffers 16-byte aligned; shorter rows may be anything
    assert validate(_args(), vocab=65536) == SV_OK
    assert validate(_args(), vocab=65543) == SV_EINVAL
    assert b"16-byte" in binding.load_library().spec_verify_last_error()
    assert validate(_args(target=0x10002), vocab=65536) == SV_EINVAL
    assert validate(_args(draft=0x20008), vocab=65536) == SV_EINVAL
    assert validate(_args(), vocab=4096) == SV_OK
    assert validate(_args(), vocab=4097) == SV_EINVAL
    assert validate(_args(), vocab=4095) == SV_OK
    assert validate(_args(), vocab=2049, dtype=SV_F32) == SV_EINVAL
    assert validate(_args(), vocab=2047, dtype=SV_F32) == SV_OK
    assert validate(_args(target=0x10004), vocab=1001) == SV_OK


@needs_lib
def test_validate_ignores_defaults_no_row_uses():
    # greedy ignores the temperature; plain ignores top-k / top-p defaults
    assert validate(_args(default_mode=SV_GREEDY, tau=0.0)) == SV_OK
    assert validate(_args(default_mode=SV_PLAIN, top_k=0, top_p=0.0)) == SV_OK
    # per-row arrays replace the defaults
    assert validate(_args(temperature=0x70000, tau=-1.0)) == SV_OK


@needs_lib
def test_validate_config():
    assert validate(_args(), dtype=7) == SV_EDTYPE
    assert validate(_args(), vocab=0) == SV_EINVAL
    assert validate(_args(), vocab=(1 << 22) + 1) == SV_EINVAL
    assert validate(_args(), max_k=65) == SV_EINVAL


@needs_lib
def test_workspace_bytes():
    small = binding.spec_verify_workspace_bytes(64, 4, 128256, SV_BF16)
    big = binding.spec_verify_workspace_bytes(128, 4, 128256, SV_BF16)
    assert 0 < small < big < 1 << 32
    assert binding.spec_verify_workspace_bytes(64, 4, 0, SV_BF16) == 0
    assert binding.spec_verify_workspace_bytes(8, 8, 32000, SV_F32) > 0


def test_oracle_and_library_share_no_code():
    lib_dir = os.path.join(ROOT, "speculative_sampling_amd")
    for dirpath, _, files in os.walk(os.path.join(ROOT, "oracle")):
        for f in files:
            if f.endswith((".cpp", ".h", ".py")):
                text = open(os.path.join(dirpath, f)).read()
                assert "speculative_sampling_amd" not in text and "sv_internal" not in text, f
                assert "spec_verify.h" not in text, f
    for dirpath, _, files in os.walk(lib_dir):
        for f in files:
            if f.endswith((".hip", ".h", ".py", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "oracle.h" not in text, f
                assert "from oracle" not in text, f


def test_product_path_fails_loudly_without_library(tmp_path):
    missing = str(tmp_path / "libspec_verify.so")
    saved = binding._lib
    binding._lib = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            binding.load_library(missing)
    finally:
        binding._lib = saved


@needs_lib
def test_stream_probe_rejects_bad_pointers_on_the_host():
    lib = binding.load_library()
    sink = ctypes.c_uint32(0)
    # NULL data or out, and data that is not 16-byte aligned, are refused
    # before anything is launched
    assert lib.spec_verify_stream_probe(None, 16384, ctypes.byref(sink), None) == SV_EINVAL
    assert lib.spec_verify_stream_probe(ctypes.c_void_p(64), 16384, None, None) == SV_EINVAL
    assert lib.spec_verify_stream_probe(ctypes.c_void_p(8), 16384, ctypes.byref(sink), None) == SV_EINVAL
    assert b"aligned" in lib.spec_verify_last_error()
    # the sweep probe checks the same, and its block and grid parameters
    assert lib.spec_verify_stream_probe_sweep(None, 16384, 8, 4, ctypes.byref(sink), None) == SV_EINVAL
    assert lib.spec_verify_stream_probe_sweep(ctypes.c_void_p(8), 16384, 8, 4, ctypes.byref(sink), None) == SV_EINVAL
    for loads, waves in [(2, 4), (12, 4), (8, 0), (8, 33), (32, 4)]:
        assert lib.spec_verify_stream_probe_sweep(ctypes.c_void_p(64), 16384, loads, waves,
                                                  ctypes.byref(sink), None) == SV_EINVAL
    # the Philox words entry: NULL arrays with n > 0 and negative n are
    # refused before anything is launched; n = 0 is a no-op
    p = ctypes.c_void_p(64)
    assert lib.spec_verify_philox_words(1, None, p, p, 4, p, None) == SV_EINVAL
    assert lib.spec_verify_philox_words(1, p, p, p, 4, None, None) == SV_EINVAL
    assert lib.spec_verify_philox_words(1, p, p, p, -1, p, None) == SV_EINVAL
    assert lib.spec_verify_philox_words(1, None, None, None, 0, None, None) == 0


def test_verifier_refuses_logits_that_disagree_with_the_handle():
    """The kernels take V (the row stride), the dtype and the device from the
    handle: a tensor that disagrees is refused before anything is launched.
    Host-only: the handle is never created."""
    import torch
    v = binding.Verifier.__new__(binding.Verifier)
    v.vocab, v.dtype, v.device, v.handle = 1000, torch.bfloat16, 0, 0
    with pytest.raises(ValueError, match="V = 999"):
        v._check_logits("target", torch.zeros(2, 3, 999, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="float32"):
        v._check_logits("draft", torch.zeros(2, 2, 1000, dtype=torch.float32))
    with pytest.raises(ValueError, match="cpu"):
        v._check_logits("target", torch.zeros(2, 3, 1000, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="V = 1001"):
        v(torch.zeros(2, 3, 1001, dtype=torch.bfloat16), None, None)
    with pytest.raises(ValueError, match="V = 7"):
        v.sample(torch.zeros(5, 7, dtype=torch.bfloat16), seed=1)


@needs_lib
def test_static_entry_refuses_calls_beyond_its_buffer_on_the_host():
    """A call whose workspace exceeds the static buffer is refused before any
    HIP call: fake device addresses are never touched."""
    lib = binding.load_library()
    need = binding.spec_verify_workspace_bytes(4096, 8, 256000, SV_BF16)
    assert need > binding.SV_STATIC_SCRATCH_BYTES
    cfg = binding.make_config(4096, 8, 256000, SV_BF16)
    rc = lib.spec_verify_run_static(ctypes.byref(cfg), ctypes.byref(_args(B=4096, K_max=8)), None)
    assert rc == SV_ECAPACITY
    msg = binding.spec_verify_last_error()
    assert str(need) in msg and "static scratch" in msg
    # argument errors are reported as by spec_verify_run
    rc = lib.spec_verify_run_static(ctypes.byref(cfg), ctypes.byref(_args(B=4096, K_max=8, target=None)), None)
    assert rc == SV_EINVAL


def test_bench_workloads_take_the_set_seeds():
    """bench.py builds every input set with config(name, gen_seed=..., seed=...);
    the small workloads are built here on the host with the same arguments
    (the worked example's logits are fixed, so its generator seed is unused)."""
    from speculative_sampling_amd import workloads
    a = workloads.config("worked_example", gen_seed=1000, seed=0, B=8)
    b = workloads.config("worked_example", gen_seed=1001, seed=1, B=8)
    assert (a.B, a.K_max, a.V) == (8, 4, 4)
    assert torch.equal(a.target, b.target) and torch.equal(a.draft, b.draft)
    c = workloads.config("latency_b1", gen_seed=1000, seed=0)
    d = workloads.config("latency_b1", gen_seed=1001, seed=1)
    assert (c.B, c.K_max, c.V) == (1, 4, 32000)
    assert not torch.equal(c.target, d.target)

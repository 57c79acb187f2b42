"""ctypes binding of libspec_verify (C ABI in include/spec_verify.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's
kernels.  The functions keep the C names.  The library must have been built
(``__graft_entry__.build()``); if it is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspec_verify.so")

SV_F32, SV_BF16 = 0, 1
SV_PLAIN, SV_TOPK, SV_TOPP, SV_GREEDY = 0, 1, 2, 3
SV_OK, SV_EINVAL, SV_ECAPACITY, SV_EDTYPE, SV_EHIP, SV_ENOMEM = 0, -1, -2, -3, -4, -5
ST_TOKEN, ST_NONFINITE, ST_EMPTY, ST_ZERO_RESIDUAL = 1, 2, 4, 8
ST_PZERO, ST_MARGIN, ST_PARAM, ST_FULLSELECT, ST_REREAD, ST_LOCATED = 16, 32, 64, 128, 256, 512
ST_ERRORS = ST_TOKEN | ST_NONFINITE | ST_EMPTY | ST_PARAM

# Every function the header declares.
EXPORTS = ("spec_verify_create", "spec_verify_run", "spec_verify_destroy",
           "spec_verify_validate", "spec_verify_workspace_bytes", "spec_verify_profile_begin",
           "spec_verify_profile_end", "spec_verify_stream_probe", "spec_verify_last_error",
           "spec_verify_run_static", "spec_verify_stream_probe_sweep", "spec_verify_philox_words")

# Size of the static device buffer spec_verify_run_static works in.
SV_STATIC_SCRATCH_BYTES = 64 << 20


class SvConfig(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("max_k", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("dtype", ctypes.c_int32), ("device", ctypes.c_int32)]


class SvArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K_max", ctypes.c_int32),
        ("target_logits", ctypes.c_void_p), ("draft_logits", ctypes.c_void_p),
        ("draft_tokens", ctypes.c_void_p), ("k_per_row", ctypes.c_void_p),
        ("mode", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
        ("top_k", ctypes.c_void_p), ("top_p", ctypes.c_void_p),
        ("default_mode", ctypes.c_int32), ("default_temperature", ctypes.c_float),
        ("default_top_k", ctypes.c_int32), ("default_top_p", ctypes.c_float),
        ("seed", ctypes.c_uint64), ("row_offset", ctypes.c_uint64),
        ("accepted", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
        ("row_status", ctypes.c_void_p), ("diag", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libspec_verify.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.spec_verify_create.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(SvConfig)]
    lib.spec_verify_create.restype = ctypes.c_int
    lib.spec_verify_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(SvArgs), ctypes.c_void_p]
    lib.spec_verify_run.restype = ctypes.c_int
    lib.spec_verify_destroy.argtypes = [ctypes.c_void_p]
    lib.spec_verify_destroy.restype = ctypes.c_int
    lib.spec_verify_validate.argtypes = [ctypes.POINTER(SvConfig), ctypes.POINTER(SvArgs)]
    lib.spec_verify_validate.restype = ctypes.c_int
    lib.spec_verify_workspace_bytes.argtypes = [ctypes.POINTER(SvConfig)]
    lib.spec_verify_workspace_bytes.restype = ctypes.c_uint64
    lib.spec_verify_profile_begin.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.spec_verify_profile_begin.restype = ctypes.c_int
    lib.spec_verify_profile_end.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    lib.spec_verify_profile_end.restype = ctypes.c_int
    lib.spec_verify_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.spec_verify_stream_probe.restype = ctypes.c_int
    lib.spec_verify_stream_probe_sweep.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.spec_verify_stream_probe_sweep.restype = ctypes.c_int
    lib.spec_verify_philox_words.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.spec_verify_philox_words.restype = ctypes.c_int
    lib.spec_verify_run_static.argtypes = [ctypes.POINTER(SvConfig), ctypes.POINTER(SvArgs), ctypes.c_void_p]
    lib.spec_verify_run_static.restype = ctypes.c_int
    lib.spec_verify_last_error.argtypes = []
    lib.spec_verify_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = load_library().spec_verify_last_error().decode()
        super().__init__(f"{where} returned {code}: {msg}")
        self.code = code


_DTYPES = {torch.bfloat16: SV_BF16, torch.float32: SV_F32}


def _ptr(t: Optional[torch.Tensor], dtype=None, n=None, name=""):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {t.numel()}")
    return t.data_ptr()


def spec_verify_last_error() -> str:
    return load_library().spec_verify_last_error().decode()


def make_config(max_batch: int, max_k: int, vocab: int, dtype, device: int = 0) -> SvConfig:
    code = dtype if isinstance(dtype, int) else _DTYPES[dtype]
    return SvConfig(max_batch, max_k, vocab, code, device)


def spec_verify_workspace_bytes(max_batch: int, max_k: int, vocab: int, dtype, device: int = 0) -> int:
    cfg = make_config(max_batch, max_k, vocab, dtype, device)
    return int(load_library().spec_verify_workspace_bytes(ctypes.byref(cfg)))


def spec_verify_create(max_batch: int, max_k: int, vocab: int, dtype, device: int = 0) -> int:
    """Returns the handle (an integer address)."""
    cfg = make_config(max_batch, max_k, vocab, dtype, device)
    h = ctypes.c_void_p()
    rc = load_library().spec_verify_create(ctypes.byref(h), ctypes.byref(cfg))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_create")
    return h.value


def spec_verify_destroy(handle: int) -> None:
    rc = load_library().spec_verify_destroy(ctypes.c_void_p(handle))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_destroy")


def make_args(target: torch.Tensor, draft: Optional[torch.Tensor], draft_tokens: Optional[torch.Tensor],
              *, accepted: torch.Tensor, out_tokens: torch.Tensor,
              row_status: Optional[torch.Tensor] = None, diag: Optional[torch.Tensor] = None,
              k_per_row=None, mode=None, temperature=None, top_k=None, top_p=None,
              default_mode: int = SV_PLAIN, default_temperature: float = 1.0,
              default_top_k: int = 1, default_top_p: float = 1.0,
              seed: int = 0, row_offset: int = 0) -> SvArgs:
    if target.dim() != 3:
        raise ValueError("target must be [B][K_max+1][V]")
    B, K1, V = target.shape
    K = K1 - 1
    if K > 0:
        # greedy verification needs only the target's argmax: the draft's
        # logits may be left out when every sequence is greedy
        greedy_only = mode is None and default_mode == SV_GREEDY
        if draft is None and not greedy_only:
            raise ValueError("draft is required unless every sequence is greedy")
        if draft is not None and (tuple(draft.shape) != (B, K, V) or draft.dtype != target.dtype):
            raise ValueError("draft must be [B][K_max][V] with the target's dtype")
        if draft_tokens is None or tuple(draft_tokens.shape) != (B, K):
            raise ValueError("draft_tokens must be [B][K_max]")
    if target.dtype not in _DTYPES:
        raise TypeError("logits must be bfloat16 or float32")
    return SvArgs(
        B, K,
        _ptr(target, name="target"),
        _ptr(draft, name="draft") if K > 0 and draft is not None else None,
        _ptr(draft_tokens, torch.int32, B * K, "draft_tokens") if K > 0 else None,
        _ptr(k_per_row, torch.int32, B, "k_per_row"),
        _ptr(mode, torch.uint8, B, "mode"),
        _ptr(temperature, torch.float32, B, "temperature"),
        _ptr(top_k, torch.int32, B, "top_k"),
        _ptr(top_p, torch.float32, B, "top_p"),
        default_mode, default_temperature, default_top_k, default_top_p,
        seed, row_offset,
        _ptr(accepted, torch.int32, B, "accepted"),
        _ptr(out_tokens, torch.int32, B * (K + 1), "out_tokens"),
        _ptr(row_status, torch.int32, B, "row_status"),  # uint32 bit patterns
        _ptr(diag, torch.float32, B * K * 2, "diag"),
    )


def spec_verify_validate(max_batch: int, max_k: int, vocab: int, dtype, args: SvArgs, device: int = 0) -> int:
    cfg = make_config(max_batch, max_k, vocab, dtype, device)
    return int(load_library().spec_verify_validate(ctypes.byref(cfg), ctypes.byref(args)))


def spec_verify_run(handle: int, args: SvArgs, stream=None) -> None:
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    rc = load_library().spec_verify_run(ctypes.c_void_p(handle), ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_run")


def spec_verify_run_static(vocab: int, dtype, args: SvArgs, device: int = 0, stream=None) -> None:
    """The step without a handle and without any allocation: the workspace is
    the library's static device buffer (SV_STATIC_SCRATCH_BYTES per device).
    Calls that overlap on one device race; order them on one stream."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    elif isinstance(stream, torch.cuda.Stream):
        stream = stream.cuda_stream
    cfg = make_config(max(1, args.B), args.K_max, vocab, dtype, device)
    rc = load_library().spec_verify_run_static(ctypes.byref(cfg), ctypes.byref(args), ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_run_static")


def spec_verify_profile_begin(handle: int, max_calls: int) -> None:
    rc = load_library().spec_verify_profile_begin(ctypes.c_void_p(handle), max_calls)
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_profile_begin")


def spec_verify_profile_end(handle: int):
    """Returns (calls recorded, [stage-0 ms summed, stage-1 ms summed])."""
    ms = (ctypes.c_double * 2)()
    rc = load_library().spec_verify_profile_end(ctypes.c_void_p(handle), ms, 2)
    if rc < 0:
        raise SpecVerifyError(rc, "spec_verify_profile_end")
    return rc, [ms[0], ms[1]]


def spec_verify_stream_probe(data_ptr: int, nbytes: int, out_ptr: int, stream: int = 0) -> None:
    """Reads nbytes // 8192 whole 8 KB blocks at data_ptr once (a
    measurement of the streaming ceiling; see the header)."""
    rc = load_library().spec_verify_stream_probe(ctypes.c_void_p(data_ptr), nbytes, ctypes.c_void_p(out_ptr),
                                                 ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_stream_probe")


def spec_verify_philox_words(seed: int, g_ptr: int, t_ptr: int, purpose_ptr: int, n: int, out_ptr: int,
                             stream: int = 0) -> None:
    """Word 0 of the device Philox4x32-10 for n counters (device arrays;
    see the header)."""
    rc = load_library().spec_verify_philox_words(seed, ctypes.c_void_p(g_ptr), ctypes.c_void_p(t_ptr),
                                                 ctypes.c_void_p(purpose_ptr), n, ctypes.c_void_p(out_ptr),
                                                 ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_philox_words")


def spec_verify_stream_probe_sweep(data_ptr: int, nbytes: int, loads_per_lane: int, waves_per_cu: int,
                                   out_ptr: int, stream: int = 0) -> None:
    """One point of the read-rate sweep: whole blocks of 64 x loads_per_lane
    16-byte vectors at data_ptr read once by a persistent grid of
    waves_per_cu waves per compute unit (see the header)."""
    rc = load_library().spec_verify_stream_probe_sweep(ctypes.c_void_p(data_ptr), nbytes, loads_per_lane,
                                                       waves_per_cu, ctypes.c_void_p(out_ptr),
                                                       ctypes.c_void_p(stream))
    if rc != SV_OK:
        raise SpecVerifyError(rc, "spec_verify_stream_probe_sweep")


class Verifier:
    """A handle plus output allocation, for callers that want tensors back."""

    def __init__(self, max_batch: int, max_k: int, vocab: int, dtype=torch.bfloat16, device: int = 0):
        if isinstance(dtype, int):
            dtype = {SV_BF16: torch.bfloat16, SV_F32: torch.float32}[dtype]
        self.max_batch, self.max_k, self.vocab, self.dtype = max_batch, max_k, vocab, dtype
        self.device = device
        self.handle = spec_verify_create(max_batch, max_k, vocab, dtype, device)

    def outputs(self, B: int, K: int):
        dev = torch.device("cuda", self.device)
        return (torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(B, K + 1, dtype=torch.int32, device=dev),
                torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(B, K, 2, dtype=torch.float32, device=dev))

    def _check_logits(self, name: str, t: Optional[torch.Tensor]) -> None:
        """The kernels take V, the dtype and the device from the handle and
        use V as the row stride, so a tensor that disagrees would be read
        out of bounds or misread: refuse it before anything is launched."""
        if t is None:
            return
        if t.shape[-1] != self.vocab:
            raise ValueError(f"{name} has V = {t.shape[-1]}, the handle was created for V = {self.vocab}")
        if t.dtype != self.dtype:
            raise TypeError(f"{name} is {t.dtype}, the handle was created for {self.dtype}")
        if not t.is_cuda or (t.device.index or 0) != self.device:
            raise ValueError(f"{name} is on {t.device}, the handle is on cuda:{self.device}")

    def __call__(self, target, draft, draft_tokens, *, out=None, stream=None, **kw):
        self._check_logits("target", target)
        self._check_logits("draft", draft)
        B, K1, _ = target.shape
        acc, toks, st, diag = out if out is not None else self.outputs(B, K1 - 1)
        args = make_args(target, draft, draft_tokens, accepted=acc, out_tokens=toks,
                         row_status=st, diag=diag, **kw)
        spec_verify_run(self.handle, args, stream)
        return acc, toks, st, diag

    def sample(self, rows: torch.Tensor, *, seed: int, row_offset: int = 0, mode=None,
               temperature=None, top_k=None, top_p=None, default_mode=SV_PLAIN,
               default_temperature=1.0, default_top_k=1, default_top_p=1.0, stream=None):
        """One draw per logit row from its filtered distribution: the step
        with K = 0 (a bonus draw), row r using counter (row_offset + r, 0,
        BONUS)."""
        self._check_logits("rows", rows)
        V = rows.shape[-1]
        flat = rows.reshape(-1, 1, V)
        n = flat.shape[0]
        dev = rows.device
        acc = torch.empty(n, dtype=torch.int32, device=dev)
        toks = torch.empty(n, 1, dtype=torch.int32, device=dev)
        st = torch.empty(n, dtype=torch.int32, device=dev)
        args = make_args(flat, None, None, accepted=acc, out_tokens=toks, row_status=st,
                         mode=mode, temperature=temperature, top_k=top_k, top_p=top_p,
                         default_mode=default_mode, default_temperature=default_temperature,
                         default_top_k=default_top_k, default_top_p=default_top_p,
                         seed=seed, row_offset=row_offset)
        spec_verify_run(self.handle, args, stream)
        return toks.reshape(rows.shape[:-1]), st

    def close(self):
        if self.handle:
            spec_verify_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

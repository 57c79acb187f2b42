"""Reference oracle for speculative sampling's verify-and-resample step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  It is the
plain single-threaded fp64 C++ implementation in ``oracle.cpp`` (see that
file's header for the passages of the pages it follows and the readings it
takes where they are silent), loaded through ctypes.  It shares no code with
the GPU library and imports nothing from it.

Logit arrays are numpy arrays: ``float32`` for fp32 logits, ``uint16`` holding
bfloat16 bit patterns for bf16 logits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
PLAIN, TOPK, TOPP, GREEDY = 0, 1, 2, 3
PURPOSE_ACCEPT, PURPOSE_RESAMPLE, PURPOSE_BONUS = 0, 1, 2

ST_TOKEN = 1 << 0
ST_NONFINITE = 1 << 1
ST_EMPTY = 1 << 2
ST_ZERO_RESIDUAL = 1 << 3
ST_PZERO = 1 << 4
ST_PARAM = 1 << 6
ST_ERRORS = ST_TOKEN | ST_NONFINITE | ST_EMPTY | ST_PARAM

FL_ACCEPT, FL_CDF, FL_TOPP = 1, 2, 4


def compile_oracle(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with g++ (single-threaded, -O2, no fast-math)."""
    cmd = ["g++", "-std=c++17", "-O2", "-Wall", "-shared", "-fPIC", src, "-o", out]
    subprocess.run(cmd, check=True, cwd=os.path.dirname(src))
    return out


class _Args(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K_max", ctypes.c_int32), ("V", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("target_logits", ctypes.c_void_p), ("draft_logits", ctypes.c_void_p),
        ("draft_tokens", ctypes.c_void_p), ("k_per_row", ctypes.c_void_p),
        ("mode", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
        ("top_k", ctypes.c_void_p), ("top_p", ctypes.c_void_p),
        ("default_mode", ctypes.c_int32), ("default_temperature", ctypes.c_float),
        ("default_top_k", ctypes.c_int32), ("default_top_p", ctypes.c_float),
        ("seed", ctypes.c_uint64), ("row_offset", ctypes.c_uint64),
        ("accepted", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
        ("row_status", ctypes.c_void_p), ("diag", ctypes.c_void_p),
        ("flags", ctypes.c_void_p), ("resid_mass", ctypes.c_void_p),
    ]


_lib = None


def load(path: str = _LIB):
    """Load (compiling first if absent) and return the oracle's ctypes handle."""
    global _lib
    if _lib is not None and path == _LIB:
        return _lib
    if not os.path.exists(path):
        compile_oracle(out=path)
    lib = ctypes.CDLL(path)
    lib.oracle_philox4x32_10.argtypes = [ctypes.c_void_p] * 3
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_philox_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_philox_words.restype = None
    lib.oracle_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
    lib.oracle_uniform.restype = ctypes.c_double
    lib.oracle_row_probs.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_float, ctypes.c_int, ctypes.c_float,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_row_probs.restype = ctypes.c_uint32
    lib.oracle_verify.argtypes = [ctypes.POINTER(_Args)]
    lib.oracle_verify.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {x.dtype}")


def philox(ctr, key, lib=None):
    """Philox4x32-10 of one 4-word counter under a 2-word key."""
    lib = lib or load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib.oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def philox_words(seed: int, g, t, purpose, lib=None) -> np.ndarray:
    """First output word of Philox at counters (g lo, t, purpose, g hi), key = seed."""
    lib = lib or load()
    g = np.ascontiguousarray(g, dtype=np.uint64)
    t = np.ascontiguousarray(np.broadcast_to(t, g.shape), dtype=np.uint32)
    p = np.ascontiguousarray(np.broadcast_to(purpose, g.shape), dtype=np.uint32)
    out = np.zeros(g.shape, np.uint32)
    lib.oracle_philox_words(seed, g.size, _ptr(g), _ptr(t), _ptr(p), _ptr(out))
    return out


def uniform(seed: int, g: int, t: int, purpose: int, lib=None) -> float:
    lib = lib or load()
    return lib.oracle_uniform(seed, g, t, purpose)


def row_probs(x: np.ndarray, mode: int, tau: float = 1.0, top_k: int = 1,
              top_p: float = 1.0, lib=None):
    """Adjusted distribution of one logit row: (pi, status, topp_margin, n_keep)."""
    lib = lib or load()
    x = np.ascontiguousarray(x)
    V = x.shape[-1]
    pi = np.zeros(V, np.float64)
    margin = ctypes.c_double()
    nk = ctypes.c_int()
    st = lib.oracle_row_probs(_ptr(x), _dtype_code(x), V, mode, tau, top_k, top_p,
                              _ptr(pi), ctypes.byref(margin), ctypes.byref(nk))
    return pi, int(st), margin.value, nk.value


def verify(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray, *,
           k_per_row=None, mode=None, temperature=None, top_k=None, top_p=None,
           default_mode: int = PLAIN, default_temperature: float = 1.0,
           default_top_k: int = 1, default_top_p: float = 1.0,
           seed: int = 0, row_offset: int = 0, lib=None) -> dict:
    """Run the oracle over B sequences.

    target [B][K_max+1][V], draft [B][K_max][V] (same dtype), tokens [B][K_max].
    Returns a dict of numpy arrays: accepted, out_tokens, row_status, diag,
    flags, resid_mass.
    """
    lib = lib or load()
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    KM = K1 - 1
    draft = np.ascontiguousarray(draft).reshape(B, KM, V)
    if draft.dtype != target.dtype:
        raise TypeError("target and draft must share a dtype")
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, KM)

    def opt(a, dt):
        return None if a is None else np.ascontiguousarray(a, dtype=dt).reshape(B)

    kpr = opt(k_per_row, np.int32)
    md = opt(mode, np.uint8)
    tmp = opt(temperature, np.float32)
    tk = opt(top_k, np.int32)
    tp = opt(top_p, np.float32)
    out = {
        "accepted": np.zeros(B, np.int32),
        "out_tokens": np.zeros((B, KM + 1), np.int32),
        "row_status": np.zeros(B, np.uint32),
        "diag": np.zeros((B, KM, 2), np.float64),
        "flags": np.zeros(B, np.uint32),
        "resid_mass": np.zeros(B, np.float64),
    }
    a = _Args(B, KM, V, _dtype_code(target), _ptr(target), _ptr(draft) if KM > 0 else None,
              _ptr(tokens) if KM > 0 else None,
              _ptr(kpr), _ptr(md), _ptr(tmp), _ptr(tk), _ptr(tp),
              default_mode, default_temperature, default_top_k, default_top_p,
              seed, row_offset,
              _ptr(out["accepted"]), _ptr(out["out_tokens"]), _ptr(out["row_status"]),
              _ptr(out["diag"]), _ptr(out["flags"]), _ptr(out["resid_mass"]))
    rc = lib.oracle_verify(ctypes.byref(a))
    if rc != 0:
        raise ValueError(f"oracle_verify rejected its arguments (rc={rc})")
    return out


def sample_rows(logits: np.ndarray, *, mode=None, temperature=None, top_k=None, top_p=None,
                default_mode: int = PLAIN, default_temperature: float = 1.0,
                default_top_k: int = 1, default_top_p: float = 1.0,
                seed: int = 0, row_offset: int = 0, lib=None) -> np.ndarray:
    """One draw per logit row from its adjusted distribution.

    This is the verify step with K = 0 (a bonus draw only), applied to rows
    viewed as independent sequences: row r uses counter (row_offset + r, 0,
    BONUS).  Used to draw draft tokens for test inputs.
    """
    x = np.ascontiguousarray(logits)
    V = x.shape[-1]
    rows = x.reshape(-1, 1, V)
    n = rows.shape[0]
    empty = np.zeros((n, 0, V), x.dtype)
    toks = np.zeros((n, 0), np.int32)
    res = verify(rows, empty, toks, mode=mode, temperature=temperature, top_k=top_k,
                 top_p=top_p, default_mode=default_mode,
                 default_temperature=default_temperature, default_top_k=default_top_k,
                 default_top_p=default_top_p, seed=seed, row_offset=row_offset, lib=lib)
    return res["out_tokens"][:, 0].reshape(x.shape[:-1])

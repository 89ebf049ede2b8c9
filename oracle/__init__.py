"""CPU oracle for exact attention (forward and gradients) — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg
may import anything here. The product path (the HIP library and its Python
binding) never imports, calls, links or loads this package, and this package
imports nothing from the product package.

Two independent CPU codes live here:

* ``attention_fwd`` / ``attention_rows`` — the definition written out in plain C,
  fp64, three passes over each stored score row (``attn_oracle.c``).
* ``attention_bwd`` — the gradients of that definition (chain rule through the
  softmax), in plain C fp64, independent of the forward code.
* ``tiled.online_softmax_attention`` — the tiled online-softmax recurrence in
  numpy fp64, in the order of the FA2 forward pseudocode, used to pin the blog's
  per-round intermediate figures and as a brute-force cross-check of the C code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle C source with gcc (-O2, OpenMP, no fast-math) into a shared library."""
    global _lib
    if not force and os.path.exists(out):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-Werror",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    if out == _LIB_PATH:
        _lib = None
    return out


def load_library(path: str):
    """Open an oracle shared library built by ``build`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_attn_fwd_f64.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                        ctypes.c_double, ctypes.c_int]
    lib.oracle_attn_fwd_f64.restype = ctypes.c_int
    lib.oracle_attn_rows_f64.argtypes = [dp, dp, dp, i64, i64, i64, i64, ctypes.c_double,
                                         ctypes.c_int, ctypes.POINTER(i64), i64, dp, dp]
    lib.oracle_attn_rows_f64.restype = ctypes.c_int
    lib.oracle_attn_bwd_f64.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, ctypes.c_double,
                                        ctypes.c_int]
    lib.oracle_attn_bwd_f64.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = load_library(_LIB_PATH)
    return _lib


def _as_f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shape3(q, k, v):
    if q.ndim < 2 or k.ndim < 2 or v.ndim < 2:
        raise ValueError("q, k, v need at least 2 dims [..., N, d]")
    lead = q.shape[:-2]
    if k.shape[:-2] != lead or v.shape[:-2] != lead:
        raise ValueError("q, k, v must share leading (batch, head) dims")
    nq, d = q.shape[-2:]
    nk = k.shape[-2]
    if k.shape[-1] != d or v.shape[-1] != d or v.shape[-2] != nk:
        raise ValueError("k must be [..., Nk, d] and v [..., Nk, d] with q's d")
    bh = int(np.prod(lead)) if lead else 1
    return lead, bh, nq, nk, d


ALIGNMENTS = {"top-left": 1, "bottom-right": 2}


def _causal_mode(causal, align: str) -> int:
    if not causal:
        return 0
    if align not in ALIGNMENTS:
        raise ValueError(f"align must be one of {sorted(ALIGNMENTS)}")
    return ALIGNMENTS[align]


def attention_fwd(q, k, v, scale: float, causal: bool = False, lib=None, align: str = "top-left"):
    """Exact attention forward in fp64 over every row.

    q: [..., Nq, d]; k, v: [..., Nk, d] (any float dtype, upcast losslessly to fp64).
    Returns (o [..., Nq, d] float64, lse [..., Nq] float64), LSE in natural log of the
    scaled scores. Causal masking is top-left aligned by default (key j valid iff
    j <= i); ``align="bottom-right"`` makes key j valid iff j <= i + Nk - Nq. A row
    with no valid key gets O = 0 and LSE = -inf.
    ``lib`` selects another build of the oracle source (default: liboracle.so).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    lead, bh, nq, nk, d = _shape3(q, k, v)
    o = np.empty(lead + (nq, d), dtype=np.float64)
    lse = np.empty(lead + (nq,), dtype=np.float64)
    rc = (lib or _load()).oracle_attn_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                              bh, nq, nk, d, float(scale), _causal_mode(causal, align))
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd_f64 failed with code {rc}")
    return o, lse


def attention_rows(q, k, v, scale: float, causal: bool, rows, lib=None, align: str = "top-left"):
    """Exact fp64 outputs for selected rows only (masking as in ``attention_fwd``).

    ``rows`` holds flat row indices bh*Nq + i. Returns (o [len(rows), d], lse [len(rows)]).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    _, bh, nq, nk, d = _shape3(q, k, v)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1))
    o = np.empty((rows.size, d), dtype=np.float64)
    lse = np.empty((rows.size,), dtype=np.float64)
    rc = (lib or _load()).oracle_attn_rows_f64(
        _ptr(q), _ptr(k), _ptr(v), bh, nq, nk, d, float(scale), _causal_mode(causal, align),
        rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows_f64 failed with code {rc}")
    return o, lse


def attention_bwd(q, k, v, dout, scale: float, causal: bool = False, lib=None, align: str = "top-left"):
    """Exact gradients (dq, dk, dv) in fp64 of a loss L with dL/dO = ``dout`` for the
    forward of ``attention_fwd`` (same shapes, masking and alignment): the forward
    definition differentiated, with P recomputed from the scores (``attn_oracle.c``).
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    lead, bh, nq, nk, d = _shape3(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must be shaped like q")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = (lib or _load()).oracle_attn_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                              bh, nq, nk, d, float(scale), _causal_mode(causal, align))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd_f64 failed with code {rc}")
    return dq, dk, dv


def num_threads() -> int:
    """Threads the oracle's OpenMP regions use (OMP_NUM_THREADS or all host cores)."""
    return int(_load().oracle_num_threads())

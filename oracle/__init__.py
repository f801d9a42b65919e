"""Plain fp64 CPU oracle for the gated delta rule.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s CPU-baseline leg may import anything from this package.  It
shares no code with the HIP path (no kernels, headers, helpers or tables), and
the product package never imports it.

Three independent formulations live here:

* ``recurrent_fwd`` / ``recurrent_step`` -- the definition, token by token, in
  plain C (``gdn_oracle.c``, fp64 / complex128, OpenMP over chains).
* ``chunked.chunked_fwd`` -- the chunkwise WY/UT form in NumPy fp64, exposing
  the per-chunk intermediates (gate cumsum, A, T, W, U, P).
* ``bruteforce.bruteforce_fwd`` -- explicit dense transition products for short
  sequences.

The C library is compiled with gcc on first use (or by ``build()``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def compile_library(src: str, out: str) -> None:
    """Compile an oracle C source into a shared library with gcc (fp64, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-shared", "-fPIC", src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)


def build(force: bool = True) -> str:
    """Build ``liboracle.so`` next to the source.  Returns its path."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        compile_library(_SRC, tmp)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    dp = ctypes.POINTER(ctypes.c_double)
    for name in ("gdn_ref_fwd_f64", "gdn_ref_fwd_c128"):
        f = getattr(lib, name)
        f.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp] + [ctypes.c_int] * 6
        f.restype = ctypes.c_int
    for name in ("gdn_ref_step_f64", "gdn_ref_step_c128"):
        f = getattr(lib, name)
        f.argtypes = [dp] * 7 + [ctypes.c_int] * 4
        f.restype = ctypes.c_int
    return lib


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the compiled oracle (building it if missing or stale).  ``path`` loads another build."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _prep(x, cplx: bool) -> np.ndarray:
    dt = np.complex128 if cplx else np.float64
    return np.ascontiguousarray(np.asarray(x), dtype=dt)


def recurrent_fwd(q, k, v, alpha, beta, S0=None, threads: int = 0, lib: ctypes.CDLL | None = None):
    """Token-by-token forward of the gated delta rule.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; alpha, beta: [B, T, H]; S0: [B, H, dk, dv] or None.
    Real or complex inputs (complex if any of q, k, v, S0 is complex).  Returns
    (o [B, T, H, dv], S_final [B, H, dk, dv], threads_used) in fp64 / complex128.
    """
    cplx = any(np.iscomplexobj(x) for x in (q, k, v) + ((S0,) if S0 is not None else ()))
    q, k, v = _prep(q, cplx), _prep(k, cplx), _prep(v, cplx)
    alpha = np.ascontiguousarray(alpha, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk) and v.shape == (B, T, H, dv)
    assert alpha.shape == (B, T, H) and beta.shape == (B, T, H)
    if S0 is not None:
        S0 = _prep(S0, cplx)
        assert S0.shape == (B, H, dk, dv)
    dt = np.complex128 if cplx else np.float64
    o = np.empty((B, T, H, dv), dtype=dt)
    S = np.empty((B, H, dk, dv), dtype=dt)
    lib = lib or load_library()
    fn = lib.gdn_ref_fwd_c128 if cplx else lib.gdn_ref_fwd_f64
    used = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S0), _ptr(o), _ptr(S),
              B, T, H, dk, dv, int(threads))
    return o, S, used


def recurrent_step(q, k, v, alpha, beta, S, threads: int = 0, lib: ctypes.CDLL | None = None):
    """One decode step on N independent states.

    q, k: [N, dk]; v: [N, dv]; alpha, beta: [N]; S: [N, dk, dv].
    Returns (o [N, dv], S_new [N, dk, dv]); the input S is not modified.
    """
    cplx = any(np.iscomplexobj(x) for x in (q, k, v, S))
    q, k, v = _prep(q, cplx), _prep(k, cplx), _prep(v, cplx)
    S = _prep(S, cplx).copy()
    alpha = np.ascontiguousarray(alpha, dtype=np.float64)
    beta = np.ascontiguousarray(beta, dtype=np.float64)
    N, dk = q.shape
    dv = v.shape[-1]
    assert S.shape == (N, dk, dv)
    o = np.empty((N, dv), dtype=S.dtype)
    lib = lib or load_library()
    fn = lib.gdn_ref_step_c128 if cplx else lib.gdn_ref_step_f64
    fn(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(S), _ptr(o), N, dk, dv, int(threads))
    return o, S

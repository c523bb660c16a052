"""fp64 CPU oracle for PaTH attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline`` leg
may import this package.  The product path (the HIP library and its Python
binding) never does, and shares no code with it.

The arithmetic lives in ``path_oracle.c`` (plain C, fp64, pthreads); this module
builds it with gcc and exposes numpy-friendly wrappers.  Inputs are widened to
float64 here; they are the exact values the GPU consumes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "path_oracle.c")
# PATHORACLE_LIB points the loader at another build of the same source (the sanitizer run builds one)
_LIB = os.environ.get("PATHORACLE_LIB") or os.path.join(_HERE, "libpathoracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile path_oracle.c with gcc (no fast-math) into oracle/libpathoracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
                        "-fno-fast-math", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        L.path_oracle_fwd.argtypes = [_D, _D, _D, _D, _D, _D, _I64, _I64, _I64, ctypes.c_double,
                                      ctypes.POINTER(_I64), _I64, _D, _D, ctypes.c_int]
        L.path_oracle_row_logits.argtypes = [_D, _D, _D, _D, _D, _I64, _I64, ctypes.c_double, _D]
        L.path_oracle_transport.argtypes = [_D, _D, _D, _I64, _I64, _I64, _D]
        L.path_oracle_decode.argtypes = [_D, _D, _D, _I64, _I64, _I64, _I64, _D, _D, _D, _D, _D, _D, _I64,
                                         ctypes.c_double, _D, _D, ctypes.c_int]
        L.path_oracle_cache_bias.argtypes = [_D, _I64, _D]
        L.path_oracle_ut_tinv.argtypes = [_D, _D, _I64, _I64, _D]
        L.path_oracle_householder_product.argtypes = [_D, _D, _I64, _I64, _D]
        L.path_oracle_chunk_terms.argtypes = [_D, _D, _D, _D, _I64, _I64, _D, _D, _D]
        L.path_oracle_cache_keys.argtypes = [_D, _D, _D, _I64, _I64, _I64, _I64, _D]
        L.path_oracle_bwd.argtypes = [_D, _D, _D, _D, _D, _D, _D, _I64, _I64, _I64, ctypes.c_double,
                                      _D, _D, _D, _D, _D, _D, ctypes.c_int]
        for f in ("path_oracle_fwd", "path_oracle_row_logits", "path_oracle_transport",
                  "path_oracle_decode", "path_oracle_ut_tinv", "path_oracle_householder_product",
                  "path_oracle_chunk_terms", "path_oracle_cache_keys", "path_oracle_cache_bias",
                  "path_oracle_bwd"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_D)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def host_threads() -> int:
    """Threads the oracle may use: the CPUs this process is allowed to run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def fwd(q, k, v, w, beta, logf=None, scale: float = 1.0, rows: Optional[Sequence[int]] = None,
        nthreads: int = 0):
    """PaTH / PaTH-FoX forward.  q,k,v,w: [..., L, d]; beta, logf: [..., L].

    Returns (out [..., R, d], lse [..., R]) in float64 where R = L, or len(rows).
    """
    q, k, v, w, beta = map(_f64, (q, k, v, w, beta))
    logf = None if logf is None else _f64(logf)
    lead = q.shape[:-2]
    L, d = q.shape[-2], q.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = L if rows_arr is None else len(rows_arr)
    out = np.zeros(lead + (R, d))
    lse = np.zeros(lead + (R,))
    rc = lib().path_oracle_fwd(_p(q), _p(k), _p(v), _p(w), _p(beta), _p(logf), BH, L, d, float(scale),
                               None if rows_arr is None else rows_arr.ctypes.data_as(ctypes.POINTER(_I64)),
                               R, _p(out), _p(lse), int(nthreads or host_threads()))
    _check(rc, "path_oracle_fwd")
    return out, lse


def row_logits(q_i, K, W, beta, i: int, logf=None, scale: float = 1.0):
    """Logits z[0..i] of query row i for one (batch, head) slice."""
    q_i, K, W, beta = map(_f64, (q_i, K, W, beta))
    logf = None if logf is None else _f64(logf)
    z = np.zeros(i + 1)
    _check(lib().path_oracle_row_logits(_p(q_i), _p(K), _p(W), _p(beta), _p(logf), i, q_i.shape[-1],
                                        float(scale), _p(z)), "path_oracle_row_logits")
    return z


def transport(x, W, beta, lo: int, hi: int):
    """H_lo H_{lo+1} ... H_hi x (identity when hi < lo)."""
    x, W, beta = map(_f64, (x, W, beta))
    out = np.zeros_like(x)
    _check(lib().path_oracle_transport(_p(x), _p(W), _p(beta), lo, hi, x.shape[-1], _p(out)),
           "path_oracle_transport")
    return out


def decode(kcache, vcache, t0: int, q, k, v, w, beta, scale: float, nthreads: int = 0, fcache=None, logf=None):
    """Run nsteps decode steps.  kcache/vcache: [BH, cap, d] float64, modified in place.

    q,k,v,w: [nsteps, BH, d]; beta: [nsteps, BH].  PaTH-FoX: fcache [BH, cap] float64 per-slot forget
    bias (modified in place) and logf [nsteps, BH].  Returns (out [nsteps,BH,d], lse [nsteps,BH]).
    """
    assert kcache.dtype == np.float64 and kcache.flags.c_contiguous
    assert vcache.dtype == np.float64 and vcache.flags.c_contiguous
    assert (fcache is None) == (logf is None)
    if fcache is not None:
        assert fcache.dtype == np.float64 and fcache.flags.c_contiguous
        logf = _f64(logf)
    q, k, v, w, beta = map(_f64, (q, k, v, w, beta))
    nsteps, BH, d = q.shape
    cap = kcache.shape[1]
    out = np.zeros((nsteps, BH, d))
    lse = np.zeros((nsteps, BH))
    _check(lib().path_oracle_decode(_p(kcache), _p(vcache), _p(fcache), BH, cap, t0, nsteps, _p(q), _p(k),
                                    _p(v), _p(w), _p(beta), _p(logf), d, float(scale), _p(out), _p(lse),
                                    int(nthreads or host_threads())), "path_oracle_decode")
    return out, lse


def ut_tinv(W, beta):
    """T^{-1} (n x n) of the compact form H_0...H_{n-1} = I - W^T T^{-1} W."""
    W, beta = map(_f64, (W, beta))
    n, d = W.shape
    out = np.zeros((n, n))
    _check(lib().path_oracle_ut_tinv(_p(W), _p(beta), n, d, _p(out)), "path_oracle_ut_tinv")
    return out


def householder_product(W, beta):
    """Explicit d x d product H_0 H_1 ... H_{n-1}."""
    W, beta = map(_f64, (W, beta))
    n, d = W.shape
    out = np.zeros((d, d))
    _check(lib().path_oracle_householder_product(_p(W), _p(beta), n, d, _p(out)),
           "path_oracle_householder_product")
    return out


def chunk_terms(q, k, W, beta):
    """(qtilde, ktilde, sintra) of one chunk by definition (see path_oracle.c)."""
    q, k, W, beta = map(_f64, (q, k, W, beta))
    n, d = q.shape
    qt, kt, s = np.zeros((n, d)), np.zeros((n, d)), np.zeros((n, n))
    _check(lib().path_oracle_chunk_terms(_p(q), _p(k), _p(W), _p(beta), n, d, _p(qt), _p(kt), _p(s)),
           "path_oracle_chunk_terms")
    return qt, kt, s


def cache_keys(K, W, beta, rows=None):
    """Key cache slots after a prompt of L tokens: slot j = H_{L-1} ... H_{j+1} k_j.

    K, W: [L, d]; beta: [L] (one batch/head).  rows: optional (j0, j1) range; default all.
    Returns [(j1 - j0), d] float64.
    """
    K, W, beta = map(_f64, (K, W, beta))
    L, d = K.shape
    j0, j1 = (0, L) if rows is None else rows
    out = np.zeros((max(j1 - j0, 0), d))
    _check(lib().path_oracle_cache_keys(_p(K), _p(W), _p(beta), L, d, j0, j1, _p(out)),
           "path_oracle_cache_keys")
    return out


def cache_bias(logf):
    """PaTH-FoX forget bias of each cache slot after a prompt: slot j = sum_{s=j+1..L-1} f_s.  logf: [L]."""
    logf = _f64(logf)
    out = np.zeros(logf.shape[0])
    _check(lib().path_oracle_cache_bias(_p(logf), logf.shape[0], _p(out)), "path_oracle_cache_bias")
    return out


def bwd(q, k, v, w, beta, dout, logf=None, scale: float = 1.0, nthreads: int = 0):
    """Gradients of the forward for the loss sum(dout * out).  Shapes as in fwd, dout like q.

    Returns (dq, dk, dv, dw, dbeta, dlogf) in float64; dlogf is None without logf.
    """
    q, k, v, w, beta, dout = map(_f64, (q, k, v, w, beta, dout))
    logf = None if logf is None else _f64(logf)
    lead = q.shape[:-2]
    L, d = q.shape[-2], q.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    dq, dk, dv, dw = (np.zeros(lead + (L, d)) for _ in range(4))
    dbeta = np.zeros(lead + (L,))
    dlogf = None if logf is None else np.zeros(lead + (L,))
    _check(lib().path_oracle_bwd(_p(q), _p(k), _p(v), _p(w), _p(beta), _p(logf), _p(dout), BH, L, d,
                                 float(scale), _p(dq), _p(dk), _p(dv), _p(dw), _p(dbeta), _p(dlogf),
                                 int(nthreads or host_threads())), "path_oracle_bwd")
    return dq, dk, dv, dw, dbeta, dlogf

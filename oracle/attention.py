"""ctypes front of the fp64 oracle core (``attention.c``).

TEST INFRASTRUCTURE: see the package docstring for who may call this.

``attention_rows`` evaluates, for each query row ``i``, softmax attention
over keys ``0 .. kend[i]-1`` (definition in ``attention.c``; "Megatron-LM
篇" §3.1-§3.3).  ``causal_attention`` is the full causal case
``kend[i] = i + 1`` - the non-CP result that every rank's merged output
must reproduce ("Megatron-LM 篇" §3.2, last paragraph).
"""
import ctypes
import math

import numpy as np

from .build import ensure_built

_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(ensure_built())
        f = lib.oracle_attention
        P = ctypes.POINTER(ctypes.c_double)
        I64 = ctypes.c_int64
        f.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_double,
                      ctypes.POINTER(ctypes.c_int64), P, P, ctypes.c_int]
        f.restype = ctypes.c_int
        fb = lib.oracle_attention_bwd
        fb.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_double,
                       ctypes.POINTER(ctypes.c_int64), P, P, P, ctypes.c_int]
        fb.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def attention_rows(q, k, v, kend, scale=None, nthreads=0):
    """Softmax attention of each query row over its visible key prefix.

    q: [b, nq, hq, d]; k, v: [b, nk, hkv, d]; kend: [nq] visible key count.
    Returns (O [b, nq, hq, d], L [b, hq, nq]) in fp64; L is natural-log.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, nq, hq, d = q.shape
    bk, nk, hkv, dk = k.shape
    if v.shape != k.shape or bk != b or dk != d:
        raise ValueError("q/k/v shapes disagree")
    kend = np.ascontiguousarray(kend, dtype=np.int64)
    if kend.shape != (nq,):
        raise ValueError("kend must have one entry per query row")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.empty((b, nq, hq, d), np.float64)
    lse = np.empty((b, hq, nq), np.float64)
    P = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_attention(
        q.ctypes.data_as(P), k.ctypes.data_as(P), v.ctypes.data_as(P),
        b, nq, nk, hq, hkv, d, float(scale),
        kend.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        o.ctypes.data_as(P), lse.ctypes.data_as(P), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return o, lse


def causal_attention(q, k, v, scale=None, nthreads=0):
    """Full causal attention (diagonal included): row i sees keys 0..i."""
    nq = np.shape(q)[1]
    if np.shape(k)[1] != nq:
        raise ValueError("causal attention needs as many keys as queries")
    return attention_rows(q, k, v, np.arange(1, nq + 1), scale, nthreads)


def attention_rows_bwd(q, k, v, dout, kend, scale=None, nthreads=0):
    """Gradients (dQ, dK, dV) of softmax attention over visible key prefixes.

    The derivative of ``attention_rows`` for a loss whose gradient with
    respect to O is ``dout`` (C core ``oracle_attention_bwd``).  q, dout:
    [b, nq, hq, d]; k, v: [b, nk, hkv, d]; kend: [nq].  dK and dV of a KV
    head sum the contributions of every query head of its group.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    b, nq, hq, d = q.shape
    bk, nk, hkv, dk_ = k.shape
    if v.shape != k.shape or dout.shape != q.shape or bk != b or dk_ != d:
        raise ValueError("q/k/v/dout shapes disagree")
    kend = np.ascontiguousarray(kend, dtype=np.int64)
    if kend.shape != (nq,):
        raise ValueError("kend must have one entry per query row")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    P = ctypes.POINTER(ctypes.c_double)
    rc = _load().oracle_attention_bwd(
        q.ctypes.data_as(P), k.ctypes.data_as(P), v.ctypes.data_as(P), dout.ctypes.data_as(P),
        b, nq, nk, hq, hkv, d, float(scale),
        kend.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        dq.ctypes.data_as(P), dk.ctypes.data_as(P), dv.ctypes.data_as(P), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention_bwd rejected its arguments")
    return dq, dk, dv


def causal_attention_bwd(q, k, v, dout, scale=None, nthreads=0):
    """Gradients of full causal attention (row i sees keys 0..i)."""
    nq = np.shape(q)[1]
    if np.shape(k)[1] != nq:
        raise ValueError("causal attention needs as many keys as queries")
    return attention_rows_bwd(q, k, v, dout, np.arange(1, nq + 1), scale, nthreads)

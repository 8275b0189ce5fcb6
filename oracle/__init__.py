"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding)
never imports, loads or calls anything here, and nothing here imports the
product path.

Two independent implementations live here:

* ``liboracle.so`` (``attn_oracle.c``, plain C, fp64, OpenMP): the
  definition of attention with a three-pass safe softmax per row, its
  chain-rule gradient, both optionally with dropout on the probabilities
  (mask from Philox4x32-10), and the pages' online (chunked) softmax and
  tiled forward in fp64.  Wrapped by :func:`fwd`, :func:`bwd`,
  :func:`dropout_keep`, :func:`philox4x32_10`, :func:`online_softmax`,
  :func:`fwd_online`.
* :mod:`oracle.brute` (NumPy, fp64): standard attention with the N x N score
  and probability matrices materialised, for tiny inputs.
* :mod:`oracle.fp8` (NumPy): decoding of E4M3 inputs from the format's
  definition, the FP8 forward's definition (the C oracle on the decoded
  values) and the element-wise error bound of rounding P to E4M3.

Inputs are fp64 NumPy arrays; fp16/bf16 tensors are upcast exactly by the
caller (every fp16/bf16 value is representable in fp64).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build  # noqa: WPS433 (local build helper)
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_fwd.restype = ctypes.c_int
    lib.oracle_fwd.argtypes = [_dp, _dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_int64, ctypes.c_double, ctypes.c_int, _i64p,
                               ctypes.c_int64, ctypes.c_int]
    lib.oracle_bwd.restype = ctypes.c_int
    lib.oracle_bwd.argtypes = [_dp] * 10 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_double, ctypes.c_int, ctypes.c_int]
    lib.oracle_fwd_rect.restype = ctypes.c_int
    lib.oracle_fwd_rect.argtypes = [_dp] * 5 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_double, ctypes.c_int, _i64p,
                                                ctypes.c_int64, ctypes.c_int]
    lib.oracle_fwd_dropout.restype = ctypes.c_int
    lib.oracle_fwd_dropout.argtypes = [_dp] * 5 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.c_double, ctypes.c_int, ctypes.c_double,
                                                   ctypes.c_uint64, ctypes.c_uint32, _i64p,
                                                   ctypes.c_int64, ctypes.c_int]
    lib.oracle_bwd_dropout.restype = ctypes.c_int
    lib.oracle_bwd_dropout.argtypes = [_dp] * 10 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                    ctypes.c_double, ctypes.c_int, ctypes.c_double,
                                                    ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int]
    lib.oracle_dropout_keep.restype = ctypes.c_int
    lib.oracle_dropout_keep.argtypes = [ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_philox4x32_10.restype = ctypes.c_int
    lib.oracle_philox4x32_10.argtypes = [ctypes.c_void_p] * 3
    lib.oracle_online_softmax.restype = ctypes.c_int64
    lib.oracle_online_softmax.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, _dp, _dp]
    lib.oracle_fwd_online.restype = ctypes.c_int
    lib.oracle_fwd_online.argtypes = [_dp] * 5 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                                  ctypes.c_int, ctypes.c_int64]
    _lib = lib
    return lib


def _c(a):
    """Contiguous fp64 view of `a` (a NumPy array or a CPU torch tensor)."""
    if hasattr(a, "detach"):
        a = a.detach().cpu().double().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(_dp)


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def _dropout_args(dropout):
    p, seed, offset = dropout
    return float(p), int(seed) & (2**64 - 1), int(offset) & (2**32 - 1)


def fwd(q, k, v, scale, causal=False, rows=None, threads=None, dropout=None):
    """Forward definition.  q, k, v: [..., N, d] (leading dims flattened to BH).

    rows: optional 1-D int array of flattened row ids (bh * N + i); the result
    then holds only those rows, as (o [n_rows, d], lse [n_rows]).  Without
    rows the result has the input's leading shape: (o [..., N, d], lse [..., N]).
    dropout: optional (p, seed, offset): dropout on the probabilities with the
    mask of :func:`dropout_keep`.
    """
    lib = _load()
    q, k, v = _c(q), _c(k), _c(v)
    lead, N, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one shape")
    BH = int(np.prod(lead)) if lead else 1
    if rows is None:
        o = np.empty(q.shape, np.float64)
        lse = np.empty(q.shape[:-1], np.float64)
        rp, nr = None, BH * N
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nr = rows.size
        o = np.empty((nr, d), np.float64)
        lse = np.empty((nr,), np.float64)
        rp = rows.ctypes.data_as(_i64p)
    if dropout is None:
        rc = lib.oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), BH, N, d,
                            float(scale), int(bool(causal)), rp, nr,
                            int(threads or default_threads()))
    else:
        rc = lib.oracle_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), BH, N, d,
                                    float(scale), int(bool(causal)), *_dropout_args(dropout), rp, nr,
                                    int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_fwd failed")
    return o, lse


def fwd_rect(q, k, v, scale, causal=False, rows=None, threads=None):
    """Forward of Nq queries against Nk keys: q [..., Nq, d], k and v
    [..., Nk, d].  Under the causal mask query i sees keys 0 .. i + Nk - Nq
    (the queries are the last Nq positions); a row that sees no key gets
    o = 0 and lse = -inf.  rows as for :func:`fwd` (ids bh * Nq + i)."""
    lib = _load()
    q, k, v = _c(q), _c(k), _c(v)
    lead, Nq, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    Nk = k.shape[-2]
    if k.shape[:-2] != lead or k.shape[-1] != d or v.shape != k.shape:
        raise ValueError("k, v must be [..., Nk, d] with q's leading dims and d")
    BH = int(np.prod(lead)) if lead else 1
    if rows is None:
        o = np.empty(q.shape, np.float64)
        lse = np.empty(q.shape[:-1], np.float64)
        rp, nr = None, BH * Nq
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nr = rows.size
        o = np.empty((nr, d), np.float64)
        lse = np.empty((nr,), np.float64)
        rp = rows.ctypes.data_as(_i64p)
    rc = lib.oracle_fwd_rect(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), BH, Nq, Nk, d,
                             float(scale), int(bool(causal)), rp, nr,
                             int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_fwd_rect failed")
    return o, lse


def bwd(q, k, v, dO, scale, causal=False, threads=None, o_in=None, dropout=None):
    """Gradients of sum(O * dO).  Returns (o, lse, dq, dk, dv), all fp64.

    o_in: optional stored forward output; when given, D_i = dO_i . o_in_i
    (the library's backward contract) instead of sum_j P_ij dP_ij.
    dropout: optional (p, seed, offset), as for :func:`fwd`.
    """
    lib = _load()
    q, k, v, dO = _c(q), _c(k), _c(v), _c(dO)
    lead, N, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    for t in (k, v, dO):
        if t.shape != q.shape:
            raise ValueError("q, k, v, dO must share one shape")
    if o_in is not None:
        o_in = _c(o_in)
        if o_in.shape != q.shape:
            raise ValueError("o_in must have q's shape")
    BH = int(np.prod(lead)) if lead else 1
    o = np.empty(q.shape, np.float64)
    lse = np.empty(q.shape[:-1], np.float64)
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(q.shape, np.float64)
    dv = np.empty(q.shape, np.float64)
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(dO), _ptr(o_in) if o_in is not None else None,
            _ptr(o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv))
    nthr = int(threads or default_threads())
    if dropout is None:
        rc = lib.oracle_bwd(*ptrs, BH, N, d, float(scale), int(bool(causal)), nthr)
    else:
        rc = lib.oracle_bwd_dropout(*ptrs, BH, N, d, float(scale), int(bool(causal)),
                                    *_dropout_args(dropout), nthr)
    if rc != 0:
        raise RuntimeError("oracle_bwd failed")
    return o, lse, dq, dk, dv


def dropout_keep(p, seed, offset, bh, N):
    """Keep mask of head bh, [N, N] uint8 (1 kept), before any causal mask."""
    lib = _load()
    keep = np.empty((N, N), np.uint8)
    rc = lib.oracle_dropout_keep(float(p), int(seed) & (2**64 - 1), int(offset) & (2**32 - 1),
                                 int(bh), int(N), keep.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_dropout_keep failed")
    return keep


def philox4x32_10(ctr, key):
    """Philox4x32-10 of one counter (4 words) under one key (2 words)."""
    lib = _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    if c.size != 4 or k.size != 2 or lib.oracle_philox4x32_10(c.ctypes.data, k.ctypes.data,
                                                              out.ctypes.data) != 0:
        raise RuntimeError("oracle_philox4x32_10 failed")
    return out


def online_softmax(x, chunk):
    """Chunked one-pass softmax.  Returns (y, states[n_chunks, 3] = (m, l, factor))."""
    lib = _load()
    x = _c(x).reshape(-1)
    n = x.size
    nc = (n + chunk - 1) // chunk
    y = np.empty(n, np.float64)
    st = np.empty((max(nc, 1), 3), np.float64)
    got = lib.oracle_online_softmax(_ptr(x), n, int(chunk), _ptr(y), _ptr(st))
    if got < 0:
        raise RuntimeError("oracle_online_softmax failed")
    return y, st[:got]


def fwd_online(q, k, v, scale, causal=False, tile=4):
    """Tiled forward with online softmax for one head (q, k, v: [N, d])."""
    lib = _load()
    q, k, v = _c(q), _c(k), _c(v)
    N, d = q.shape
    o = np.empty((N, d), np.float64)
    lse = np.empty((N,), np.float64)
    rc = lib.oracle_fwd_online(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), N, d,
                               float(scale), int(bool(causal)), int(tile))
    if rc != 0:
        raise RuntimeError("oracle_fwd_online failed")
    return o, lse

"""Plain fp64 CPU oracle for sparse causal attention over a fixed neighbour graph.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  Nothing in
``sparse_causal_attention_amd`` imports this package, and this package imports
nothing from it.  The arithmetic lives in ``oracle.c`` (plain C, IEEE double,
OpenMP over independent rows); this module only marshals numpy arrays.

What it computes (sources cited per function in ``oracle.c``):

* the neighbour set N(i) = {i - delta : delta in {0..W-1} U offsets, i - delta >= 0}
  -- SpatialLM-Mini news page, section "How tokens choose whom to listen to",
  and the window predicate of the sliding-window mask listing, MiniGPT (Part 6),
  section "A mask is not enough";
* a softmax over N(i) only of either the scaled dot product or the coordinate
  distance score -gamma*||c_q - c_k||^2 + beta, and the weighted sum of values;
* the exact gradients of sum_i <dO_i, O_i> with respect to every input.

Every function here has a pin in ``tests/test_oracle.py``; none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16 = 0, 1, 2
SCORE_DOT, SCORE_COORD, SCORE_UNIFORM = 0, 1, 2

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra", "-Wno-unused-parameter",
             _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
        L.oracle_row.restype = i64
        L.oracle_row.argtypes = [i64, i64, vp, i32, i64, vp]
        L.oracle_graph_csr.restype = i64
        L.oracle_graph_csr.argtypes = [i64, i64, vp, i32, i64, i64, vp, vp, i64]
        L.oracle_fwd.restype = ctypes.c_int
        L.oracle_fwd.argtypes = [i64, i64, i64, vp, i32, ctypes.c_int, dbl, ctypes.c_int,
                                 vp, vp, vp, ctypes.c_int, vp, vp, dbl, dbl, vp, i64, vp, vp]
        L.oracle_bwd.restype = ctypes.c_int
        L.oracle_bwd.argtypes = [i64, i64, i64, vp, i32, ctypes.c_int, dbl, ctypes.c_int,
                                 vp, vp, vp, ctypes.c_int, vp, vp, dbl, dbl, vp,
                                 vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_fwd_csr.restype = ctypes.c_int
        L.oracle_fwd_csr.argtypes = [i64, i64, vp, vp, ctypes.c_int, dbl, ctypes.c_int,
                                     vp, vp, vp, ctypes.c_int, vp, vp, dbl, dbl, vp, vp]
        L.oracle_bwd_csr.restype = ctypes.c_int
        L.oracle_bwd_csr.argtypes = [i64, i64, vp, vp, ctypes.c_int, dbl, ctypes.c_int,
                                     vp, vp, vp, ctypes.c_int, vp, vp, dbl, dbl, vp,
                                     vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_dense_causal.restype = ctypes.c_int
        L.oracle_dense_causal.argtypes = [i64, i64, dbl, ctypes.c_int, vp, vp, vp, vp, vp]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the OpenMP regions that follow (timing only)."""
    lib().oracle_set_num_threads(int(n))


# ---------------------------------------------------------------- marshalling
def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _as_input(a):
    """Return (contiguous array, dtype code).  bf16 arrives as uint16 bits."""
    if a is None:
        return None, F64
    a = np.ascontiguousarray(a)
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError("oracle inputs are float64, float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _check_shapes(T, D, **arrays):
    for name, a in arrays.items():
        if a is None:
            continue
        want = (T, 3) if name in ("cq", "ck") else (T, D)
        if tuple(np.shape(a)) != want:
            raise ValueError("%s has shape %s, expected %s" % (name, np.shape(a), want))


def _offs(offsets):
    o = np.ascontiguousarray(np.asarray(list(offsets), dtype=np.int64).reshape(-1))
    return o


# ---------------------------------------------------------------- graph
def row(T: int, W: int, offsets, i: int) -> np.ndarray:
    """N(i), ascending."""
    o = _offs(offsets)
    buf = np.empty(min(W, T) + len(o), dtype=np.int64)
    n = lib().oracle_row(T, W, _ptr(o), len(o), i, _ptr(buf))
    if n < 0:
        raise ValueError("oracle_row: bad argument")
    return buf[:n].copy()


def graph_csr(T: int, W: int, offsets, r0: int = 0, r1: int | None = None):
    """(row_ptr int64[n+1], cols int64[E]) for rows [r0, r1)."""
    r1 = T if r1 is None else r1
    o = _offs(offsets)
    rp = np.empty(r1 - r0 + 1, dtype=np.int64)
    e = lib().oracle_graph_csr(T, W, _ptr(o), len(o), r0, r1, _ptr(rp), None, 0)
    if e == -1:
        raise ValueError("oracle_graph_csr: bad argument")
    E = -(e + 2)
    cols = np.empty(max(E, 1), dtype=np.int64)
    e = lib().oracle_graph_csr(T, W, _ptr(o), len(o), r0, r1, _ptr(rp), _ptr(cols), E)
    if e != E:
        raise RuntimeError("oracle_graph_csr: inconsistent edge count")
    return rp, cols[:E]


# ---------------------------------------------------------------- forward
def fwd(T, W, offsets, v, q=None, k=None, cq=None, ck=None, gamma=0.0, beta=0.0,
        scale=None, rows=None):
    """One (batch, head) slice.  Dot mode when q, k are given, coordinate mode
    when cq, ck are, uniform mode (equal weights) when neither is.  Returns
    (O [n, D] float64, LSE [n] float64)."""
    o = _offs(offsets)
    v, vdt = _as_input(v)
    D = v.shape[-1]
    _check_shapes(T, D, v=v, q=q, k=k, cq=cq, ck=ck)
    coord = cq is not None
    if coord:
        mode, dt = SCORE_COORD, vdt
        cq, cdt = _as_input(cq)
        ck, cdt2 = _as_input(ck)
        assert cdt == cdt2
        q_ = k_ = None
    elif q is None and k is None:
        mode, dt, cdt = SCORE_UNIFORM, vdt, F64
        q_ = k_ = None
    else:
        mode, cdt = SCORE_DOT, F64
        q_, dt = _as_input(q)
        k_, dt2 = _as_input(k)
        assert dt == dt2 == vdt, "q, k, v share one element type"
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is not None:
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = len(rows)
    else:
        n = T
    O = np.empty((n, D), dtype=np.float64)
    L = np.empty(n, dtype=np.float64)
    rc = lib().oracle_fwd(T, D, W, _ptr(o), len(o), mode, float(scale), dt, _ptr(q_), _ptr(k_),
                          _ptr(v), cdt, _ptr(cq), _ptr(ck), float(gamma), float(beta),
                          _ptr(rows), n, _ptr(O), _ptr(L))
    if rc != 0:
        raise ValueError("oracle_fwd failed (%d)" % rc)
    return O, L


def dense_causal(q, k, v, scale=None):
    q, dt = _as_input(q)
    k, _ = _as_input(k)
    v, _ = _as_input(v)
    T, D = q.shape
    _check_shapes(T, D, q=q, k=k, v=v)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    O = np.empty((T, D), dtype=np.float64)
    L = np.empty(T, dtype=np.float64)
    rc = lib().oracle_dense_causal(T, D, float(scale), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(O), _ptr(L))
    if rc != 0:
        raise ValueError("oracle_dense_causal failed (%d)" % rc)
    return O, L


# ---------------------------------------------------------------- backward
def bwd(T, W, offsets, v, dO, q=None, k=None, cq=None, ck=None, gamma=0.0, beta=0.0,
        scale=None):
    """One (batch, head) slice.  Returns a dict of float64 gradients:
    dot mode {dq, dk, dv}; coordinate mode {dv, dcq, dck, dgamma, dbeta, l1};
    uniform mode (neither q, k nor cq, ck given) {dv}."""
    o = _offs(offsets)
    v, vdt = _as_input(v)
    dO, ddt = _as_input(dO)
    assert ddt == vdt, "dO shares the element type of v"
    D = v.shape[-1]
    _check_shapes(T, D, v=v, dO=dO, q=q, k=k, cq=cq, ck=ck)
    coord = cq is not None
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dV = np.empty((T, D), dtype=np.float64)
    out = {"dv": dV}
    g = np.zeros(1)
    b = np.zeros(1)
    l1 = np.zeros(1)
    if coord:
        cq, cdt = _as_input(cq)
        ck, _ = _as_input(ck)
        dcq = np.empty((T, 3), dtype=np.float64)
        dck = np.empty((T, 3), dtype=np.float64)
        rc = lib().oracle_bwd(T, D, W, _ptr(o), len(o), SCORE_COORD, float(scale), vdt, None, None,
                              _ptr(v), cdt, _ptr(cq), _ptr(ck), float(gamma), float(beta), _ptr(dO),
                              None, None, _ptr(dV), _ptr(dcq), _ptr(dck), _ptr(g), _ptr(b), _ptr(l1))
        out.update(dcq=dcq, dck=dck, dgamma=float(g[0]), dbeta=float(b[0]), l1=float(l1[0]))
    elif q is None and k is None:
        rc = lib().oracle_bwd(T, D, W, _ptr(o), len(o), SCORE_UNIFORM, float(scale), vdt, None, None,
                              _ptr(v), F64, None, None, 0.0, 0.0, _ptr(dO),
                              None, None, _ptr(dV), None, None, None, None, None)
    else:
        q, dt = _as_input(q)
        k, _ = _as_input(k)
        assert dt == vdt
        dQ = np.empty((T, D), dtype=np.float64)
        dK = np.empty((T, D), dtype=np.float64)
        rc = lib().oracle_bwd(T, D, W, _ptr(o), len(o), SCORE_DOT, float(scale), vdt, _ptr(q), _ptr(k),
                              _ptr(v), F64, None, None, 0.0, 0.0, _ptr(dO),
                              _ptr(dQ), _ptr(dK), _ptr(dV), None, None, None, None, None)
        out.update(dq=dQ, dk=dK)
    if rc != 0:
        raise ValueError("oracle_bwd failed (%d)" % rc)
    return out


# ---------------------------------------------------------------- batched helpers
def fwd_bh(W, offsets, v, q=None, k=None, cq=None, ck=None, gamma=None, beta=None,
           scale=None, rows=None):
    """[B, H, T, D] arrays (c: [B, H, T, 3], gamma/beta: [H]).  Loops over
    (b, h) slices.  Returns O [B, H, n, D], LSE [B, H, n]."""
    B, H, T, D = v.shape
    n = T if rows is None else len(rows)
    O = np.empty((B, H, n, D))
    L = np.empty((B, H, n))
    for b in range(B):
        for h in range(H):
            if cq is not None:
                O[b, h], L[b, h] = fwd(T, W, offsets, v[b, h], cq=cq[b, h], ck=ck[b, h],
                                       gamma=float(gamma[h]), beta=float(beta[h]), rows=rows)
            elif q is None:
                O[b, h], L[b, h] = fwd(T, W, offsets, v[b, h], rows=rows)
            else:
                O[b, h], L[b, h] = fwd(T, W, offsets, v[b, h], q=q[b, h], k=k[b, h],
                                       scale=scale, rows=rows)
    return O, L


def bwd_bh(W, offsets, v, dO, q=None, k=None, cq=None, ck=None, gamma=None, beta=None,
           scale=None):
    """[B, H, T, D] arrays.  Returns batched gradients; dgamma/dbeta/l1 are [H]
    sums over the batch."""
    B, H, T, D = v.shape
    res = {}
    for b in range(B):
        for h in range(H):
            if cq is not None:
                r = bwd(T, W, offsets, v[b, h], dO[b, h], cq=cq[b, h], ck=ck[b, h],
                        gamma=float(gamma[h]), beta=float(beta[h]))
            elif q is None:
                r = bwd(T, W, offsets, v[b, h], dO[b, h])
            else:
                r = bwd(T, W, offsets, v[b, h], dO[b, h], q=q[b, h], k=k[b, h], scale=scale)
            for key, val in r.items():
                if key in ("dgamma", "dbeta", "l1"):
                    res.setdefault(key, np.zeros(H))[h] += val
                else:
                    res.setdefault(key, np.empty((B, H) + val.shape))[b, h] = val
    return res


# ---------------------------------------------------------------- explicit graphs
def _csr(row_ptr, cols):
    rp = np.ascontiguousarray(np.asarray(row_ptr, dtype=np.int64))
    cl = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    return rp, cl


def _mode_args(q, k, cq, ck, vdt):
    """(mode, dtype of q/k or v, cdtype, q, k, cq, ck) as the C calls take them."""
    if cq is not None:
        cq, cdt = _as_input(cq)
        ck, _ = _as_input(ck)
        return SCORE_COORD, vdt, cdt, None, None, cq, ck
    if q is None and k is None:
        return SCORE_UNIFORM, vdt, F64, None, None, None, None
    q, dt = _as_input(q)
    k, dt2 = _as_input(k)
    assert dt == dt2 == vdt, "q, k, v share one element type"
    return SCORE_DOT, dt, F64, q, k, None, None


def fwd_csr(row_ptr, cols, v, q=None, k=None, cq=None, ck=None, gamma=0.0, beta=0.0, scale=None):
    """One (batch, head) slice over an explicit graph (row i: keys
    cols[row_ptr[i]:row_ptr[i+1]], ascending, each <= i).  Modes as in fwd.
    Returns (O [T, D], LSE [T]) float64."""
    rp, cl = _csr(row_ptr, cols)
    v, vdt = _as_input(v)
    T, D = v.shape
    _check_shapes(T, D, v=v, q=q, k=k, cq=cq, ck=ck)
    mode, dt, cdt, q_, k_, cq_, ck_ = _mode_args(q, k, cq, ck, vdt)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    O = np.empty((T, D), dtype=np.float64)
    L = np.empty(T, dtype=np.float64)
    rc = lib().oracle_fwd_csr(T, D, _ptr(rp), _ptr(cl), mode, float(scale), dt, _ptr(q_), _ptr(k_), _ptr(v),
                              cdt, _ptr(cq_), _ptr(ck_), float(gamma), float(beta), _ptr(O), _ptr(L))
    if rc != 0:
        raise ValueError("oracle_fwd_csr failed (%d)" % rc)
    return O, L


def bwd_csr(row_ptr, cols, v, dO, q=None, k=None, cq=None, ck=None, gamma=0.0, beta=0.0, scale=None):
    """Backward over an explicit graph; returns the gradients of bwd."""
    rp, cl = _csr(row_ptr, cols)
    v, vdt = _as_input(v)
    dO, ddt = _as_input(dO)
    assert ddt == vdt, "dO shares the element type of v"
    T, D = v.shape
    _check_shapes(T, D, v=v, dO=dO, q=q, k=k, cq=cq, ck=ck)
    mode, dt, cdt, q_, k_, cq_, ck_ = _mode_args(q, k, cq, ck, vdt)
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    out = {"dv": np.empty((T, D))}
    g, b, l1 = np.zeros(1), np.zeros(1), np.zeros(1)
    dQ = dK = dcq = dck = None
    if mode == SCORE_DOT:
        dQ, dK = np.empty((T, D)), np.empty((T, D))
        out.update(dq=dQ, dk=dK)
    if mode == SCORE_COORD:
        dcq, dck = np.empty((T, 3)), np.empty((T, 3))
    rc = lib().oracle_bwd_csr(T, D, _ptr(rp), _ptr(cl), mode, float(scale), dt, _ptr(q_), _ptr(k_), _ptr(v),
                              cdt, _ptr(cq_), _ptr(ck_), float(gamma), float(beta), _ptr(dO),
                              _ptr(dQ), _ptr(dK), _ptr(out["dv"]), _ptr(dcq), _ptr(dck),
                              _ptr(g) if mode == SCORE_COORD else None, _ptr(b) if mode == SCORE_COORD else None,
                              _ptr(l1) if mode == SCORE_COORD else None)
    if rc != 0:
        raise ValueError("oracle_bwd_csr failed (%d)" % rc)
    if mode == SCORE_COORD:
        out.update(dcq=dcq, dck=dck, dgamma=float(g[0]), dbeta=float(b[0]), l1=float(l1[0]))
    return out

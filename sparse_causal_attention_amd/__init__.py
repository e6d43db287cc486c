"""Sparse causal attention over a fixed per-query neighbour graph, for MI355X.

Thin Python binding of the C ABI in ``include/sa.h`` (same names).  It only
marshals arguments: torch supplies device memory and the current stream;
every step of the computation runs in the HIP kernels of ``libsa.so``.  There
is no CPU or PyTorch fallback: tensors must live on the GPU and the library
must be built (``python -m sparse_causal_attention_amd.build``).

    g = sa_build_graph(T, window=4, offsets=[2**k for k in range(14)])
    o, lse = sa_fwd(g, q, k, v)                 # [B, H, T, D], [B, H, T]
    grads = sa_bwd(g, q, k, v, o, lse, dout)    # {"dq", "dk", "dv"}

Any other causal graph is given as explicit per-row key lists:
``sa_build_graph_csr(T, row_ptr, cols)``.  Its lists are copied into a
device buffer (held by the Graph for its whole life) on first use, or by
``Graph.upload``; a graph is uploaded once, to one device.

Streams: calls run on ``stream`` (default: torch's current stream).  When
``stream`` is another stream, it first waits for the current stream's queued
work (which produced the inputs), and every tensor the binding allocates
(outputs, the backward's workspace) is allocated on ``stream`` itself, so the
caching allocator never hands that memory to other work before the kernels
on ``stream`` are done with it.

Coordinate score (-gamma_h ||c_q - c_k||^2 + beta_h): pass ``cq``, ``ck``
([B, H, T, 3] fp32), ``gamma``, ``beta`` ([H] fp32) instead of ``q``, ``k``.
Uniform score (every neighbour weighted 1 / |N(i)|): pass ``v`` alone; the
backward then returns ``{"dv"}`` only.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _abi
from ._abi import (SA_ALGO_AUTO, SA_ALGO_BAND, SA_ALGO_GATHER, SA_BF16, SA_F32, SA_GRAPH_CSR,
                   SA_MAX_DILATED, SA_SCORE_COORD, SA_SCORE_DOT, SA_SCORE_UNIFORM, SaError)

__all__ = ["sa_build_graph", "sa_build_graph_csr", "sa_fwd", "sa_bwd", "sa_bwd_noalloc", "sa_decode",
           "sa_decode_prepared", "sa_fwd_prepared", "sa_bwd_prepared",
           "sa_bwd_workspace_size", "sa_describe_plan", "Graph", "SaError"]

_ALGOS = {"auto": SA_ALGO_AUTO, "gather": SA_ALGO_GATHER, "band": SA_ALGO_BAND}


class Graph:
    """Owns an ``sa_graph`` handle (host memory) and, for explicit lists, the
    device buffer they were uploaded into."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        self._dev = None  # device copy of explicit lists (torch uint8 tensor)
        L = _abi.lib()
        T, W, nd, ne = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int64()
        dil = (ctypes.c_int64 * SA_MAX_DILATED)()
        _abi.check(L.sa_graph_info(self._h, ctypes.byref(T), ctypes.byref(W), ctypes.byref(nd),
                                   dil, ctypes.byref(ne)), "sa_graph_info")
        self.T, self.window, self.n_edges = T.value, W.value, ne.value
        self.dilations = tuple(dil[t] for t in range(nd.value))
        kind = ctypes.c_int32()
        _abi.check(L.sa_graph_kind(self._h, ctypes.byref(kind)), "sa_graph_kind")
        self.kind = kind.value

    @property
    def handle(self):
        return self._h

    @property
    def is_csr(self) -> bool:
        return self.kind == SA_GRAPH_CSR

    def device_bytes(self) -> int:
        n = ctypes.c_size_t()
        _abi.check(_abi.lib().sa_graph_device_bytes(self._h, ctypes.byref(n)), "sa_graph_device_bytes")
        return n.value

    def upload(self, device, stream=None):
        """Copies explicit lists into a device buffer this Graph keeps until it
        is freed (no-op for distance graphs or when already on `device`).  The
        library fixes a graph's device lists at the first upload, so a graph
        used on one device cannot move to another: build a second graph."""
        if not self.is_csr:
            return self
        torch = _torch()
        device = torch.device(device)
        if device.type != "cuda":
            raise ValueError("explicit lists are uploaded to a GPU device, got %s" % device)
        if device.index is None:
            device = torch.device("cuda", torch.cuda.current_device())
        if self._dev is not None:
            if self._dev.device == device:
                return self
            raise ValueError("this graph's lists are on %s; build another graph for %s"
                             % (self._dev.device, device))
        n = self.device_bytes()
        buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
        off = (-buf.data_ptr()) % 256  # the library wants 256-byte alignment
        view = buf[off:off + n]
        with torch.cuda.device(device):
            _abi.check(_abi.lib().sa_graph_upload(self._h, ctypes.c_void_p(view.data_ptr()), n,
                                                  _stream(stream)), "sa_graph_upload")
        self._dev = buf  # kept for the Graph's lifetime: the library refers to it
        return self

    def _used_on(self, stream):
        """Marks the uploaded lists as read by kernels on `stream` (when that is
        not the current stream), so that dropping the Graph while such kernels
        run does not release the buffer to other work."""
        if self._dev is None or stream is None:
            return
        torch = _torch()
        if stream.cuda_stream != torch.cuda.current_stream(self._dev.device).cuda_stream:
            self._dev.record_stream(stream)

    def _rows(self, fn, r0, r1):
        r1 = self.T if r1 is None else r1
        rp = np.zeros(max(r1 - r0, 0) + 1, dtype=np.int64)
        st = fn(self._h, r0, r1, rp.ctypes.data, None, 0)
        need = int(rp[-1])
        if st != _abi.SA_OK and need == 0:
            _abi.check(st, "graph rows")
        cols = np.empty(max(need, 1), dtype=np.int64)
        _abi.check(fn(self._h, r0, r1, rp.ctypes.data, cols.ctypes.data, need), "graph rows")
        return rp, cols[:need]

    def rows(self, r0: int = 0, r1: int | None = None):
        """CSR (row_ptr, cols) of rows [r0, r1), keys ascending."""
        return self._rows(_abi.lib().sa_graph_rows, r0, r1)

    def rows_reverse(self, r0: int = 0, r1: int | None = None):
        """CSR of the reverse graph: for key j, the queries that attend to it."""
        return self._rows(_abi.lib().sa_graph_rows_reverse, r0, r1)

    def __del__(self):
        if getattr(self, "_h", None) is not None and self._h.value and _abi._lib is not None:
            _abi._lib.sa_graph_free(self._h)
            self._h = None

    def __repr__(self):
        if self.is_csr:
            return "Graph(T=%d, explicit lists, edges/head=%d)" % (self.T, self.n_edges)
        return "Graph(T=%d, window=%d, dilations=%s, edges/head=%d)" % (
            self.T, self.window, list(self.dilations), self.n_edges)


def sa_build_graph(T: int, window: int, offsets=()) -> Graph:
    L = _abi.lib()
    offs = np.ascontiguousarray(np.asarray(list(offsets), dtype=np.int64).reshape(-1))
    h = ctypes.c_void_p()
    _abi.check(L.sa_build_graph(int(T), int(window), offs.ctypes.data if len(offs) else None,
                                len(offs), ctypes.byref(h)), "sa_build_graph")
    return Graph(h.value)


def sa_build_graph_csr(T: int, row_ptr, cols) -> Graph:
    """Graph from explicit lists: row i attends to cols[row_ptr[i]:row_ptr[i+1]]
    (strictly ascending, each <= i, at least one per row)."""
    L = _abi.lib()
    rp = np.ascontiguousarray(np.asarray(row_ptr, dtype=np.int64).reshape(-1))
    cl = np.ascontiguousarray(np.asarray(cols, dtype=np.int64).reshape(-1))
    if len(rp) != int(T) + 1:
        raise ValueError("row_ptr must have T + 1 entries")
    if len(cl) < int(rp[-1]):
        raise ValueError("cols has fewer than row_ptr[T] entries")
    h = ctypes.c_void_p()
    _abi.check(L.sa_build_graph_csr(int(T), rp.ctypes.data, cl.ctypes.data if len(cl) else None,
                                    ctypes.byref(h)), "sa_build_graph_csr")
    return Graph(h.value)


# ------------------------------------------------------------------ marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    raise TypeError("tensors are float32 or bfloat16, got %s" % t.dtype)


def _strides(t, name):
    if t is None:
        return (0, 0, 0)
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("%s must be [B, H, T, D] with a contiguous last dimension" % name)
    return tuple(int(s) for s in t.stride()[:3])


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require_gpu(**ts):
    for name, t in ts.items():
        if t is not None and not t.is_cuda:
            raise ValueError("%s must be a GPU tensor (there is no CPU path)" % name)


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class _on_stream:
    """Context for marshalling a call that will run on `stream`: if that is not
    torch's current stream, the launch stream first waits for the current
    stream's queued work, and tensors allocated inside the context belong to
    the launch stream (torch.cuda.stream), so the caching allocator reuses
    their memory only after the launch stream's kernels.  A no-op for the
    current stream (and so under graph capture, where the captured stream is
    the current one)."""

    def __init__(self, stream, device):
        self.stream = stream
        self.device = device
        self._ctx = None

    def __enter__(self):
        torch = _torch()
        if self.stream is None:
            return self
        cur = torch.cuda.current_stream(self.device)
        if self.stream.cuda_stream != cur.cuda_stream:
            self.stream.wait_stream(cur)
            self._ctx = torch.cuda.stream(self.stream)
            self._ctx.__enter__()
        return self

    def __exit__(self, *exc):
        if self._ctx is not None:
            self._ctx.__exit__(*exc)
        return False


def _make_desc(ref, *, score, algo, scale, grad_dtype, q=None, k=None, v=None, o=None, dout=None,
               dq=None, dk=None, dv=None, heads=None) -> _abi.SaAttnDesc:
    """ref: a [B, H_kv, T, D] key/value-side tensor; heads: the query heads H
    (None: H_kv).  Query-side tensors are checked against [B, H, T, D],
    key/value-side ones against [B, H_kv, T, D]."""
    B, Hkv, T, D = ref.shape
    H = Hkv if heads is None else int(heads)
    if H % Hkv != 0:
        raise ValueError("query heads (%d) must be a multiple of key/value heads (%d)" % (H, Hkv))
    d = _abi.SaAttnDesc()
    d.B, d.H, d.T, d.D = B, H, T, D
    d.H_kv = Hkv
    d.dtype = _dtype_code(ref)
    d.grad_dtype = grad_dtype
    d.score = score
    d.algo = _ALGOS[algo] if isinstance(algo, str) else int(algo)
    d.scale = 0.0 if scale is None else float(scale)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        want = (B, Hkv if name in ("k", "v", "dk", "dv") else H, T, D)
        if t is not None and tuple(t.shape) != want:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), want))
        getattr(d, "stride_" + name)[:] = _strides(t, name)
    return d


def _query_heads(q, o, v):
    """H: from q when given, else from o, else the key/value heads of v."""
    for t in (q, o):
        if t is not None:
            return t.shape[1]
    return v.shape[1]


def _coord_args(cq, ck, gamma, beta, B, H, T):
    torch = _torch()
    for name, t, shp in (("cq", cq, (B, H, T, 3)), ("ck", ck, (B, H, T, 3)), ("gamma", gamma, (H,)),
                         ("beta", beta, (H,))):
        if t is None or t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
            raise ValueError("%s must be a contiguous float32 tensor of shape %s" % (name, shp))


def _score_mode(q, k, cq):
    """Coordinate mode when c_q is given, uniform when neither q, k nor c_q
    is, dot otherwise."""
    if cq is not None:
        return SA_SCORE_COORD
    if q is None and k is None:
        return SA_SCORE_UNIFORM
    return SA_SCORE_DOT


def _fwd_args(graph, q, k, v, cq, ck, gamma, beta, scale, o, lse, algo, stream):
    torch = _torch()
    mode = _score_mode(q, k, cq)
    coord = mode == SA_SCORE_COORD
    _require_gpu(q=q, k=k, v=v, cq=cq, ck=ck, gamma=gamma, beta=beta, o=o, lse=lse)
    B, _, T, D = v.shape
    H = _query_heads(q, o, v)
    if coord:
        _coord_args(cq, ck, gamma, beta, B, H, T)
    with _on_stream(stream, v.device):
        if o is None:
            o = torch.empty((B, H, T, D), dtype=v.dtype, device=v.device)
        if lse is None:
            lse = torch.empty((B, H, T), dtype=torch.float32, device=v.device)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, T] tensor")
    d = _make_desc(v, score=mode, algo=algo, scale=scale, heads=H,
                   grad_dtype=SA_F32, q=None if coord else q, k=None if coord else k, v=v, o=o)
    graph.upload(v.device, stream)
    graph._used_on(stream)
    args = (graph.handle, ctypes.byref(d), _ptr(None if coord else q), _ptr(None if coord else k),
            _ptr(v), _ptr(cq), _ptr(ck), _ptr(gamma), _ptr(beta), _ptr(o), _ptr(lse), _stream(stream))
    return args, (d, o, lse)


def sa_fwd(graph: Graph, q=None, k=None, v=None, *, cq=None, ck=None, gamma=None, beta=None,
           scale=None, o=None, lse=None, algo="auto", stream=None):
    """Returns (o, lse).  o has v's dtype and shape, lse is [B, H, T] fp32."""
    args, (_d, o, lse) = _fwd_args(graph, q, k, v, cq, ck, gamma, beta, scale, o, lse, algo, stream)
    _abi.check(_abi.lib().sa_fwd(*args), "sa_fwd")
    return o, lse


def sa_fwd_prepared(graph: Graph, q=None, k=None, v=None, *, cq=None, ck=None, gamma=None,
                    beta=None, scale=None, o=None, lse=None, algo="auto", stream=None):
    """Marshals the arguments of sa_fwd once and returns a zero-argument
    callable that enqueues the same call again (same tensors, same stream).
    For tight loops where per-call Python marshalling would dominate.  The
    callable adds no stream synchronisation of its own: with a stream other
    than the current one, ordering against other streams is the caller's."""
    args, keep = _fwd_args(graph, q, k, v, cq, ck, gamma, beta, scale, o, lse, algo, stream)
    fn = _abi.lib().sa_fwd

    def call():
        _abi.check(fn(*args), "sa_fwd")
        return keep[1], keep[2]

    call.keepalive = (keep, graph)
    return call


def sa_bwd_workspace_size(graph: Graph, v, grad_dtype=None, heads=None) -> int:
    """Workspace bytes of sa_bwd for key/value tensor v ([B, H_kv, T, D]) and
    `heads` query heads (None: H_kv)."""
    d = _make_desc(v, score=SA_SCORE_DOT, algo="auto", scale=None, heads=heads,
                   grad_dtype=SA_F32 if grad_dtype is None else _dtype_code_of(grad_dtype))
    n = ctypes.c_size_t()
    _abi.check(_abi.lib().sa_bwd_workspace_size(graph.handle, ctypes.byref(d), ctypes.byref(n)),
               "sa_bwd_workspace_size")
    return n.value


def _dtype_code_of(dt) -> int:
    torch = _torch()
    return {torch.float32: SA_F32, torch.bfloat16: SA_BF16}[dt]


_NO_WORKSPACE = object()  # marks a backward marshalled for sa_bwd_noalloc


def _bwd_args(graph, q, k, v, o, lse, dout, cq, ck, gamma, beta, scale, grad_dtype, dq, dk, dv,
              dcq, dck, dgamma, dbeta, workspace, algo, stream):
    torch = _torch()
    mode = _score_mode(q, k, cq)
    coord = mode == SA_SCORE_COORD
    uniform = mode == SA_SCORE_UNIFORM
    _require_gpu(q=q, k=k, v=v, o=o, lse=lse, dout=dout, cq=cq, ck=ck, gamma=gamma, beta=beta)
    B, Hkv, T, D = v.shape
    H = _query_heads(q, o, v)
    gdt = torch.float32 if grad_dtype is None else grad_dtype
    gcode = _dtype_code_of(gdt)
    dev = v.device
    if coord:
        _coord_args(cq, ck, gamma, beta, B, H, T)
    with _on_stream(stream, dev):
        if coord:
            dcq = torch.empty((B, H, T, 3), dtype=torch.float32, device=dev) if dcq is None else dcq
            dck = torch.empty((B, H, T, 3), dtype=torch.float32, device=dev) if dck is None else dck
            dgamma = torch.empty((H,), dtype=torch.float32, device=dev) if dgamma is None else dgamma
            dbeta = torch.empty((H,), dtype=torch.float32, device=dev) if dbeta is None else dbeta
        elif uniform:
            dq = dk = None
        else:
            dq = torch.empty((B, H, T, D), dtype=gdt, device=dev) if dq is None else dq
            dk = torch.empty((B, Hkv, T, D), dtype=gdt, device=dev) if dk is None else dk
        dv = torch.empty((B, Hkv, T, D), dtype=gdt, device=dev) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is not None and t.dtype != gdt:
            raise ValueError("%s must have the gradient dtype %s" % (name, gdt))
    d = _make_desc(v, score=mode, algo=algo, scale=scale, heads=H,
                   grad_dtype=gcode, q=None if coord else q, k=None if coord else k, v=v, o=o,
                   dout=dout, dq=None if coord else dq, dk=None if coord else dk, dv=dv)
    L = _abi.lib()
    n = ctypes.c_size_t()
    _abi.check(L.sa_bwd_workspace_size(graph.handle, ctypes.byref(d), ctypes.byref(n)),
               "sa_bwd_workspace_size")
    ws_ptr, ws_bytes = None, 0
    if workspace is _NO_WORKSPACE:  # the allocation-free entry point brings its own
        workspace = None
    else:
        if workspace is None:
            with _on_stream(stream, dev):  # freed after the call, on the stream that used it
                workspace = torch.empty(max(n.value, 256), dtype=torch.uint8, device=dev)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    graph.upload(dev, stream)
    graph._used_on(stream)
    args = (graph.handle, ctypes.byref(d), _ptr(None if coord else q), _ptr(None if coord else k),
            _ptr(v), _ptr(cq), _ptr(ck), _ptr(gamma), _ptr(beta), _ptr(o), _ptr(lse), _ptr(dout),
            _ptr(None if coord else dq), _ptr(None if coord else dk), _ptr(dv),
            _ptr(dcq if coord else None), _ptr(dck if coord else None),
            _ptr(dgamma if coord else None), _ptr(dbeta if coord else None),
            ws_ptr, ws_bytes, _stream(stream))
    if coord:
        out = {"dv": dv, "dcq": dcq, "dck": dck, "dgamma": dgamma, "dbeta": dbeta}
    elif uniform:
        out = {"dv": dv}
    else:
        out = {"dq": dq, "dk": dk, "dv": dv}
    return args, (d, workspace, out)


def sa_bwd(graph: Graph, q=None, k=None, v=None, o=None, lse=None, dout=None, *, cq=None, ck=None,
           gamma=None, beta=None, scale=None, grad_dtype=None, dq=None, dk=None, dv=None,
           dcq=None, dck=None, dgamma=None, dbeta=None, workspace=None, algo="auto", stream=None):
    """Gradients of sum <dout, o>.  Dot mode returns {dq, dk, dv}; coordinate
    mode {dv, dcq, dck, dgamma, dbeta}; uniform mode {dv}.  Gradients default
    to fp32."""
    args, (_d, _ws, out) = _bwd_args(graph, q, k, v, o, lse, dout, cq, ck, gamma, beta, scale,
                                     grad_dtype, dq, dk, dv, dcq, dck, dgamma, dbeta, workspace,
                                     algo, stream)
    _abi.check(_abi.lib().sa_bwd(*args), "sa_bwd")
    return out


def sa_bwd_noalloc(graph: Graph, q=None, k=None, v=None, o=None, lse=None, dout=None, *, cq=None, ck=None,
                   gamma=None, beta=None, scale=None, grad_dtype=None, dq=None, dk=None, dv=None,
                   dcq=None, dck=None, dgamma=None, dbeta=None, algo="auto", stream=None):
    """sa_bwd through the library's allocation-free entry point: the workspace
    is the library's built-in device scratch (SA_NOALLOC_SCRATCH_BYTES per GPU),
    so with every output given (dq, dk, dv, or the coordinate-mode ones) the
    call allocates no device memory.  Calls that overlap on one GPU share that
    scratch and race: keep them on one stream."""
    args, (_d, _ws, out) = _bwd_args(graph, q, k, v, o, lse, dout, cq, ck, gamma, beta, scale,
                                     grad_dtype, dq, dk, dv, dcq, dck, dgamma, dbeta, _NO_WORKSPACE,
                                     algo, stream)
    _abi.check(_abi.lib().sa_bwd_noalloc(*(args[:19] + args[21:])), "sa_bwd_noalloc")
    return out


def sa_bwd_prepared(graph: Graph, q=None, k=None, v=None, o=None, lse=None, dout=None, *, cq=None,
                    ck=None, gamma=None, beta=None, scale=None, grad_dtype=None, dq=None, dk=None,
                    dv=None, dcq=None, dck=None, dgamma=None, dbeta=None, workspace=None,
                    algo="auto", stream=None):
    """Like sa_fwd_prepared, for sa_bwd."""
    args, keep = _bwd_args(graph, q, k, v, o, lse, dout, cq, ck, gamma, beta, scale, grad_dtype,
                           dq, dk, dv, dcq, dck, dgamma, dbeta, workspace, algo, stream)
    fn = _abi.lib().sa_bwd

    def call():
        _abi.check(fn(*args), "sa_bwd")
        return keep[2]

    call.keepalive = (keep, graph)
    return call


def _decode_args(graph, q, k, v, positions, cq, ck, gamma, beta, scale, o, lse, stream):
    torch = _torch()
    mode = _score_mode(q, k, cq)
    _require_gpu(q=q, k=k, v=v, positions=positions, cq=cq, ck=ck, gamma=gamma, beta=beta, o=o, lse=lse)
    B, _, T, D = v.shape
    H = q.shape[1] if q is not None else (o.shape[1] if o is not None else v.shape[1])
    if mode == SA_SCORE_COORD:
        for name, t, shp in (("cq", cq, (B, H, 3)), ("ck", ck, (B, H, T, 3)), ("gamma", gamma, (H,)),
                             ("beta", beta, (H,))):
            if t is None or t.dtype != torch.float32 or tuple(t.shape) != shp or not t.is_contiguous():
                raise ValueError("%s must be a contiguous float32 tensor of shape %s" % (name, shp))
    if positions is not None and (positions.dtype != torch.int32 or tuple(positions.shape) != (B,)
                                  or not positions.is_contiguous()):
        raise ValueError("positions must be a contiguous int32 [B] tensor")
    with _on_stream(stream, v.device):
        if o is None:
            o = torch.empty((B, H, D), dtype=v.dtype, device=v.device)
        if lse is None:
            lse = torch.empty((B, H), dtype=torch.float32, device=v.device)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H] tensor")
    d = _make_desc(v, score=mode, algo="auto", scale=scale, grad_dtype=SA_F32, heads=H,
                   k=k if mode == SA_SCORE_DOT else None, v=v)
    for name, t in (("q", q if mode == SA_SCORE_DOT else None), ("o", o)):
        if t is None:
            continue
        if t.dim() != 3 or tuple(t.shape) != (B, H, D) or t.stride(2) != 1:
            raise ValueError("%s must be [B, H, D] with a contiguous last dimension" % name)
        getattr(d, "stride_" + name)[:] = (int(t.stride(0)), int(t.stride(1)), 0)
    graph.upload(v.device, stream)
    graph._used_on(stream)
    args = (graph.handle, ctypes.byref(d), _ptr(positions), _ptr(q if mode == SA_SCORE_DOT else None),
            _ptr(k if mode == SA_SCORE_DOT else None), _ptr(v), _ptr(cq), _ptr(ck), _ptr(gamma), _ptr(beta),
            _ptr(o), _ptr(lse), _stream(stream))
    return args, (d, o, lse)


def sa_decode(graph: Graph, q=None, k=None, v=None, *, positions=None, cq=None, ck=None, gamma=None,
              beta=None, scale=None, o=None, lse=None, stream=None):
    """One new token per (batch, head) against the key/value caches.
    q [B, H, D] (dot) or cq [B, H, 3] (coordinate) or neither (uniform);
    k, v (or ck) caches [B, H, T, D] with T the graph's T; positions: int32
    [B] GPU tensor with each sequence's row (None: T - 1).  Returns
    (o [B, H, D], lse [B, H])."""
    args, (_d, o, lse) = _decode_args(graph, q, k, v, positions, cq, ck, gamma, beta, scale, o, lse,
                                      stream)
    _abi.check(_abi.lib().sa_decode(*args), "sa_decode")
    return o, lse


def sa_decode_prepared(graph: Graph, q=None, k=None, v=None, *, positions=None, cq=None, ck=None,
                       gamma=None, beta=None, scale=None, o=None, lse=None, stream=None):
    """Like sa_fwd_prepared, for sa_decode."""
    args, keep = _decode_args(graph, q, k, v, positions, cq, ck, gamma, beta, scale, o, lse, stream)
    fn = _abi.lib().sa_decode

    def call():
        _abi.check(fn(*args), "sa_decode")
        return keep[1], keep[2]

    call.keepalive = (keep, graph, positions)
    return call


def sa_describe_plan(graph: Graph, v, *, coord=False, algo="auto", which="fwd", score=None, heads=None) -> str:
    """Names of the kernels sa_fwd ("fwd") or sa_bwd ("bwd") would launch.
    score: "dot", "coord" or "uniform" (default: "coord" if coord else "dot")."""
    modes = {"dot": SA_SCORE_DOT, "coord": SA_SCORE_COORD, "uniform": SA_SCORE_UNIFORM}
    mode = modes[score] if score is not None else (SA_SCORE_COORD if coord else SA_SCORE_DOT)
    d = _make_desc(v, score=mode, algo=algo, scale=None, grad_dtype=SA_F32, heads=heads)
    buf = ctypes.create_string_buffer(256)
    _abi.check(_abi.lib().sa_describe_plan(graph.handle, ctypes.byref(d), 0 if which == "fwd" else 1,
                                           buf, 256), "sa_describe_plan")
    return buf.value.decode()

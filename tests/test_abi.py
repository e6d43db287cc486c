"""The C ABI library on a host without a GPU: it loads, exports every entry
point include/sa.h declares, and rejects every invalid request with its
status before any HIP call (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

from sparse_causal_attention_amd import _abi, sa_build_graph

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(_abi.EXPORTED)
    L = _abi.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = _abi.lib()
    for s in range(6):
        assert L.sa_status_str(s)
    assert L.sa_status_str(99) == b"unknown status"


FAKE = 0x10000  # 16-byte aligned stand-in; never dereferenced on these paths


def desc(B=1, H=2, T=64, D=32, dtype=0, score=0, algo=0, grad=0):
    d = _abi.SaAttnDesc()
    d.B, d.H, d.T, d.D = B, H, T, D
    d.dtype, d.grad_dtype, d.score, d.algo = dtype, grad, score, algo
    es = 2 if dtype == 1 else 4
    for name in ("q", "k", "v", "o", "do"):
        getattr(d, "stride_" + name)[:] = (H * T * D, T * D, D)
    for name in ("dq", "dk", "dv"):
        getattr(d, "stride_" + name)[:] = (H * T * D, T * D, D)
    _ = es
    return d


def fwd(g, d, q=FAKE, k=FAKE, v=FAKE, cq=None, ck=None, gm=None, bt=None, o=FAKE, lse=FAKE):
    return _abi.lib().sa_fwd(g.handle if g is not None else None, ctypes.byref(d) if d is not None else None,
                             q, k, v, cq, ck, gm, bt, o, lse, None)


def bwd(g, d, ws=FAKE, ws_bytes=1 << 30, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, cq=None, ck=None, gm=None, bt=None, o=FAKE, lse=FAKE, do=FAKE,
                dq=FAKE, dk=FAKE, dv=FAKE, dcq=None, dck=None, dg=None, db=None)
    args.update(kw)
    return _abi.lib().sa_bwd(g.handle, ctypes.byref(d), *args.values(), ws, ws_bytes, None)


@pytest.fixture
def g64():
    return sa_build_graph(64, 4, [4, 8, 16, 32])


def test_fwd_validation(g64):
    E = _abi
    assert fwd(None, desc()) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, None) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(T=65)) == E.SA_ERR_SHAPE_MISMATCH
    assert fwd(g64, desc(D=48)) == E.SA_ERR_UNSUPPORTED
    assert fwd(g64, desc(D=256)) == E.SA_ERR_UNSUPPORTED
    assert fwd(g64, desc(B=0)) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(H=-1)) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(dtype=7)) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(score=3)) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(algo=9)) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(), q=None) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(), v=None) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(), o=None) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(), lse=None) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(), q=FAKE + 4) == E.SA_ERR_INVALID_ARG  # misaligned row start
    d = desc()
    d.stride_k[2] = 33  # 132-byte rows: not 16-byte aligned
    assert fwd(g64, d) == E.SA_ERR_INVALID_ARG
    d = desc()
    d.stride_v[0] = -64
    assert fwd(g64, d) == E.SA_ERR_INVALID_ARG
    # coordinate mode needs c_q, c_k, gamma, beta
    assert fwd(g64, desc(score=1), q=None, k=None) == E.SA_ERR_INVALID_ARG
    assert fwd(g64, desc(score=1), q=None, k=None, cq=FAKE, ck=FAKE, gm=FAKE) == E.SA_ERR_INVALID_ARG
    # the band kernels do not apply to fp32 inputs
    assert fwd(g64, desc(algo=2)) == E.SA_ERR_UNSUPPORTED


def test_bwd_validation(g64):
    E = _abi
    d = desc()
    assert bwd(g64, d, ws=None) == E.SA_ERR_WORKSPACE
    assert bwd(g64, d, ws=FAKE + 16) == E.SA_ERR_WORKSPACE  # not 256-byte aligned
    need = ctypes.c_size_t()
    assert _abi.lib().sa_bwd_workspace_size(g64.handle, ctypes.byref(d), ctypes.byref(need)) == 0
    assert need.value >= 1 * 2 * 64 * 4
    assert bwd(g64, d, ws_bytes=need.value - 1) == E.SA_ERR_WORKSPACE
    assert bwd(g64, d, do=None) == E.SA_ERR_INVALID_ARG
    assert bwd(g64, d, dq=None) == E.SA_ERR_INVALID_ARG
    assert bwd(g64, d, dv=None) == E.SA_ERR_INVALID_ARG
    assert bwd(g64, d, lse=None) == E.SA_ERR_INVALID_ARG
    assert bwd(g64, d, dk=FAKE + 8) == E.SA_ERR_INVALID_ARG
    assert bwd(g64, desc(T=32)) == E.SA_ERR_SHAPE_MISMATCH
    dc = desc(score=1)
    assert bwd(g64, dc, q=None, k=None, cq=FAKE, ck=FAKE, gm=FAKE, bt=FAKE, dq=None, dk=None,
               dcq=FAKE, dck=FAKE, dg=FAKE) == E.SA_ERR_INVALID_ARG  # dbeta missing
    assert _abi.lib().sa_bwd_workspace_size(g64.handle, ctypes.byref(desc(T=8)),
                                            ctypes.byref(need)) == E.SA_ERR_SHAPE_MISMATCH


def plan(g, d, which):
    buf = ctypes.create_string_buffer(128)
    st = _abi.lib().sa_describe_plan(g.handle, ctypes.byref(d), which, buf, 128)
    return st, buf.value.decode()


def test_plan_selection():
    g = sa_build_graph(16384, 256, ())
    st, name = plan(g, desc(B=1, H=8, T=16384, D=64, dtype=1), 0)
    assert st == 0 and name
    st, name = plan(g, desc(B=1, H=8, T=16384, D=64, dtype=0), 0)
    assert st == 0 and name.startswith("gather")
    st, name = plan(g, desc(B=1, H=8, T=16384, D=64, dtype=1, algo=1), 1)
    assert st == 0 and name.startswith("gather_bwd")
    st, name = plan(g, desc(B=1, H=8, T=16384, D=64, dtype=1, score=1), 0)
    assert st == 0 and name == "gather_fwd_kernel(coord)"


def test_plan_band_backward_slice_limit():
    """The band backward loads its tiles with 32-bit offsets over one (batch,
    head) slice: past 2^31 bytes per slice the backward takes the gather
    kernels (BAND fails) while the forward stays on the band kernel."""
    for T, band_bwd in ((1 << 23, True), (1 << 25, False)):
        g = sa_build_graph(T, 256, ())
        d = desc(B=1, H=1, T=T, D=64, dtype=1)
        st, name = plan(g, d, 0)
        assert st == 0 and name == "band_fwd_kernel"
        st, name = plan(g, d, 1)
        assert st == 0
        assert name.startswith("band_bwd") == band_bwd, (T, name)
        st, _ = plan(g, desc(B=1, H=1, T=T, D=64, dtype=1, algo=2), 1)
        assert st == (0 if band_bwd else _abi.SA_ERR_UNSUPPORTED)
    # a wide row stride counts: 2^21 rows at 2 KiB per row exceed 2^31 bytes
    g = sa_build_graph(1 << 21, 256, ())
    d = desc(B=1, H=16, T=1 << 21, D=64, dtype=1)
    for name_ in ("q", "k", "v", "do"):
        getattr(d, "stride_" + name_)[:] = (16 * (1 << 21) * 64, 64, 16 * 64)
    st, name = plan(g, d, 1)
    assert st == 0 and name.startswith("gather_bwd"), name
    # so does a batch stride of 2^31 elements or more (the strides are held in 32 bits)
    g = sa_build_graph(4096, 256, ())
    d = desc(B=2, H=1, T=4096, D=64, dtype=1)
    st, name = plan(g, d, 1)
    assert st == 0 and name.startswith("band_bwd"), name
    d.stride_k[0] = 1 << 31
    st, name = plan(g, d, 1)
    assert st == 0 and name.startswith("gather_bwd"), name


def test_plan_uniform_mode():
    """The uniform score reads v alone and runs on the gather kernels; its
    backward is the key-side pass only; the band kernels do not apply."""
    g = sa_build_graph(16384, 4, [2 ** k for k in range(14)])
    st, name = plan(g, desc(B=4, H=8, T=16384, D=64, dtype=1, score=2), 0)
    assert st == 0 and name == "gather_fwd_kernel(uniform)"
    st, name = plan(g, desc(B=4, H=8, T=16384, D=64, dtype=1, score=2), 1)
    assert st == 0 and name == "gather_bwd_kv_kernel(uniform)"
    gb = sa_build_graph(16384, 256, ())
    st, _ = plan(gb, desc(B=1, H=8, T=16384, D=64, dtype=1, score=2, algo=2), 0)
    assert st == _abi.SA_ERR_UNSUPPORTED
    # q, k, cq, ck, gamma, beta are not needed: only v must be given
    assert fwd(g64_graph(), desc(score=2), q=None, k=None, v=None) == _abi.SA_ERR_INVALID_ARG


def g64_graph():
    return sa_build_graph(64, 4, [4, 8, 16, 32])


def decode(g, d, positions=None, q=FAKE, k=FAKE, v=FAKE, cq=None, ck=None, gm=None, bt=None, o=FAKE, lse=FAKE):
    return _abi.lib().sa_decode(g.handle, ctypes.byref(d) if d is not None else None, positions, q, k, v,
                                cq, ck, gm, bt, o, lse, None)


def test_decode_validation(g64):
    E = _abi
    assert _abi.lib().sa_decode(None, ctypes.byref(desc()), None, FAKE, FAKE, FAKE, None, None, None, None,
                                FAKE, FAKE, None) == E.SA_ERR_INVALID_ARG
    assert decode(g64, desc(T=65)) == E.SA_ERR_SHAPE_MISMATCH
    assert decode(g64, desc(D=48)) == E.SA_ERR_UNSUPPORTED
    assert decode(g64, desc(score=5)) == E.SA_ERR_INVALID_ARG
    assert decode(g64, desc(), v=None) == E.SA_ERR_INVALID_ARG
    assert decode(g64, desc(), q=None) == E.SA_ERR_INVALID_ARG
    assert decode(g64, desc(), k=None) == E.SA_ERR_INVALID_ARG
    assert decode(g64, desc(), o=None) == E.SA_ERR_INVALID_ARG
    assert decode(g64, desc(), lse=None) == E.SA_ERR_INVALID_ARG
    assert decode(g64, desc(), q=FAKE + 4) == E.SA_ERR_INVALID_ARG
    d = desc()
    d.stride_o[1] = 33  # 132-byte rows of o: not 16-byte aligned
    assert decode(g64, d) == E.SA_ERR_INVALID_ARG
    # coordinate mode needs cq, ck, gamma, beta; uniform mode needs v alone
    assert decode(g64, desc(score=1), q=None, k=None, cq=FAKE, ck=FAKE, gm=FAKE) == E.SA_ERR_INVALID_ARG
    assert decode(g64, desc(score=2), q=None, k=None, v=None) == E.SA_ERR_INVALID_ARG


def test_grouped_heads_validation(g64):
    """H must be a multiple of H_kv; coordinate mode needs H_kv = H; grouped
    heads need no extra workspace."""
    E = _abi
    d = desc(H=4)
    d.H_kv = 3
    assert fwd(g64, d) == E.SA_ERR_INVALID_ARG
    d.H_kv = -1
    assert fwd(g64, d) == E.SA_ERR_INVALID_ARG
    d = desc(H=4, score=1)
    d.H_kv = 2
    assert fwd(g64, d, q=None, k=None, cq=FAKE, ck=FAKE, gm=FAKE, bt=FAKE) == E.SA_ERR_UNSUPPORTED
    need1, need2 = ctypes.c_size_t(), ctypes.c_size_t()
    d = desc(H=4)
    assert _abi.lib().sa_bwd_workspace_size(g64.handle, ctypes.byref(d), ctypes.byref(need1)) == 0
    d.H_kv = 2
    assert _abi.lib().sa_bwd_workspace_size(g64.handle, ctypes.byref(d), ctypes.byref(need2)) == 0
    assert need2.value == need1.value  # grouped heads need no extra workspace
    d.H_kv = 3
    assert _abi.lib().sa_bwd_workspace_size(g64.handle, ctypes.byref(d),
                                            ctypes.byref(need2)) == E.SA_ERR_INVALID_ARG
    # H_kv = 0 means H (callers that zero-fill the descriptor)
    d.H_kv = 0
    assert _abi.lib().sa_bwd_workspace_size(g64.handle, ctypes.byref(d), ctypes.byref(need2)) == 0
    assert need2.value == need1.value


def test_explicit_lists_need_an_upload_and_pick_indexed_kernels():
    """An explicit-list graph: plans name the indexed kernels, the band kernels
    are unsupported, and every compute call is refused until the lists are in
    device memory.  sa_graph_upload rejects a bad buffer before touching the
    GPU, and is a no-op for a distance graph."""
    from sparse_causal_attention_amd import sa_build_graph_csr

    E = _abi
    L = _abi.lib()
    T = 64
    rp = [0]
    cols = []
    for i in range(T):
        row = sorted({0, i // 2, i})
        cols += row
        rp.append(len(cols))
    g = sa_build_graph_csr(T, rp, cols)
    assert plan(g, desc(), 0) == (0, "csr_fwd_kernel(dot)")
    assert plan(g, desc(score=1), 1) == (
        0, "csr_bwd_q_kernel(coord)+csr_bwd_kv_kernel(coord)+coord_param_reduce_kernel")
    assert plan(g, desc(score=2), 1) == (0, "csr_bwd_kv_kernel(uniform)")
    assert plan(g, desc(dtype=1, D=64), 0) == (0, "csr_fwd_kernel(dot)")  # never the band kernels
    assert plan(g, desc(dtype=1, D=64, algo=2), 0)[0] == E.SA_ERR_UNSUPPORTED
    assert fwd(g, desc()) == E.SA_ERR_INVALID_ARG
    assert bwd(g, desc()) == E.SA_ERR_INVALID_ARG
    assert decode(g, desc()) == E.SA_ERR_INVALID_ARG
    n = g.device_bytes()
    assert n > 0
    assert L.sa_graph_upload(g.handle, None, n, None) == E.SA_ERR_INVALID_ARG
    assert L.sa_graph_upload(g.handle, FAKE + 16, n, None) == E.SA_ERR_INVALID_ARG  # not 256-byte aligned
    assert L.sa_graph_upload(g.handle, FAKE, n - 1, None) == E.SA_ERR_INVALID_ARG
    assert L.sa_graph_upload(None, FAKE, n, None) == E.SA_ERR_INVALID_ARG
    d = g64_graph()
    assert d.device_bytes() == 0 and not d.is_csr
    assert L.sa_graph_upload(d.handle, None, 0, None) == E.SA_OK
    kind = ctypes.c_int32(-1)
    assert L.sa_graph_kind(g.handle, ctypes.byref(kind)) == E.SA_OK and kind.value == E.SA_GRAPH_CSR
    assert L.sa_graph_kind(None, ctypes.byref(kind)) == E.SA_ERR_INVALID_ARG


def test_overlapping_outputs_are_rejected(g64):
    """Output rows must be disjoint: a zero or too-small stride would let
    several workgroups store the same row in no fixed order.  Inputs may
    alias (broadcast k, v over heads with a zero head stride, say)."""
    E = _abi
    d = desc()
    d.stride_o[2] = 0  # every t of a head on one row
    assert fwd(g64, d) == E.SA_ERR_INVALID_ARG
    d = desc()
    d.stride_o[1] = 0  # both heads on the same rows
    assert fwd(g64, d) == E.SA_ERR_INVALID_ARG
    d = desc()
    d.stride_o[2] = 16  # rows of 32 elements 16 apart: overlap
    assert fwd(g64, d) == E.SA_ERR_INVALID_ARG
    d = desc()
    d.stride_k[1] = 0  # an input broadcast over heads is fine: the call gets past
    d.stride_o[2] = 0  # ... the inputs and fails on the output
    assert fwd(g64, d) == E.SA_ERR_INVALID_ARG
    for name in ("dq", "dk", "dv"):
        d = desc()
        getattr(d, "stride_" + name)[2] = 0
        assert bwd(g64, d) == E.SA_ERR_INVALID_ARG, name
        d = desc()
        getattr(d, "stride_" + name)[1] = 8  # heads overlapping within a row
        assert bwd(g64, d) == E.SA_ERR_INVALID_ARG, name
        # disjoint layouts pass the gradient checks and reach the workspace check
        d = desc()
        getattr(d, "stride_" + name)[:] = (2 * 64 * 32, 32, 2 * 32)  # [B, T, H, D] storage
        assert bwd(g64, d, ws=None) == E.SA_ERR_WORKSPACE, name
        d = desc(B=1)
        getattr(d, "stride_" + name)[0] = 0  # an extent-1 dimension may have any stride
        assert bwd(g64, d, ws=None) == E.SA_ERR_WORKSPACE, name


def test_grid_must_fit_int32():
    """Workgroup counts are int32: B * H * ceil(T / 8) must stay below 2^31."""
    E = _abi
    T = 1 << 30
    g = sa_build_graph(T, 4, [])
    d = desc(B=1, H=16, T=T)
    assert fwd(g, d) == E.SA_ERR_UNSUPPORTED  # 16 * 2^27 = 2^31 workgroups
    d = desc(B=1, H=8, T=T)  # 2^30: fits, so the check passes and a later one fails
    assert fwd(g, d, lse=None) == E.SA_ERR_INVALID_ARG


def test_second_upload_is_refused_by_the_binding():
    """A graph's device lists are fixed at its first upload: the binding
    refuses to move an uploaded graph to another device (the library refuses a
    second sa_graph_upload; that half runs in the GPU tests)."""
    import torch

    from sparse_causal_attention_amd import sa_build_graph_csr

    g = sa_build_graph_csr(3, [0, 1, 2, 3], [0, 1, 2])

    class FakeBuf:  # stands in for the uploaded buffer on cuda:0
        device = torch.device("cuda", 0)

    g._dev = FakeBuf()
    assert g.upload("cuda:0") is g  # already there: nothing to do
    with pytest.raises(ValueError, match="build another graph"):
        g.upload("cuda:1")
    with pytest.raises(ValueError):
        g.upload("cpu")
    g._dev = None


def test_side_stream_marshalling(monkeypatch):
    """With stream= another stream than torch's current one, the launch stream
    waits for the current stream and the binding's allocations happen on the
    launch stream (so the caching allocator does not hand the memory to
    other work before those kernels finish); with the current stream nothing
    extra happens.  torch.cuda is replaced by fakes: no GPU is needed."""
    import torch

    import sparse_causal_attention_amd as pkg

    log = []

    class FakeStream:
        def __init__(self, h):
            self.cuda_stream = h

        def wait_stream(self, other):
            log.append(("wait", self.cuda_stream, other.cuda_stream))

    current = FakeStream(1)

    class FakeCtx:
        def __init__(self, s):
            self.s = s

        def __enter__(self):
            log.append(("enter", self.s.cuda_stream))

        def __exit__(self, *a):
            log.append(("exit", self.s.cuda_stream))

    monkeypatch.setattr(torch.cuda, "current_stream", lambda device=None: current)
    monkeypatch.setattr(torch.cuda, "stream", lambda s: FakeCtx(s))
    with pkg._on_stream(FakeStream(1), None):
        log.append("alloc")
    assert log == ["alloc"]
    log.clear()
    with pkg._on_stream(None, None):
        log.append("alloc")
    assert log == ["alloc"]
    log.clear()
    with pkg._on_stream(FakeStream(7), None):
        log.append("alloc")
    assert log == [("wait", 7, 1), ("enter", 7), "alloc", ("exit", 7)]

    # the uploaded lists of an explicit-list graph are recorded on the side stream
    recorded = []

    class FakeBuf:
        device = None

        def record_stream(self, s):
            recorded.append(s.cuda_stream)

    g = pkg.sa_build_graph_csr(2, [0, 1, 2], [0, 1])
    g._dev = FakeBuf()
    g._used_on(FakeStream(1))
    g._used_on(None)
    assert recorded == []
    g._used_on(FakeStream(9))
    assert recorded == [9]
    g._dev = None


def test_noalloc_validation():
    """sa_bwd_noalloc validates like sa_bwd (no workspace arguments) and
    rejects, before any HIP call, a shape whose workspace exceeds its built-in
    scratch."""
    E = _abi
    L = _abi.lib()

    def noalloc(g, d, **kw):
        args = dict(q=FAKE, k=FAKE, v=FAKE, cq=None, ck=None, gm=None, bt=None, o=FAKE, lse=FAKE, do=FAKE,
                    dq=FAKE, dk=FAKE, dv=FAKE, dcq=None, dck=None, dg=None, db=None)
        args.update(kw)
        return L.sa_bwd_noalloc(g.handle, ctypes.byref(d), *args.values(), None)

    T = 1 << 16
    g = sa_build_graph(T, 4, [])
    need = ctypes.c_size_t()
    big = desc(B=1, H=40, T=T, D=64, dtype=1)
    assert L.sa_bwd_workspace_size(g.handle, ctypes.byref(big), ctypes.byref(need)) == 0
    assert need.value > E.SA_NOALLOC_SCRATCH_BYTES
    assert noalloc(g, big) == E.SA_ERR_WORKSPACE
    assert noalloc(g, big, do=None) == E.SA_ERR_INVALID_ARG  # argument errors come first
    assert noalloc(g, desc(B=1, H=40, T=T - 1, D=64, dtype=1)) == E.SA_ERR_SHAPE_MISMATCH
    fits = desc(B=1, H=8, T=T, D=64, dtype=1)
    assert L.sa_bwd_workspace_size(g.handle, ctypes.byref(fits), ctypes.byref(need)) == 0
    assert need.value <= E.SA_NOALLOC_SCRATCH_BYTES
    d = desc(B=1, H=8, T=T, D=64, dtype=1)
    d.stride_dq[2] = 0
    assert noalloc(g, d) == E.SA_ERR_INVALID_ARG


def test_probe_library_exports_its_header():
    """libsa_probe.so (the benchmark's measurement probes) exports exactly the
    functions include/sa_probe.h declares."""
    import subprocess

    text = open(os.path.join(ROOT, "include", "sa_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    declared = set(re.findall(r"\b(sa_probe_[a-z_]+)\s*\(", text))
    lib = os.path.join(ROOT, "sparse_causal_attention_amd", "libsa_probe.so")
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T sa_probe_" in ln}
    assert declared == exported == {"sa_probe_copy", "sa_probe_mfma", "sa_probe_mfma_flops", "sa_probe_empty",
                                    "sa_probe_mix_variants", "sa_probe_mix_counts", "sa_probe_mix"}
    L = ctypes.CDLL(lib)
    flops = ctypes.c_double()
    assert L.sa_probe_mfma_flops(2, 3, ctypes.byref(flops)) == 0
    assert flops.value == 2 * 4 * 3 * 4 * 2 * 32 * 32 * 16  # workgroups x waves x iters x chains x flops
    assert L.sa_probe_mfma_flops(0, 3, ctypes.byref(flops)) == 1
    assert L.sa_probe_copy(None, None, ctypes.c_size_t(16), None) == 1  # validated before any launch


def test_huge_batch_and_heads_are_refused_before_any_product():
    """B and H are bounded one by one before B * H is formed (a product of two
    int64 values near 2^33 would overflow): with broadcast (stride 0) inputs,
    which pass every offset check, such shapes are SA_ERR_UNSUPPORTED for the
    forward, the backward, the workspace size and the decode step."""
    E = _abi
    g = sa_build_graph(64, 4, [])
    for B, H in ((1 << 33, 1 << 33), (1 << 40, 1), (1, 1 << 40), ((1 << 24) + 1, 1), (1 << 12, (1 << 12) + 1)):
        d = desc(B=B, H=H, T=64, D=32)
        for name in ("q", "k", "v", "do"):
            getattr(d, "stride_" + name)[:] = (0, 0, 32)
        assert fwd(g, d) == E.SA_ERR_UNSUPPORTED, (B, H)
        assert bwd(g, d) == E.SA_ERR_UNSUPPORTED, (B, H)
        n = ctypes.c_size_t(0)
        assert _abi.lib().sa_bwd_workspace_size(g.handle, ctypes.byref(d), ctypes.byref(n)) == \
            E.SA_ERR_UNSUPPORTED, (B, H)
    for B, H in ((1 << 33, 1 << 33), (1 << 31, 1), ((1 << 16), (1 << 15))):
        d = desc(B=B, H=H, T=64, D=32)
        for name in ("q", "k", "v", "o"):
            getattr(d, "stride_" + name)[:] = (0, 0, 32)
        st = _abi.lib().sa_decode(g.handle, ctypes.byref(d), None, FAKE, FAKE, FAKE, None, None, None, None,
                                  FAKE, FAKE, None)
        assert st == E.SA_ERR_UNSUPPORTED, (B, H)
    # the largest accepted slice count still validates (and fails later, on the null lse)
    d = desc(B=1 << 12, H=1 << 12, T=64, D=32)
    for name in ("q", "k", "v", "do"):
        getattr(d, "stride_" + name)[:] = (0, 0, 32)
    assert fwd(g, d, lse=None) == E.SA_ERR_INVALID_ARG

"""sa_build_graph and the CSR exports of libsa.so against the oracle's
set-union graph: bit-exact, CPU only (no GPU call is made)."""
import numpy as np
import pytest

import oracle
from sparse_causal_attention_amd import SaError, sa_build_graph
from sparse_causal_attention_amd.inputs import WORKLOADS


def oracle_reverse(T, W, offs):
    rp, cols = oracle.graph_csr(T, W, offs)
    rows = np.repeat(np.arange(T), np.diff(rp))
    order = np.lexsort((rows, cols))  # by key j, then query i
    rcols = rows[order]
    counts = np.bincount(cols, minlength=T)
    rrp = np.concatenate([[0], np.cumsum(counts)])
    return rrp, rcols


CASES = [
    (1, 1, ()), (2, 1, ()), (5, 9, ()), (12, 3, (1, 2, 4, 8)), (64, 4, tuple(2 ** k for k in range(7))),
    (256, 8, (16, 32, 64, 128)), (256, 256, ()), (300, 7, (0, 3, 3, 500, 299, 300, 150, 8)),
    (1000, 64, tuple(2 ** k for k in range(6, 10))), (2048, 2048, ()), (4097, 256, ()),
]


@pytest.mark.parametrize("T,W,offs", CASES)
def test_rows_bit_exact_against_oracle(T, W, offs):
    g = sa_build_graph(T, W, offs)
    rp, cols = g.rows()
    orp, ocols = oracle.graph_csr(T, W, offs)
    assert np.array_equal(rp, orp) and np.array_equal(cols, ocols)
    assert g.n_edges == orp[-1]
    rrp, rcols = g.rows_reverse()
    orrp, orcols = oracle_reverse(T, W, offs)
    assert np.array_equal(rrp, orrp) and np.array_equal(rcols, orcols)


@pytest.mark.parametrize("seed", range(20))
def test_rows_random_graphs(seed):
    r = np.random.default_rng(100 + seed)
    T = int(r.integers(1, 2000))
    W = int(r.integers(1, 300))
    offs = [int(x) for x in r.integers(0, 2 * T, size=int(r.integers(0, 20)))]
    g = sa_build_graph(T, W, offs)
    orp, ocols = oracle.graph_csr(T, W, offs)
    rp, cols = g.rows()
    assert np.array_equal(rp, orp) and np.array_equal(cols, ocols)
    # a sub-range, relative row pointers
    a = int(r.integers(0, T))
    b = int(r.integers(a, T + 1))
    srp, scols = g.rows(a, b)
    assert np.array_equal(srp, orp[a:b + 1] - orp[a])
    assert np.array_equal(scols, ocols[orp[a]:orp[b]])


@pytest.mark.parametrize("name", ["tiny", "tiny_dense", "band", "band_dense", "dilated"])
def test_workload_graphs(name):
    w = WORKLOADS[name]
    g = sa_build_graph(w.T, w.window, w.offsets)
    orp, ocols = oracle.graph_csr(w.T, w.window, w.offsets)
    rp, cols = g.rows()
    assert g.n_edges == orp[-1]
    assert np.array_equal(rp, orp) and np.array_equal(cols, ocols)


def test_ultra_long_graph_descriptor_and_sampled_rows():
    w = WORKLOADS["ultra"]
    g = sa_build_graph(w.T, w.window, w.offsets)
    assert g.window == 64 and g.dilations == tuple(2 ** k for k in range(6, 26))
    assert g.n_edges == 5570033760  # > 2^31: int64 count
    r = np.random.default_rng(7)
    for i in [0, 1, 63, 64, 65, 2 ** 25 - 1, 2 ** 25, 2 ** 25 + 1, w.T - 1] + list(r.integers(0, w.T, 50)):
        rp, cols = g.rows(int(i), int(i) + 1)
        assert np.array_equal(cols, oracle.row(w.T, w.window, w.offsets, int(i)))


def test_descriptor_normalisation():
    g = sa_build_graph(100, 5, [64, 3, 0, 8, 8, 200, 100, 99, 5, 4])
    # dropped: 3, 0, 4 (inside the window), 200, 100 (>= T); 8 deduplicated
    assert g.window == 5 and g.dilations == (5, 8, 64, 99)
    g = sa_build_graph(10, 50, [1, 2, 3])
    assert g.window == 10 and g.dilations == ()
    assert g.n_edges == 55


@pytest.mark.parametrize("args", [(0, 1, ()), (-3, 1, ()), (10, 0, ()), (10, -1, ()), (10, 2, (3, -1))])
def test_build_rejects_invalid(args):
    with pytest.raises(SaError) as e:
        sa_build_graph(*args)
    assert e.value.status == 1  # SA_ERR_INVALID_ARG


def test_build_rejects_unsupported():
    with pytest.raises(SaError) as e:
        sa_build_graph(2 ** 31, 4, ())
    assert e.value.status == 2
    with pytest.raises(SaError) as e:
        sa_build_graph(10 ** 6, 1, list(range(1, 70)))  # 69 kept distances > 64
    assert e.value.status == 2


# ------------------------------------------------------------------ explicit lists
def transpose_lists(T, rp, cols):
    """Reverse lists by sorting the edges on (key, query): independent of the
    library's counting pass."""
    rows = np.repeat(np.arange(T), np.diff(rp))
    order = np.lexsort((rows, cols))
    return np.concatenate([[0], np.cumsum(np.bincount(cols, minlength=T))]), rows[order]


@pytest.mark.parametrize("T,window,extra,seed", [(1, 1, 0, 1), (7, 1, 3, 2), (300, 4, 12, 3), (513, 16, 40, 4),
                                                 (64, 64, 0, 5)])
def test_csr_lists_round_trip_and_reverse(T, window, extra, seed):
    from sparse_causal_attention_amd import SA_GRAPH_CSR, sa_build_graph_csr
    from sparse_causal_attention_amd.inputs import random_causal_lists

    rp, cols = random_causal_lists(T, window, extra, seed)
    g = sa_build_graph_csr(T, rp, cols)
    assert g.kind == SA_GRAPH_CSR and g.is_csr and g.n_edges == rp[-1] and g.window == 0 and not g.dilations
    grp, gcols = g.rows()
    assert np.array_equal(grp, rp) and np.array_equal(gcols, cols)
    rrp, rcols = g.rows_reverse()
    trp, tcols = transpose_lists(T, rp, cols)
    assert np.array_equal(rrp, trp) and np.array_equal(rcols, tcols)
    a, b = T // 3, T - T // 4
    srp, scols = g.rows_reverse(a, b)
    assert np.array_equal(srp, trp[a:b + 1] - trp[a]) and np.array_equal(scols, tcols[trp[a]:trp[b]])
    pad = lambda n: (n + 255) // 256 * 256
    assert g.device_bytes() == 2 * (pad(4 * (T + 1)) + pad(4 * int(rp[-1])))


@pytest.mark.parametrize("T,W,offs", CASES[:8])
def test_csr_of_a_distance_graph_has_its_reverse(T, W, offs):
    """The window + distances graph given as lists: same rows, same reverse
    rows as the descriptor form."""
    from sparse_causal_attention_amd import sa_build_graph_csr

    orp, ocols = oracle.graph_csr(T, W, offs)
    g = sa_build_graph_csr(T, orp, ocols)
    assert g.n_edges == orp[-1]
    rrp, rcols = g.rows_reverse()
    orrp, orcols = oracle_reverse(T, W, offs)
    assert np.array_equal(rrp, orrp) and np.array_equal(rcols, orcols)


MALFORMED = [
    ("empty row", 3, [0, 1, 1, 3], [0, 1, 2]),
    ("descending", 3, [0, 1, 3, 5], [0, 1, 0, 0, 2]),
    ("duplicate", 3, [0, 1, 3, 5], [0, 0, 0, 1, 2]),
    ("looks ahead", 3, [0, 1, 3, 4], [0, 0, 2, 2]),
    ("negative key", 3, [0, 1, 2, 4], [0, -1, 0, 2]),
    ("row_ptr[0] != 0", 2, [1, 2, 4], [0, 0, 0, 1]),
    ("row_ptr decreasing", 3, [0, 2, 1, 3], [0, 0, 1]),
]


@pytest.mark.parametrize("why,T,rp,cols", MALFORMED, ids=[m[0] for m in MALFORMED])
def test_csr_rejects_what_the_oracle_rejects(why, T, rp, cols):
    from sparse_causal_attention_amd import sa_build_graph_csr

    with pytest.raises(SaError):
        sa_build_graph_csr(T, rp, cols)
    v = np.zeros((T, 4))
    with pytest.raises(ValueError):
        oracle.fwd_csr(rp, cols, v)


def test_csr_accepts_what_the_oracle_accepts_and_rejects_bad_sizes():
    from sparse_causal_attention_amd import _abi, sa_build_graph_csr

    rp, cols = [0, 1, 3, 4], [0, 0, 1, 1]  # row 2 lists only key 1
    sa_build_graph_csr(3, rp, cols)
    oracle.fwd_csr(rp, cols, np.zeros((3, 4)))
    L = _abi.lib()
    import ctypes
    h = ctypes.c_void_p()
    assert L.sa_build_graph_csr(0, None, None, ctypes.byref(h)) == _abi.SA_ERR_INVALID_ARG
    big = np.array([0, 1], dtype=np.int64)
    assert L.sa_build_graph_csr(1 << 31, big.ctypes.data, big.ctypes.data,
                                ctypes.byref(h)) == _abi.SA_ERR_UNSUPPORTED
    assert L.sa_build_graph_csr(1, big.ctypes.data, None, ctypes.byref(h)) == _abi.SA_ERR_INVALID_ARG
    assert L.sa_build_graph_csr(1, big.ctypes.data, big.ctypes.data, None) == _abi.SA_ERR_INVALID_ARG

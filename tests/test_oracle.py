"""Pins of the fp64 CPU oracle against facts fixed outside it.

Each check ties the oracle to something other than itself: a hand-worked
fixture, the pages' window predicate evaluated densely, closed-form counts,
a library routine (torch CPU fp64 scaled_dot_product_attention / autograd),
special cases with known answers, invariants of the mathematics, and central
finite differences.  A dropped term, a wrong sign or index, or a transposed
operand in oracle.c fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers
def dense_mask(T, W, offsets):
    """Dense bool [T, T] mask: the window predicate of MiniGPT Part 6's
    sliding_window_mask listing (j <= i and i - j < w), widened by the
    long-range distances of the SpatialLM-Mini graph (i - j in offsets)."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    dist = i - j
    keep = (j <= i) & (dist < W)
    for d in offsets:
        keep |= (j <= i) & (dist == d)
    return keep


def closed_form_degree(T, W, offsets, i):
    dil = sorted({d for d in offsets if W <= d < T})
    return min(i + 1, W) + sum(1 for d in dil if d <= i)


def closed_form_edges(T, W, offsets):
    Wc = min(W, T)
    dil = sorted({d for d in offsets if Wc <= d < T})
    return Wc * (Wc + 1) // 2 + Wc * (T - Wc) + sum(T - d for d in dil)


def sdpa_masked(q, k, v, mask, scale):
    """torch CPU fp64 SDPA with a boolean mask (True = attend)."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64))[None, None]
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64))[None, None]
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))[None, None]
    mt = torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    return o[0, 0].numpy()


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ graph
def test_graph_golden_fixture():
    path = os.path.join(GOLDEN, "graph_T12_W3_pow2.txt")
    rows = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("T "):
            T = int(line.split()[1])
        elif line.startswith("W "):
            W = int(line.split()[1])
        elif line.startswith("OFFSETS"):
            offs = [int(x) for x in line.split()[1:]]
        else:
            i, js = line.split(":")
            rows[int(i)] = [int(x) for x in js.split()]
    assert len(rows) == T
    rp, cols = oracle.graph_csr(T, W, offs)
    for i in range(T):
        assert list(cols[rp[i]:rp[i + 1]]) == rows[i], i
        assert list(oracle.row(T, W, offs, i)) == rows[i]


@pytest.mark.parametrize("T,W", [(1, 1), (7, 1), (16, 3), (33, 8), (64, 64), (50, 80), (129, 16)])
def test_graph_window_equals_page_predicate(T, W):
    keep = dense_mask(T, W, ())
    rp, cols = oracle.graph_csr(T, W, ())
    for i in range(T):
        assert list(cols[rp[i]:rp[i + 1]]) == list(np.nonzero(keep[i])[0]), (T, W, i)


@pytest.mark.parametrize("seed", range(12))
def test_graph_random_offsets_equal_dense_predicate(seed):
    r = rng(seed)
    T = int(r.integers(1, 300))
    W = int(r.integers(1, 40))
    n = int(r.integers(0, 12))
    offs = [int(x) for x in r.integers(0, 2 * T + 2, size=n)]  # unsorted, repeats, 0, >= T
    keep = dense_mask(T, W, offs)
    rp, cols = oracle.graph_csr(T, W, offs)
    assert rp[-1] == keep.sum()
    for i in range(T):
        assert list(cols[rp[i]:rp[i + 1]]) == list(np.nonzero(keep[i])[0])
    assert rp[-1] == closed_form_edges(T, W, offs)


@pytest.mark.parametrize("T,W,offs,E", [
    # tiny workload: window 8 + 16..128
    (256, 8, (16, 32, 64, 128), 2804),
    (256, 256, (), 32896),
    # dilated training shape: window 4 + 2^0..2^13
    (16384, 4, tuple(2 ** k for k in range(14)), 245758),
    # band: W = 256
    (16384, 256, (), 4161664),
])
def test_graph_edge_counts_closed_form(T, W, offs, E):
    assert closed_form_edges(T, W, offs) == E
    rp, _ = oracle.graph_csr(T, W, offs)
    assert rp[-1] == E
    deg = np.diff(rp)
    for i in list(range(0, min(T, 300))) + list(range(T - 50, T)):
        assert deg[i] == closed_form_degree(T, W, offs, i)


def test_graph_ultra_long_sampled_rows():
    T, W = 2 ** 26, 64
    offs = [2 ** k for k in range(6, 26)]
    r = rng(5)
    rows = list(r.integers(0, T, size=200)) + [0, 1, 63, 64, 65, 2 ** 25 - 1, 2 ** 25, 2 ** 25 + 1, T - 1]
    for i in rows:
        nb = oracle.row(T, W, offs, int(i))
        assert len(nb) == closed_form_degree(T, W, offs, int(i))
        expect = sorted({int(i) - d for d in list(range(W)) + offs if int(i) - d >= 0})
        assert list(nb) == expect
    # 5,570,033,760 edges: larger than 2^31
    assert closed_form_edges(T, W, offs) == 5570033760


def test_graph_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.graph_csr(10, 0, ())
    with pytest.raises(ValueError):
        oracle.graph_csr(10, 3, (2, -1))
    with pytest.raises(ValueError):
        oracle.row(10, 3, (), 10)


# ------------------------------------------------------------------ forward, dot
GRAPHS = [
    (1, 1, ()), (2, 1, ()), (37, 5, (8, 16, 32)), (64, 4, (1, 2, 4, 8, 16, 32)),
    (200, 8, (16, 32, 64, 128)), (129, 129, ()), (96, 200, ()), (150, 1, (3, 7, 7, 0, 500)),
]


@pytest.mark.parametrize("T,W,offs", GRAPHS)
def test_fwd_dot_matches_torch_sdpa_masked(T, W, offs):
    r = rng(T * 31 + W)
    D = 16
    q, k, v = (r.standard_normal((T, D)) for _ in range(3))
    scale = 1 / math.sqrt(D)
    O, L = oracle.fwd(T, W, offs, v, q=q, k=k)
    mask = dense_mask(T, W, offs)
    ref = sdpa_masked(q, k, v, mask, scale)
    assert np.max(np.abs(O - ref)) < 1e-12
    # LSE against the dense -inf-masked score matrix (natural log)
    s = np.where(mask, (q @ k.T) * scale, -np.inf)
    m = s.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    assert np.max(np.abs(L - lse)) < 1e-12


@pytest.mark.parametrize("T,D", [(64, 8), (256, 32), (300, 16)])
def test_fwd_full_window_is_exactly_causal(T, D):
    """W >= T returns exactly the causal-attention numbers (MiniGPT Part 6,
    claim after the chunked_swa listing): bitwise against the dense causal
    loop, and to rounding against torch's is_causal kernel."""
    r = rng(T + D)
    q, k, v = (r.standard_normal((T, D)) for _ in range(3))
    for W in (T, T + 1, 10 * T):
        O, L = oracle.fwd(T, W, (), v, q=q, k=k)
        Oc, Lc = oracle.dense_causal(q, k, v)
        assert np.array_equal(O, Oc) and np.array_equal(L, Lc)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x)[None, None] for x in (q, k, v)), is_causal=True)[0, 0].numpy()
    assert np.max(np.abs(O - ref)) < 1e-12


def test_fwd_closed_form_rows():
    r = rng(3)
    T, D, W, offs = 120, 8, 6, (8, 16, 32, 64)
    q, k, v = (r.standard_normal((T, D)) for _ in range(3))
    O, L = oracle.fwd(T, W, offs, v, q=q, k=k)
    # row 0 has the single key 0
    assert np.array_equal(O[0], v[0])
    assert L[0] == (q[0] @ k[0]) / math.sqrt(D) or abs(L[0] - (q[0] @ k[0]) / math.sqrt(D)) < 1e-15
    # q = 0: every score is 0, so O_i is the plain mean of v over N(i)
    O0, L0 = oracle.fwd(T, W, offs, v, q=np.zeros_like(q), k=k)
    mask = dense_mask(T, W, offs)
    mean = (mask.astype(np.float64) @ v) / mask.sum(axis=1, keepdims=True)
    assert np.max(np.abs(O0 - mean)) < 1e-13
    assert np.max(np.abs(L0 - np.log(mask.sum(axis=1)))) < 1e-13
    # constant values pass through unchanged
    Oc, _ = oracle.fwd(T, W, offs, np.full_like(v, 2.5), q=q, k=k)
    assert np.max(np.abs(Oc - 2.5)) < 1e-13


def test_fwd_weights_are_a_softmax_over_the_graph_rows():
    """With one-hot values v_j = e_j, O_i is row i of P: non-negative, zero
    off the graph, summing to one."""
    r = rng(4)
    T, W, offs = 40, 3, (4, 8, 16)
    q, k = r.standard_normal((T, T)), r.standard_normal((T, T))
    O, _ = oracle.fwd(T, W, offs, np.eye(T), q=q, k=k, scale=0.3)
    mask = dense_mask(T, W, offs)
    assert np.all(O[~mask] == 0.0) and np.all(O[mask] > 0.0)
    assert np.max(np.abs(O.sum(axis=1) - 1.0)) < 1e-15


def test_fwd_sampled_rows_and_dtypes():
    r = rng(6)
    T, D, W, offs = 300, 32, 8, (16, 32, 64, 128)
    x32 = [r.standard_normal((T, D)).astype(np.float32) for _ in range(3)]
    O64, L64 = oracle.fwd(T, W, offs, x32[2].astype(np.float64), q=x32[0].astype(np.float64),
                          k=x32[1].astype(np.float64))
    O32, L32 = oracle.fwd(T, W, offs, x32[2], q=x32[0], k=x32[1])
    assert np.array_equal(O64, O32) and np.array_equal(L64, L32)
    # bf16 bits: exact upcast (torch rounds fp32 -> bf16, then widens exactly)
    tb = [torch.from_numpy(x).to(torch.bfloat16) for x in x32]
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in tb]
    wide = [t.to(torch.float64).numpy() for t in tb]
    Ob, Lb = oracle.fwd(T, W, offs, bits[2], q=bits[0], k=bits[1])
    Ow, Lw = oracle.fwd(T, W, offs, wide[2], q=wide[0], k=wide[1])
    assert np.array_equal(Ob, Ow) and np.array_equal(Lb, Lw)
    rows = [299, 0, 17, 128, 5]
    Os, Ls = oracle.fwd(T, W, offs, x32[2], q=x32[0], k=x32[1], rows=rows)
    assert np.array_equal(Os, O32[rows]) and np.array_equal(Ls, L32[rows])


# ------------------------------------------------------------------ forward, coordinates
def test_fwd_coord_reduces_to_dot_product_sdpa():
    """-gamma||cq - ck||^2 + beta = <[cq, 1], [2 gamma ck, -gamma||ck||^2]>
    + (-gamma||cq||^2 + beta); the last term is constant per row, so the
    weights equal scale-1 SDPA on the augmented 4-vectors."""
    r = rng(7)
    T, D, W, offs = 180, 16, 5, (8, 16, 32, 64, 128)
    cq, ck, v = r.standard_normal((T, 3)), r.standard_normal((T, 3)), r.standard_normal((T, D))
    gamma, beta = 1.3, -0.07
    O, L = oracle.fwd(T, W, offs, v, cq=cq, ck=ck, gamma=gamma, beta=beta)
    qa = np.concatenate([cq, np.ones((T, 1))], axis=1)
    ka = np.concatenate([2 * gamma * ck, -gamma * (ck ** 2).sum(1, keepdims=True)], axis=1)
    mask = dense_mask(T, W, offs)
    ref = sdpa_masked(qa, ka, v, mask, 1.0)
    assert np.max(np.abs(O - ref)) < 1e-12
    s = np.where(mask, qa @ ka.T, -np.inf)
    m = s.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    lse += -gamma * (cq ** 2).sum(1) + beta
    assert np.max(np.abs(L - lse)) < 1e-11


def test_fwd_coord_invariants():
    r = rng(8)
    T, D, W, offs = 90, 8, 4, (4, 8, 16, 32, 64)
    cq, ck, v = r.standard_normal((T, 3)), r.standard_normal((T, 3)), r.standard_normal((T, D))
    O1, L1 = oracle.fwd(T, W, offs, v, cq=cq, ck=ck, gamma=0.8, beta=0.0)
    O2, L2 = oracle.fwd(T, W, offs, v, cq=cq, ck=ck, gamma=0.8, beta=0.37)
    assert np.max(np.abs(O1 - O2)) < 1e-14       # beta cancels in the softmax
    assert np.max(np.abs(L2 - L1 - 0.37)) < 1e-14  # and shifts LSE
    # translating both coordinate sets leaves every score unchanged
    O3, L3 = oracle.fwd(T, W, offs, v, cq=cq + 5.0, ck=ck + 5.0, gamma=0.8, beta=0.0)
    assert np.max(np.abs(O3 - O1)) < 1e-11 and np.max(np.abs(L3 - L1)) < 1e-11
    # gamma = 0: uniform weights over N(i)
    O0, _ = oracle.fwd(T, W, offs, v, cq=cq, ck=ck, gamma=0.0, beta=0.2)
    mask = dense_mask(T, W, offs)
    mean = (mask.astype(np.float64) @ v) / mask.sum(axis=1, keepdims=True)
    assert np.max(np.abs(O0 - mean)) < 1e-13
    # nearer keys weigh more: with gamma > 0 and one key at the query's point,
    # that key gets the largest weight in the row
    i = 70
    ck2 = ck.copy()
    nb = oracle.row(T, W, offs, i)
    ck2[nb[1]] = cq[i]
    Oe, _ = oracle.fwd(T, W, offs, np.eye(T), cq=cq, ck=ck2, gamma=1.0, beta=0.0, rows=[i])
    assert int(np.argmax(Oe[0])) == nb[1]


# ------------------------------------------------------------------ backward
def torch_masked_attention(mask, v, q=None, k=None, cq=None, ck=None, gamma=None, beta=None,
                           scale=None):
    """Differentiable fp64 dense formulation (torch CPU autograd)."""
    m = torch.from_numpy(mask)
    if cq is not None:
        diff = cq[:, None, :] - ck[None, :, :]
        s = -gamma * (diff ** 2).sum(-1) + beta
    else:
        s = (q @ k.T) * scale
    s = s.masked_fill(~m, float("-inf"))
    return torch.softmax(s, dim=-1) @ v


@pytest.mark.parametrize("T,W,offs", [(64, 3, (4, 8, 16, 32)), (128, 128, ()), (100, 1, (1, 2, 4, 8, 16, 32, 64)),
                                      (97, 9, (16, 32, 64))])
def test_bwd_dot_matches_torch_autograd(T, W, offs):
    r = rng(T + 100 * W)
    D = 16
    q, k, v, dO = (r.standard_normal((T, D)) for _ in range(4))
    scale = 1 / math.sqrt(D)
    g = oracle.bwd(T, W, offs, v, dO, q=q, k=k)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch_masked_attention(dense_mask(T, W, offs), tv, q=tq, k=tk, scale=scale)
    out.backward(torch.from_numpy(dO))
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert np.max(np.abs(g[name] - t.grad.numpy())) < 1e-12, name


def test_bwd_coord_matches_torch_autograd():
    r = rng(11)
    T, D, W, offs = 120, 8, 4, (4, 8, 16, 32, 64)
    cq, ck, v, dO = r.standard_normal((T, 3)), r.standard_normal((T, 3)), r.standard_normal((T, D)), \
        r.standard_normal((T, D))
    gamma, beta = 0.9, 0.05
    g = oracle.bwd(T, W, offs, v, dO, cq=cq, ck=ck, gamma=gamma, beta=beta)
    tcq, tck, tv = (torch.tensor(x, requires_grad=True) for x in (cq, ck, v))
    tg = torch.tensor(gamma, dtype=torch.float64, requires_grad=True)
    tb = torch.tensor(beta, dtype=torch.float64, requires_grad=True)
    out = torch_masked_attention(dense_mask(T, W, offs), tv, cq=tcq, ck=tck, gamma=tg, beta=tb)
    out.backward(torch.from_numpy(dO))
    assert np.max(np.abs(g["dcq"] - tcq.grad.numpy())) < 1e-12
    assert np.max(np.abs(g["dck"] - tck.grad.numpy())) < 1e-12
    assert np.max(np.abs(g["dv"] - tv.grad.numpy())) < 1e-12
    assert abs(g["dgamma"] - tg.grad.item()) < 1e-11
    assert abs(g["dbeta"] - tb.grad.item()) < 1e-12


def _loss_dot(T, W, offs, q, k, v, dO, scale):
    O, _ = oracle.fwd(T, W, offs, v, q=q, k=k, scale=scale)
    return float((O * dO).sum())


def _loss_coord(T, W, offs, cq, ck, v, dO, gamma, beta):
    O, _ = oracle.fwd(T, W, offs, v, cq=cq, ck=ck, gamma=gamma, beta=beta)
    return float((O * dO).sum())


def _fd_check(f, x, grad, tol=1e-6):
    flat = x.reshape(-1)
    gflat = grad.reshape(-1)
    for idx in range(flat.size):
        x0 = flat[idx]
        h = 1e-6 * max(1.0, abs(x0))
        flat[idx] = x0 + h
        fp = f()
        flat[idx] = x0 - h
        fm = f()
        flat[idx] = x0
        fd = (fp - fm) / (2 * h)
        assert abs(fd - gflat[idx]) <= tol * max(1.0, abs(fd)), (idx, fd, gflat[idx])


def test_bwd_dot_finite_differences():
    r = rng(12)
    T, D, W, offs = 40, 6, 3, (4, 8, 16, 32)
    scale = 0.45
    q, k, v, dO = (r.standard_normal((T, D)) for _ in range(4))
    g = oracle.bwd(T, W, offs, v, dO, q=q, k=k, scale=scale)
    f = lambda: _loss_dot(T, W, offs, q, k, v, dO, scale)  # noqa: E731
    _fd_check(f, q, g["dq"])
    _fd_check(f, k, g["dk"])
    _fd_check(f, v, g["dv"])


def test_bwd_coord_finite_differences():
    r = rng(13)
    T, D, W, offs = 40, 5, 2, (2, 4, 8, 16, 32)
    cq, ck, v, dO = r.standard_normal((T, 3)), r.standard_normal((T, 3)), r.standard_normal((T, D)), \
        r.standard_normal((T, D))
    par = np.array([1.1, 0.2])  # gamma, beta
    g = oracle.bwd(T, W, offs, v, dO, cq=cq, ck=ck, gamma=par[0], beta=par[1])
    f = lambda: _loss_coord(T, W, offs, cq, ck, v, dO, par[0], par[1])  # noqa: E731
    _fd_check(f, cq, g["dcq"])
    _fd_check(f, ck, g["dck"])
    _fd_check(f, v, g["dv"])
    _fd_check(f, par, np.array([g["dgamma"], g["dbeta"]]))


def test_bwd_invariants():
    r = rng(14)
    T, D, W, offs = 300, 16, 8, (16, 32, 64, 128)
    q, k, v, dO = (r.standard_normal((T, D)) for _ in range(4))
    g = oracle.bwd(T, W, offs, v, dO, q=q, k=k)
    # each row of P sums to one, so sum_j dV_j = sum_i dO_i
    assert np.max(np.abs(g["dv"].sum(0) - dO.sum(0))) < 1e-11
    # scores are invariant under q -> a q, k -> k / a, hence sum <q,dQ> = sum <k,dK>
    assert abs((q * g["dq"]).sum() - (k * g["dk"]).sum()) < 1e-10
    cq, ck = r.standard_normal((T, 3)), r.standard_normal((T, 3))
    gamma = 1.4
    gc = oracle.bwd(T, W, offs, v, dO, cq=cq, ck=ck, gamma=gamma, beta=0.3)
    # translation invariance of the distance score
    assert np.max(np.abs(gc["dcq"].sum(0) + gc["dck"].sum(0))) < 1e-11
    # beta cancels in the softmax
    assert abs(gc["dbeta"]) < 1e-11
    # scaling all coordinates by a equals scaling gamma by a^2
    lhs = (cq * gc["dcq"]).sum() + (ck * gc["dck"]).sum()
    assert abs(lhs - 2 * gamma * gc["dgamma"]) < 1e-10


def test_bwd_bf16_inputs_upcast_exactly():
    r = rng(15)
    T, D, W, offs = 70, 8, 4, (4, 8, 16, 32, 64)
    xs = [torch.from_numpy(r.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16) for _ in range(4)]
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in xs]
    wide = [t.to(torch.float64).numpy() for t in xs]
    gb = oracle.bwd(T, W, offs, bits[2], bits[3], q=bits[0], k=bits[1])
    gw = oracle.bwd(T, W, offs, wide[2], wide[3], q=wide[0], k=wide[1])
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(gb[key], gw[key])


# ------------------------------------------------------------------ uniform score mode
def neighbours_from_definition(T, W, offsets, i):
    """N(i) straight from the definition: itself and the W - 1 predecessors,
    plus i - d for every long-range distance d, never before row 0."""
    return sorted({i - d for d in range(W) if i - d >= 0} | {i - d for d in offsets if 0 <= i - d})


@pytest.mark.parametrize("T,W,offs", [(64, 4, (4, 8, 16, 32)), (97, 1, (1, 2, 4, 8, 16, 32, 64)),
                                      (40, 8, ()), (33, 50, (3, 40))])
def test_fwd_uniform_is_the_neighbour_mean(T, W, offs):
    """Equal weights over each row's neighbour list: O_i is the arithmetic
    mean of the neighbours' v rows and LSE_i = ln |N(i)|, |N(i)| from the
    closed-form degree."""
    rng = np.random.default_rng(T * 7 + W)
    v = rng.standard_normal((T, 6))
    O, L = oracle.fwd(T, W, offs, v)
    for i in range(T):
        nb = neighbours_from_definition(T, W, offs, i)
        np.testing.assert_allclose(O[i], v[nb].mean(axis=0), rtol=0, atol=1e-13)
        assert len(nb) == closed_form_degree(T, W, offs, i)
        assert abs(L[i] - math.log(len(nb))) < 1e-14


def test_bwd_uniform_is_the_reverse_graph_sum():
    """dV_j = sum over the rows i that list j of dO_i / |N(i)|; nothing else
    is returned (the mode has no score parameters)."""
    T, W, offs = 77, 3, (4, 8, 16, 32, 64)
    rng = np.random.default_rng(5)
    v = rng.standard_normal((T, 5))
    dO = rng.standard_normal((T, 5))
    g = oracle.bwd(T, W, offs, v, dO)
    assert sorted(g) == ["dv"]
    nbs = [neighbours_from_definition(T, W, offs, i) for i in range(T)]
    ref = np.zeros((T, 5))
    for i, nb in enumerate(nbs):
        for j in nb:
            ref[j] += dO[i] / len(nb)
    np.testing.assert_allclose(g["dv"], ref, rtol=0, atol=1e-13)
    # the forward is linear in v: <dO, O(v + e)> - <dO, O(v)> = <dV, e> exactly
    e = rng.standard_normal((T, 5))
    O0, _ = oracle.fwd(T, W, offs, v)
    O1, _ = oracle.fwd(T, W, offs, v + e)
    assert abs(np.sum(dO * (O1 - O0)) - np.sum(g["dv"] * e)) < 1e-11


def test_fwd_uniform_equals_dot_mode_with_zero_queries():
    """With q = 0 every dot-product score is 0, so dot mode reduces to the
    uniform mode on the same graph."""
    T, W, offs = 50, 4, (8, 16)
    rng = np.random.default_rng(9)
    v = rng.standard_normal((T, 8))
    k = rng.standard_normal((T, 8))
    O_u, L_u = oracle.fwd(T, W, offs, v)
    O_d, L_d = oracle.fwd(T, W, offs, v, q=np.zeros((T, 8)), k=k)
    np.testing.assert_allclose(O_u, O_d, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L_u, L_d, rtol=0, atol=1e-14)


# ------------------------------------------------------------------ explicit (CSR) graphs
def random_causal_csr(T, max_deg, seed):
    """Row i: itself plus up to max_deg - 1 distinct earlier keys, ascending."""
    rng = np.random.default_rng(seed)
    rp, cols = [0], []
    for i in range(T):
        others = rng.choice(i, size=min(i, int(rng.integers(0, max_deg))), replace=False) if i else []
        row = sorted(set(int(j) for j in others) | {i})
        cols += row
        rp.append(len(cols))
    return np.array(rp), np.array(cols)


def csr_mask(T, rp, cols):
    m = np.zeros((T, T), dtype=bool)
    for i in range(T):
        m[i, cols[rp[i]:rp[i + 1]]] = True
    return m


@pytest.mark.parametrize("T,deg,seed", [(60, 5, 1), (97, 12, 2), (33, 40, 3)])
def test_fwd_csr_matches_torch_sdpa_masked(T, deg, seed):
    """Any causal neighbour list: torch fp64 scaled_dot_product_attention with
    the graph as a boolean mask."""
    rp, cols = random_causal_csr(T, deg, seed)
    rng = np.random.default_rng(seed + 10)
    D = 8
    q, k, v = (rng.standard_normal((T, D)) for _ in range(3))
    O, L = oracle.fwd_csr(rp, cols, v, q=q, k=k)
    mask = torch.from_numpy(csr_mask(T, rp, cols))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], attn_mask=mask[None])
    np.testing.assert_allclose(O, ref[0].numpy(), rtol=0, atol=1e-12)
    s = (q @ k.T) / math.sqrt(D)
    s[~mask.numpy()] = -np.inf
    np.testing.assert_allclose(L, np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1), rtol=0,
                               atol=1e-12)


def test_bwd_csr_matches_torch_autograd():
    T, D = 70, 6
    rp, cols = random_causal_csr(T, 9, 4)
    rng = np.random.default_rng(14)
    q, k, v, dO = (rng.standard_normal((T, D)) for _ in range(4))
    g = oracle.bwd_csr(rp, cols, v, dO, q=q, k=k)
    mask = torch.from_numpy(csr_mask(T, rp, cols))
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None], attn_mask=mask[None])
    (o[0] * torch.from_numpy(dO)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        np.testing.assert_allclose(g[name], t.grad.numpy(), rtol=0, atol=1e-11)
    # uniform mode on the same lists: dV_j = sum over the rows i listing j of dO_i / |N(i)|
    gu = oracle.bwd_csr(rp, cols, v, dO)
    ref = np.zeros((T, D))
    for i in range(T):
        row = cols[rp[i]:rp[i + 1]]
        ref[row] += dO[i] / len(row)
    np.testing.assert_allclose(gu["dv"], ref, rtol=0, atol=1e-13)


def test_csr_of_the_distance_graph_reproduces_it():
    T, W, offs = 80, 3, (4, 8, 16, 32, 64)
    rp, cols = oracle.graph_csr(T, W, offs)
    rng = np.random.default_rng(21)
    q, k, v, dO = (rng.standard_normal((T, 8)) for _ in range(4))
    O1, L1 = oracle.fwd_csr(rp, cols, v, q=q, k=k)
    O2, L2 = oracle.fwd(T, W, offs, v, q=q, k=k)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)
    g1, g2 = oracle.bwd_csr(rp, cols, v, dO, q=q, k=k), oracle.bwd(T, W, offs, v, dO, q=q, k=k)
    for key in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(g1[key], g2[key])


@pytest.mark.parametrize("rp,cols", [
    ([0, 1, 2], [0, 2]),        # key after the query
    ([0, 1, 3], [0, 1, 0]),     # not ascending
    ([0, 1, 3], [0, 1, 1]),     # repeated key
    ([0, 1, 1], [0]),           # empty row
    ([1, 2, 3], [0, 1, 1]),     # row_ptr not starting at 0
])
def test_csr_rejects_malformed_lists(rp, cols):
    v = np.zeros((2, 4))
    with pytest.raises(ValueError):
        oracle.fwd_csr(rp, cols, v)

"""HIP path against the fp64 oracle, element by element, through the C ABI.

Tolerances (max-abs over every output element): 1e-4 for fp32 inputs and
2e-2 for bf16 inputs with fp32 accumulation.  The per-head coordinate-score
parameter gradients (sums over up to 8M edges) use
|err| <= max(tol, 1e-6 * sum_edges |dS| (1 + ||c_q - c_k||^2)).
Gradients requested in bf16 are rounded once more, to nearest even, after
the fp32 computation: each element may differ from the oracle by the tolerance
plus half a bf16 unit in the last place at the magnitude the fp32 result can
have, |g| + tol (see bf16_stored_excess).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from sparse_causal_attention_amd import (sa_build_graph, sa_build_graph_csr, sa_bwd, sa_decode, sa_describe_plan,
                                        sa_fwd)
from sparse_causal_attention_amd.inputs import (WORKLOADS, Workload, host_view, make_device_inputs_chunked,
                                                make_inputs, random_causal_lists, sample_rows, workload_lists)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print("\n[parity] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from sparse_causal_attention_amd import _abi
    _abi.lib()  # loud failure when libsa.so is missing


def tol_of(w_dtype):
    return 1e-4 if w_dtype == torch.float32 else 2e-2


def maxabs(t, ref):
    return float(np.max(np.abs(t.detach().double().cpu().numpy() - ref))) if ref.size else 0.0


def bf16_half_ulp(x):
    """Half a bf16 unit in the last place at magnitude |x| (8 significant
    bits: for |x| in [2^e, 2^(e+1)) the unit is 2^(e-7)); 0 at 0."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(ax)  # ax = f * 2^e with f in [0.5, 1): binade 2^(e-1)
    return np.where(ax > 0, np.ldexp(1.0, e - 9), 0.0)


def bf16_stored_excess(t, ref, tol):
    """Largest error of a bf16-stored result beyond its final rounding: the
    kernel computes g in fp32 within tol of the oracle's value ref, then
    stores RNE(g), which moves it by at most half a bf16 ulp of |g| <= |ref| + tol.
    Returns max(|t - ref| - half_ulp(|ref| + tol)), to be compared with tol."""
    if not ref.size:
        return 0.0
    err = np.abs(t.detach().double().cpu().numpy() - ref)
    return float(np.max(err - bf16_half_ulp(np.abs(ref) + tol)))


def grad_err(t, ref, tol, grad_dtype):
    """Max-abs error of a gradient; for bf16-stored gradients, the error
    beyond the final rounding (bf16_stored_excess)."""
    if grad_dtype == torch.bfloat16:
        assert t.dtype == torch.bfloat16
        return bf16_stored_excess(t, ref, tol)
    return maxabs(t, ref)


def run_and_compare(w: Workload, algo="auto", backward=True, grad_dtype=None, **shape):
    x = make_inputs(w, device="cpu", backward=backward, **shape)
    B, H, T, D = x["v"].shape
    g = sa_build_graph(T, w.window, w.offsets)
    xd = {k: v.to(DEV) for k, v in x.items()}
    score = "coord" if w.coord else ("uniform" if w.uniform else "dot")
    _say("%s algo=%s shape=%s plan=%s" % (w.name, algo, (B, H, T, D),
                                          sa_describe_plan(g, xd["v"], score=score, algo=algo)))
    if w.coord:
        o, lse = sa_fwd(g, v=xd["v"], cq=xd["cq"], ck=xd["ck"], gamma=xd["gamma"], beta=xd["beta"],
                        algo=algo)
    elif w.uniform:
        o, lse = sa_fwd(g, v=xd["v"], algo=algo)
    else:
        o, lse = sa_fwd(g, xd["q"], xd["k"], xd["v"], algo=algo)
    torch.cuda.synchronize()
    hv = {k: host_view(v) for k, v in x.items()}
    tol = tol_of(w.dtype)
    if w.coord:
        O, L = oracle.fwd_bh(w.window, w.offsets, hv["v"], cq=hv["cq"], ck=hv["ck"], gamma=hv["gamma"],
                             beta=hv["beta"])
    elif w.uniform:
        O, L = oracle.fwd_bh(w.window, w.offsets, hv["v"])
    else:
        O, L = oracle.fwd_bh(w.window, w.offsets, hv["v"], q=hv["q"], k=hv["k"])
    errs = {"o": maxabs(o, O), "lse": maxabs(lse, L)}
    if backward:
        if w.coord:
            gr = sa_bwd(g, v=xd["v"], o=o, lse=lse, dout=xd["do"], cq=xd["cq"], ck=xd["ck"],
                        gamma=xd["gamma"], beta=xd["beta"], algo=algo, grad_dtype=grad_dtype)
            ref = oracle.bwd_bh(w.window, w.offsets, hv["v"], hv["do"], cq=hv["cq"], ck=hv["ck"],
                                gamma=hv["gamma"], beta=hv["beta"])
            torch.cuda.synchronize()
            for key in ("dv", "dcq", "dck"):
                errs[key] = grad_err(gr[key], ref[key], tol, grad_dtype if key == "dv" else None)
            for key in ("dgamma", "dbeta"):
                err = np.abs(gr[key].double().cpu().numpy() - ref[key])
                bound = np.maximum(tol, 1e-6 * ref["l1"])
                errs[key] = float(np.max(err / bound)) * tol  # scaled so that <= tol passes
        elif w.uniform:
            gr = sa_bwd(g, v=xd["v"], o=o, lse=lse, dout=xd["do"], algo=algo, grad_dtype=grad_dtype)
            ref = oracle.bwd_bh(w.window, w.offsets, hv["v"], hv["do"])
            torch.cuda.synchronize()
            assert sorted(gr) == ["dv"]
            errs["dv"] = grad_err(gr["dv"], ref["dv"], tol, grad_dtype)
        else:
            gr = sa_bwd(g, xd["q"], xd["k"], xd["v"], o, lse, xd["do"], algo=algo, grad_dtype=grad_dtype)
            ref = oracle.bwd_bh(w.window, w.offsets, hv["v"], hv["do"], q=hv["q"], k=hv["k"])
            torch.cuda.synchronize()
            for key in ("dq", "dk", "dv"):
                errs[key] = grad_err(gr[key], ref[key], tol, grad_dtype)
    _say("%s errors %s (tol %g%s)" % (w.name, {k: "%.2e" % v for k, v in errs.items()}, tol,
                                      ", gradient errors beyond their bf16 rounding"
                                      if grad_dtype == torch.bfloat16 else ""))
    for key, e in errs.items():
        assert e <= tol, (w.name, key, e)
    return o, lse


# ------------------------------------------------------------------ the workloads
@pytest.mark.parametrize("name", ["tiny", "tiny_dense"])
def test_tiny_fp32(name):
    run_and_compare(WORKLOADS[name])


def test_tiny_dense_equals_causal():
    w = WORKLOADS["tiny_dense"]
    x = make_inputs(w, backward=False)
    g = sa_build_graph(w.T, w.T, ())
    o, lse = sa_fwd(g, *(x[k].to(DEV) for k in ("q", "k", "v")))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(x[k].double() for k in ("q", "k", "v")), is_causal=True)
    assert float((o.cpu().double() - ref).abs().max()) <= 1e-4


@pytest.mark.parametrize("algo", ["auto", "gather"])
def test_band_full_size(algo):
    run_and_compare(WORKLOADS["band"], algo=algo)


@pytest.mark.parametrize("algo", ["auto", "gather"])
def test_band_dense_full_size(algo):
    run_and_compare(WORKLOADS["band_dense"], algo=algo)


def test_dilated_full_size():
    run_and_compare(WORKLOADS["dilated"])


def test_coord_full_size():
    run_and_compare(WORKLOADS["coord"])


def test_coord_band_graph():
    run_and_compare(WORKLOADS["coord_band"])


def test_dilated_bf16_gradients():
    run_and_compare(WORKLOADS["dilated"], grad_dtype=torch.bfloat16, B=1, H=4)


def test_band_bf16_gradients_full_size():
    """The band kernels' bf16-gradient path (the bench's band_bf16grad
    workload) on every element of the full-size band workload."""
    run_and_compare(WORKLOADS["band_bf16grad"], grad_dtype=torch.bfloat16)


def test_ultra_long_sampled_rows():
    w = WORKLOADS["ultra"]
    _say("ultra: generating %d x %d bf16 inputs on device" % (w.T, w.D))
    x = make_device_inputs_chunked(w, DEV)
    g = sa_build_graph(w.T, w.window, w.offsets)
    _say("ultra: plan %s" % sa_describe_plan(g, x["v"]))
    o, lse = sa_fwd(g, x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    rows = sample_rows(w, 4096, boundary=[0, 1, 63, 64, 65, 2 ** 25 - 1, 2 ** 25, 2 ** 25 + 1, w.T - 1])
    # host copies hold only the rows the sampled queries touch (lazy zero pages elsewhere)
    need = set()
    for i in rows.tolist():
        need.update(oracle.row(w.T, w.window, w.offsets, i).tolist())
    need = torch.tensor(sorted(need | set(rows.tolist())), dtype=torch.int64)
    host = {}
    for name in ("q", "k", "v"):
        arr = np.zeros((w.T, w.D), dtype=np.uint16)
        arr[need.numpy()] = host_view(x[name][0, 0].index_select(0, need.to(DEV)))
        host[name] = arr
    O, L = oracle.fwd(w.T, w.window, w.offsets, host["v"], q=host["q"], k=host["k"], rows=rows.numpy())
    og = o[0, 0].index_select(0, rows.to(DEV))
    lg = lse[0, 0].index_select(0, rows.to(DEV))
    eo, el = maxabs(og, O), maxabs(lg, L)
    _say("ultra: %d rows, errors o %.2e lse %.2e" % (len(rows), eo, el))
    assert eo <= 2e-2 and el <= 2e-2
    del x, o, lse
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ shapes and edge cases
RAGGED = [
    (1, 1, 1, 16, torch.float32, 1, ()),
    (2, 3, 17, 32, torch.float32, 4, (4, 8, 16)),
    (1, 2, 1000, 64, torch.bfloat16, 4, tuple(2 ** k for k in range(10))),
    (1, 1, 4097, 64, torch.bfloat16, 256, (512, 1024, 2048)),
    (2, 2, 333, 128, torch.float32, 9, (16, 32, 64, 128, 256)),
    (1, 3, 257, 128, torch.bfloat16, 40, (64, 128)),
    (3, 1, 95, 16, torch.bfloat16, 200, ()),
    (1, 1, 4097, 64, torch.bfloat16, 5000, ()),
]


@pytest.mark.parametrize("B,H,T,D,dt,W,offs", RAGGED)
def test_ragged_shapes(B, H, T, D, dt, W, offs):
    w = Workload("ragged", 9, B, H, T, D, dt, W, offs)
    run_and_compare(w)


# Windows narrower than a 64-key tile, forced onto the band kernels (the call
# fails if they do not apply): a 32 x 32 block of keys and queries can then
# cross both bounds of the window at once, and a wavefront's first and
# diagonal blocks are the same or adjacent -- the two-sided mask case of the
# forward, the dq units and the dk/dv units.
@pytest.mark.parametrize("T,W,offs", [
    (300, 16, ()),
    (517, 17, (64, 256)),
    (1000, 31, ()),
    (777, 33, (40, 100, 500)),
    (1200, 63, ()),
    (16, 16, ()),          # the smallest band graph: T = W = 16
    (40, 16, (32,)),       # shorter than one tile, one long-range distance
    (100, 5000, ()),       # window far past T: dense causal
])
def test_band_narrow_windows(T, W, offs):
    w = Workload("band_narrow", 13, 2, 2, T, 64, torch.bfloat16, W, offs)
    run_and_compare(w, algo="band")


@pytest.mark.parametrize("B,H,T,D,dt,W,offs", [
    (2, 3, 300, 32, torch.float32, 3, (4, 8, 16, 32, 64, 128)),
    (1, 2, 1000, 64, torch.bfloat16, 4, tuple(2 ** k for k in range(10))),
    (1, 1, 129, 128, torch.bfloat16, 300, ()),
    (3, 1, 1, 16, torch.float32, 1, ()),
])
def test_uniform_small(B, H, T, D, dt, W, offs):
    w = Workload("uniform_small", 6, B, H, T, D, dt, W, offs, uniform=True)
    run_and_compare(w)


def test_uniform_full_size():
    run_and_compare(WORKLOADS["uniform"])


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_coord_small(dt):
    w = Workload("coord_small", 8, 2, 3, 300, 32, dt, 3, (4, 8, 16, 32, 64, 128), coord=True)
    run_and_compare(w)


@pytest.mark.parametrize("T, D", [(300, 64), (77, 128), (16, 64)])
def test_coord_two_fragments_per_lane(T, D):
    """The coordinate score on bf16 rows of 64 and 128 elements (two 16-byte
    fragments per lane, whole-row output stores after a cross-half swap), with
    ragged last wavefronts: rows past T are neither stored nor mixed into
    stored rows."""
    w = Workload("coord_wide", 8, 2, 3, T, D, torch.bfloat16, 5, (8, 16, 32, 64), coord=True)
    run_and_compare(w)


@pytest.mark.parametrize("W,kernels", [(6, "gather"), (64, "band")])
def test_strided_inputs(W, kernels):
    """q, k, v, dout as [B, T, H, D] storage viewed as [B, H, T, D] (row
    stride H D), on the gather kernels (W = 6) and on the band kernels
    (W = 64), both with long-range distances."""
    B, H, T, D, offs = 2, 4, 777, 64, (8, 16, 32, 64, 128, 256)
    gen = torch.Generator().manual_seed(77)
    base = {n: torch.randn((B, T, H, D), generator=gen).to(torch.bfloat16) for n in ("q", "k", "v", "do")}
    xd = {n: t.to(DEV).permute(0, 2, 1, 3) for n, t in base.items()}
    g = sa_build_graph(T, W, offs)
    for which in ("fwd", "bwd"):
        assert sa_describe_plan(g, xd["v"], which=which).startswith(kernels), which
    o, lse = sa_fwd(g, xd["q"], xd["k"], xd["v"])
    gr = sa_bwd(g, xd["q"], xd["k"], xd["v"], o, lse, xd["do"])
    hv = {n: host_view(t.permute(0, 2, 1, 3).contiguous()) for n, t in base.items()}
    O, L = oracle.fwd_bh(W, offs, hv["v"], q=hv["q"], k=hv["k"])
    ref = oracle.bwd_bh(W, offs, hv["v"], hv["do"], q=hv["q"], k=hv["k"])
    assert maxabs(o, O) <= 2e-2 and maxabs(lse, L) <= 2e-2
    for key in ("dq", "dk", "dv"):
        assert maxabs(gr[key], ref[key]) <= 2e-2, key


@pytest.mark.parametrize("W,offs,kernels", [(4, tuple(2 ** k for k in range(14)), "gather"),
                                             (256, (), "band"), (64, (128, 1024), "band")])
def test_row_zero_identity_and_determinism(W, offs, kernels):
    """Row 0 (one key) returns v_0 exactly; forward and backward are bitwise
    identical from run to run (no atomics, fixed summation order), on the
    gather kernels and on the band kernels (persistent backward)."""
    w = WORKLOADS["dilated"]
    x = {k: v.to(DEV) for k, v in make_inputs(w, B=1, H=2, T=4096).items()}
    g = sa_build_graph(4096, W, offs)
    for which in ("fwd", "bwd"):
        assert sa_describe_plan(g, x["v"], which=which).startswith(kernels), which
    o1, l1 = sa_fwd(g, x["q"], x["k"], x["v"])
    o2, l2 = sa_fwd(g, x["q"], x["k"], x["v"])
    # row 0 has one key: o_0 = v_0 exactly, lse_0 = s_00
    assert torch.equal(o1[:, :, 0], x["v"][:, :, 0])
    s00 = (x["q"][:, :, 0].float() * x["k"][:, :, 0].float()).sum(-1) / 8.0
    assert float((l1[:, :, 0] - s00).abs().max()) < 1e-5
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = sa_bwd(g, x["q"], x["k"], x["v"], o1, l1, x["do"])
    g2 = sa_bwd(g, x["q"], x["k"], x["v"], o1, l1, x["do"])
    for key in ("dq", "dk", "dv"):
        assert torch.equal(g1[key], g2[key]), key


@pytest.mark.parametrize("W,offs,kernels", [(4, (4, 8, 16, 32, 64), "gather"), (256, (), "band"),
                                             (64, (100, 700), "band")])
def test_outputs_stay_in_bounds(W, offs, kernels):
    """Canaries around every output: nothing outside the tensors is written
    (T = 1001 is not a multiple of any row block or tile)."""
    B, H, T, D = 1, 2, 1001, 64
    x = {k: v.to(DEV) for k, v in make_inputs(WORKLOADS["dilated"], B=B, H=H, T=T).items()}
    g = sa_build_graph(T, W, offs)
    for which in ("fwd", "bwd"):
        assert sa_describe_plan(g, x["v"], which=which).startswith(kernels), which
    n = B * H * T * D
    pad = 4096
    canary = -1536.0  # exact in bf16 and fp32

    def guarded(numel, dtype):
        buf = torch.full((numel + 2 * pad,), canary, dtype=dtype, device=DEV)
        return buf, buf[pad:pad + numel]

    ob, o = guarded(n, torch.bfloat16)
    lb, lse = guarded(B * H * T, torch.float32)
    sa_fwd(g, x["q"], x["k"], x["v"], o=o.view(B, H, T, D), lse=lse.view(B, H, T))
    grads = {}
    bufs = {}
    for key in ("dq", "dk", "dv"):
        bufs[key], grads[key] = guarded(n, torch.float32)
    sa_bwd(g, x["q"], x["k"], x["v"], o.view(B, H, T, D), lse.view(B, H, T), x["do"],
           dq=grads["dq"].view(B, H, T, D), dk=grads["dk"].view(B, H, T, D), dv=grads["dv"].view(B, H, T, D))
    torch.cuda.synchronize()
    for buf in [ob, lb] + list(bufs.values()):
        assert bool((buf[:pad].float() == canary).all()) and bool((buf[-pad:].float() == canary).all())


# ------------------------------------------------------------------ decode step
def decode_reference(W, offs, pos, v, q=None, k=None, cq=None, ck=None, gamma=None, beta=None):
    """Oracle forward of row pos[b] of each (b, h) slice, the new token's query
    placed at that row."""
    B, H, T, D = v.shape
    O = np.empty((B, H, D))
    L = np.empty((B, H))
    for b in range(B):
        t = int(pos[b])
        for h in range(H):
            if cq is not None:
                cqf = np.zeros((T, 3))
                cqf[t] = cq[b, h]
                o, l_ = oracle.fwd(T, W, offs, v[b, h], cq=cqf, ck=ck[b, h], gamma=float(gamma[h]),
                                   beta=float(beta[h]), rows=[t])
            elif q is None:
                o, l_ = oracle.fwd(T, W, offs, v[b, h], rows=[t])
            else:
                qf = np.zeros((T, D), dtype=q.dtype)
                qf[t] = q[b, h]
                o, l_ = oracle.fwd(T, W, offs, v[b, h], q=qf, k=k[b, h], rows=[t])
            O[b, h], L[b, h] = o[0], l_[0]
    return O, L


@pytest.mark.parametrize("score,dt,D,W,offs", [
    ("dot", torch.bfloat16, 64, 64, tuple(2 ** k for k in range(6, 12))),
    ("dot", torch.float32, 32, 4, tuple(2 ** k for k in range(12))),
    ("dot", torch.bfloat16, 128, 300, ()),
    ("coord", torch.bfloat16, 64, 4, tuple(2 ** k for k in range(12))),
    ("uniform", torch.float32, 16, 8, (16, 32, 64, 1024)),
])
def test_decode_matches_oracle_rows(score, dt, D, W, offs):
    B, H, T = 6, 3, 3000
    pos = np.array([0, 1, W - 1 if W > 1 else 2, 1500, 2047, T - 1], dtype=np.int32)[:B]
    gen = torch.Generator().manual_seed(4242 + D)
    v = torch.randn((B, H, T, D), generator=gen).to(dt)
    g = sa_build_graph(T, W, offs)
    posd = torch.from_numpy(pos).to(DEV)
    kw = {}
    if score == "dot":
        q = torch.randn((B, H, D), generator=gen).to(dt)
        k = torch.randn((B, H, T, D), generator=gen).to(dt)
        o, lse = sa_decode(g, q.to(DEV), k.to(DEV), v.to(DEV), positions=posd)
        kw = dict(q=host_view(q), k=host_view(k))
    elif score == "coord":
        cq = torch.randn((B, H, 3), generator=gen)
        ck = torch.randn((B, H, T, 3), generator=gen)
        gamma = torch.rand((H,), generator=gen) * 1.5 + 0.5
        beta = torch.randn((H,), generator=gen) * 0.1
        o, lse = sa_decode(g, v=v.to(DEV), positions=posd, cq=cq.to(DEV), ck=ck.to(DEV), gamma=gamma.to(DEV),
                           beta=beta.to(DEV))
        kw = dict(cq=cq.numpy().astype(np.float64), ck=ck.numpy().astype(np.float64), gamma=gamma.numpy(),
                  beta=beta.numpy())
    else:
        o, lse = sa_decode(g, v=v.to(DEV), positions=posd)
    torch.cuda.synchronize()
    O, L = decode_reference(W, offs, pos, host_view(v), **kw)
    tol = tol_of(dt)
    eo, el = maxabs(o, O), maxabs(lse, L)
    _say("decode %s %s D=%d W=%d errors o %.2e lse %.2e" % (score, dt, D, W, eo, el))
    assert eo <= tol and el <= tol


def test_decode_default_position_and_bad_positions():
    """positions=None decodes row T - 1; a position outside [0, T) gives NaN
    for that sequence only."""
    B, H, T, D, W, offs = 3, 2, 500, 64, 16, (32, 64, 128, 256)
    gen = torch.Generator().manual_seed(99)
    q = torch.randn((B, H, D), generator=gen).to(torch.bfloat16)
    k = torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)
    v = torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)
    g = sa_build_graph(T, W, offs)
    o, lse = sa_decode(g, q.to(DEV), k.to(DEV), v.to(DEV))
    O, L = decode_reference(W, offs, np.full(B, T - 1, dtype=np.int32), host_view(v), q=host_view(q),
                            k=host_view(k))
    assert maxabs(o, O) <= 2e-2 and maxabs(lse, L) <= 2e-2
    pos = torch.tensor([-1, 7, T], dtype=torch.int32, device=DEV)
    o2, lse2 = sa_decode(g, q.to(DEV), k.to(DEV), v.to(DEV), positions=pos)
    torch.cuda.synchronize()
    assert torch.isnan(o2[0]).all() and torch.isnan(lse2[0]).all()
    assert torch.isnan(o2[2]).all() and torch.isnan(lse2[2]).all()
    O7, L7 = decode_reference(W, offs, np.array([0, 7, 0], dtype=np.int32), host_view(v), q=host_view(q),
                              k=host_view(k))
    assert maxabs(o2[1], O7[1]) <= 2e-2 and maxabs(lse2[1], L7[1]) <= 2e-2


def test_decode_full_size_sampled():
    """64 sequences x 8 heads, a 16,384-row cache, window 256: every
    (b, h) against the oracle at its row."""
    B, H, T, D, W = 64, 8, 16384, 64, 256
    gen = torch.Generator().manual_seed(7007)
    q = torch.randn((B, H, D), generator=gen).to(torch.bfloat16)
    k = torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)
    v = torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)
    pos = torch.randint(0, T, (B,), generator=gen, dtype=torch.int32)
    g = sa_build_graph(T, W, ())
    o, lse = sa_decode(g, q.to(DEV), k.to(DEV), v.to(DEV), positions=pos.to(DEV))
    torch.cuda.synchronize()
    O, L = decode_reference(W, (), pos.numpy(), host_view(v), q=host_view(q), k=host_view(k))
    assert maxabs(o, O) <= 2e-2 and maxabs(lse, L) <= 2e-2


# ------------------------------------------------------------------ grouped key/value heads
def gqa_reference(W, offs, G, v, dO=None, q=None, k=None):
    """Per query head h the oracle with k, v of head h // G; dk, dv of a
    key/value head are the sums over its G query heads (the gradient of a sum
    of per-head losses that share k and v)."""
    B, Hkv, T, D = v.shape
    H = Hkv * G
    O = np.empty((B, H, T, D))
    L = np.empty((B, H, T))
    grads = {"dv": np.zeros((B, Hkv, T, D))}
    if q is not None:
        grads.update(dq=np.empty((B, H, T, D)), dk=np.zeros((B, Hkv, T, D)))
    for b in range(B):
        for h in range(H):
            hk = h // G
            kw = dict(q=q[b, h], k=k[b, hk]) if q is not None else {}
            O[b, h], L[b, h] = oracle.fwd(T, W, offs, v[b, hk], **kw)
            if dO is not None:
                r = oracle.bwd(T, W, offs, v[b, hk], dO[b, h], **kw)
                grads["dv"][b, hk] += r["dv"]
                if q is not None:
                    grads["dq"][b, h] = r["dq"]
                    grads["dk"][b, hk] += r["dk"]
    return O, L, grads


@pytest.mark.parametrize("B,H,Hkv,T,D,dt,W,offs,score,algo", [
    (1, 8, 2, 2048, 64, torch.bfloat16, 256, (), "dot", "auto"),             # band kernels
    (1, 4, 1, 1500, 64, torch.bfloat16, 64, (128, 256, 512), "dot", "auto"),  # band + long range
    (2, 6, 3, 1100, 64, torch.bfloat16, 128, (), "dot", "auto"),             # band, two heads per workgroup
    (1, 6, 2, 900, 64, torch.bfloat16, 96, (256,), "dot", "auto"),           # band, groups of three
    (2, 6, 3, 700, 32, torch.float32, 4, tuple(2 ** k for k in range(10)), "dot", "auto"),  # gather
    (1, 4, 2, 2048, 64, torch.bfloat16, 256, (), "dot", "gather"),
    (2, 4, 1, 500, 64, torch.bfloat16, 4, (8, 16, 32, 64), "uniform", "auto"),
])
def test_grouped_kv_heads(B, H, Hkv, T, D, dt, W, offs, score, algo):
    G = H // Hkv
    gen = torch.Generator().manual_seed(31 * H + Hkv + T)
    v = torch.randn((B, Hkv, T, D), generator=gen).to(dt)
    do = torch.randn((B, H, T, D), generator=gen).to(dt)
    g = sa_build_graph(T, W, offs)
    _say("gqa B=%d H=%d Hkv=%d T=%d D=%d %s W=%d %s %s plan %s / %s" % (
        B, H, Hkv, T, D, dt, W, score, algo,
        sa_describe_plan(g, v.to(DEV), score=score, algo=algo, heads=H),
        sa_describe_plan(g, v.to(DEV), score=score, algo=algo, heads=H, which="bwd")))
    if score == "dot":
        q = torch.randn((B, H, T, D), generator=gen).to(dt)
        k = torch.randn((B, Hkv, T, D), generator=gen).to(dt)
        o, lse = sa_fwd(g, q.to(DEV), k.to(DEV), v.to(DEV), algo=algo)
        gr = sa_bwd(g, q.to(DEV), k.to(DEV), v.to(DEV), o, lse, do.to(DEV), algo=algo)
        O, L, ref = gqa_reference(W, offs, G, host_view(v), host_view(do), q=host_view(q), k=host_view(k))
    else:
        o = torch.empty((B, H, T, D), dtype=dt, device=DEV)
        o, lse = sa_fwd(g, v=v.to(DEV), o=o, algo=algo)
        gr = sa_bwd(g, v=v.to(DEV), o=o, lse=lse, dout=do.to(DEV), algo=algo)
        O, L, ref = gqa_reference(W, offs, G, host_view(v), host_view(do))
    torch.cuda.synchronize()
    tol = tol_of(dt)
    errs = {"o": maxabs(o, O), "lse": maxabs(lse, L)}
    for key in ref:
        errs[key] = maxabs(gr[key], ref[key])
    _say("gqa errors %s (tol %g)" % ({k_: "%.2e" % e for k_, e in errs.items()}, tol))
    for key, e in errs.items():
        assert e <= tol, (key, e)


def test_decode_grouped_kv_heads():
    B, H, Hkv, T, D, W, offs = 3, 8, 2, 2000, 64, 16, (32, 64, 128, 256, 512, 1024)
    gen = torch.Generator().manual_seed(1234)
    q = torch.randn((B, H, D), generator=gen).to(torch.bfloat16)
    k = torch.randn((B, Hkv, T, D), generator=gen).to(torch.bfloat16)
    v = torch.randn((B, Hkv, T, D), generator=gen).to(torch.bfloat16)
    pos = np.array([5, 1999, 1024], dtype=np.int32)
    g = sa_build_graph(T, W, offs)
    o, lse = sa_decode(g, q.to(DEV), k.to(DEV), v.to(DEV), positions=torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    G = H // Hkv
    kk = np.repeat(host_view(k), G, axis=1)  # query head h reads key/value head h // G
    vv = np.repeat(host_view(v), G, axis=1)
    O, L = decode_reference(W, offs, pos, vv, q=host_view(q), k=kk)
    assert maxabs(o, O) <= 2e-2 and maxabs(lse, L) <= 2e-2


# ------------------------------------------------------------------ explicit neighbour lists
def csr_reference(rp, cols, G, v, dO=None, q=None, k=None, cq=None, ck=None, gamma=None, beta=None):
    """Oracle per (b, h) over the lists; query head h reads key/value head
    h // G, so dk, dv of a key/value head sum over its G query heads;
    dgamma, dbeta, l1 are per head, summed over the batch."""
    B, Hkv, T, D = v.shape
    H = Hkv * G
    O, L = np.empty((B, H, T, D)), np.empty((B, H, T))
    grads = {}
    for b in range(B):
        for h in range(H):
            hk = h // G
            if cq is not None:
                kw = dict(cq=cq[b, h], ck=ck[b, h], gamma=float(gamma[h]), beta=float(beta[h]))
            elif q is not None:
                kw = dict(q=q[b, h], k=k[b, hk])
            else:
                kw = {}
            O[b, h], L[b, h] = oracle.fwd_csr(rp, cols, v[b, hk], **kw)
            if dO is None:
                continue
            r = oracle.bwd_csr(rp, cols, v[b, hk], dO[b, h], **kw)
            for key, val in r.items():
                if key in ("dgamma", "dbeta", "l1"):
                    grads.setdefault(key, np.zeros(H))[h] += val
                elif key in ("dk", "dv"):
                    grads.setdefault(key, np.zeros((B, Hkv, T, D)))[b, hk] += val
                else:
                    grads.setdefault(key, np.empty((B, H) + val.shape))[b, h] = val
    return O, L, grads


def run_csr(rp, cols, B, H, Hkv, D, dt, score, seed, grad_dtype=None):
    T = len(rp) - 1
    G = H // Hkv
    gen = torch.Generator().manual_seed(seed)
    x = {"v": torch.randn((B, Hkv, T, D), generator=gen).to(dt),
         "do": torch.randn((B, H, T, D), generator=gen).to(dt)}
    if score == "dot":
        x["q"] = torch.randn((B, H, T, D), generator=gen).to(dt)
        x["k"] = torch.randn((B, Hkv, T, D), generator=gen).to(dt)
    elif score == "coord":
        x["cq"] = torch.randn((B, H, T, 3), generator=gen)
        x["ck"] = torch.randn((B, H, T, 3), generator=gen)
        x["gamma"] = torch.rand((H,), generator=gen) * 1.5 + 0.5
        x["beta"] = torch.randn((H,), generator=gen) * 0.1
    g = sa_build_graph_csr(T, rp, cols)
    xd = {k_: t.to(DEV) for k_, t in x.items()}
    _say("csr B=%d H=%d Hkv=%d T=%d D=%d %s %s E=%d plan %s / %s" % (
        B, H, Hkv, T, D, dt, score, rp[-1], sa_describe_plan(g, xd["v"], score=score, heads=H),
        sa_describe_plan(g, xd["v"], score=score, heads=H, which="bwd")))
    if score == "dot":
        o, lse = sa_fwd(g, xd["q"], xd["k"], xd["v"])
        gr = sa_bwd(g, xd["q"], xd["k"], xd["v"], o, lse, xd["do"], grad_dtype=grad_dtype)
    elif score == "coord":
        cw = dict(cq=xd["cq"], ck=xd["ck"], gamma=xd["gamma"], beta=xd["beta"])
        o, lse = sa_fwd(g, v=xd["v"], **cw)
        gr = sa_bwd(g, v=xd["v"], o=o, lse=lse, dout=xd["do"], grad_dtype=grad_dtype, **cw)
    else:
        o = torch.empty((B, H, T, D), dtype=dt, device=DEV)
        o, lse = sa_fwd(g, v=xd["v"], o=o)
        gr = sa_bwd(g, v=xd["v"], o=o, lse=lse, dout=xd["do"], grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    hv = {k_: host_view(t) for k_, t in x.items()}
    O, L, ref = csr_reference(rp, cols, G, hv["v"], hv["do"], q=hv.get("q"), k=hv.get("k"), cq=hv.get("cq"),
                              ck=hv.get("ck"), gamma=hv.get("gamma"), beta=hv.get("beta"))
    tol = tol_of(dt)
    errs = {"o": maxabs(o, O), "lse": maxabs(lse, L)}
    assert sorted(gr) == sorted(k_ for k_ in ref if k_ != "l1")
    for key in gr:
        if key in ("dgamma", "dbeta"):
            err = np.abs(gr[key].double().cpu().numpy() - ref[key])
            errs[key] = float(np.max(err / np.maximum(tol, 1e-6 * ref["l1"]))) * tol
        else:
            errs[key] = grad_err(gr[key], ref[key], tol, grad_dtype if key in ("dq", "dk", "dv") else None)
    _say("csr errors %s (tol %g)" % ({k_: "%.2e" % e for k_, e in errs.items()}, tol))
    for key, e in errs.items():
        assert e <= tol, (key, e)
    return g, xd, o, lse, gr


def lists_of(kind, T, seed=0):
    if kind == "random":
        return random_causal_lists(T, 4, 12, seed)
    if kind == "wide":       # long, very uneven rows: window 16 + up to 40 random keys
        return random_causal_lists(T, 16, 40, seed)
    if kind == "dense":      # every j <= i (dense causal attention)
        return random_causal_lists(T, T, 0, seed)
    if kind == "self":       # only the row itself
        return random_causal_lists(T, 1, 0, seed)
    if kind == "hub":        # rows {0, i}: key 0 has T queries, the others one
        rp = np.concatenate([[0, 1], 1 + 2 * np.arange(1, T, dtype=np.int64)])
        cols = np.concatenate([[0]] + [[0, i] for i in range(1, T)]).astype(np.int64)
        return rp, cols
    raise ValueError(kind)


@pytest.mark.parametrize("kind,B,H,Hkv,T,D,dt,score", [
    ("random", 2, 2, 2, 300, 32, torch.float32, "dot"),
    ("random", 2, 2, 2, 300, 32, torch.float32, "coord"),
    ("random", 2, 2, 2, 300, 32, torch.float32, "uniform"),
    ("wide", 1, 4, 2, 777, 64, torch.bfloat16, "dot"),
    ("wide", 1, 3, 3, 513, 64, torch.bfloat16, "coord"),
    ("dense", 1, 2, 2, 257, 128, torch.float32, "dot"),
    ("self", 2, 1, 1, 129, 16, torch.float32, "dot"),
    ("hub", 1, 2, 1, 1000, 64, torch.bfloat16, "dot"),
    ("hub", 1, 2, 2, 1000, 64, torch.bfloat16, "uniform"),
])
def test_explicit_lists_small(kind, B, H, Hkv, T, D, dt, score):
    rp, cols = lists_of(kind, T, seed=T + D)
    run_csr(rp, cols, B, H, Hkv, D, dt, score, seed=7 * T + D)


def test_explicit_lists_self_only_is_identity():
    """A graph where each row lists only itself: o = v exactly, lse = s_ii."""
    T, D = 100, 32
    rp, cols = lists_of("self", T)
    g = sa_build_graph_csr(T, rp, cols)
    v = torch.randn((1, 1, T, D), generator=torch.Generator().manual_seed(3), device="cpu").to(DEV)
    o, lse = sa_fwd(g, v=v)
    torch.cuda.synchronize()
    assert torch.equal(o, v) and float(lse.abs().max()) == 0.0


@pytest.mark.parametrize("name", ["csr_dilated", "csr_random"])
def test_explicit_lists_full_size(name):
    """The full-size list workloads (B=4, H=8, T=16384, D=64, bf16), every
    output element against the oracle; the dilated graph as lists also
    against the descriptor path on the same inputs."""
    w = WORKLOADS[name]
    if w.graph == "random":
        rp, cols = workload_lists(w)
    else:
        rp, cols = oracle.graph_csr(w.T, w.window, w.offsets)
    x = make_inputs(w, device="cpu")
    gtest = run_csr_inputs(w, rp, cols, x)
    if w.graph == "lists":
        g, xd, o, lse, gr = gtest
        gd = sa_build_graph(w.T, w.window, w.offsets)
        o2, lse2 = sa_fwd(gd, xd["q"], xd["k"], xd["v"], algo="gather")
        gr2 = sa_bwd(gd, xd["q"], xd["k"], xd["v"], o2, lse2, xd["do"], algo="gather")
        torch.cuda.synchronize()
        diffs = {"o": float((o.float() - o2.float()).abs().max()), "lse": float((lse - lse2).abs().max())}
        diffs.update({k_: float((gr[k_] - gr2[k_]).abs().max()) for k_ in gr})
        _say("lists vs descriptor path: %s" % {k_: "%.2e" % e for k_, e in diffs.items()})
        assert all(e <= 2e-2 for e in diffs.values()), diffs


def run_csr_inputs(w, rp, cols, x):
    """run_csr on a workload's own seeded inputs (dot score)."""
    B, H, T, D = x["q"].shape
    g = sa_build_graph_csr(T, rp, cols)
    xd = {k_: t.to(DEV) for k_, t in x.items()}
    _say("%s full size B=%d H=%d T=%d E=%d" % (w.name, B, H, T, rp[-1]))
    o, lse = sa_fwd(g, xd["q"], xd["k"], xd["v"])
    gr = sa_bwd(g, xd["q"], xd["k"], xd["v"], o, lse, xd["do"])
    torch.cuda.synchronize()
    hv = {k_: host_view(t) for k_, t in x.items()}
    O, L, ref = csr_reference(rp, cols, 1, hv["v"], hv["do"], q=hv["q"], k=hv["k"])
    errs = {"o": maxabs(o, O), "lse": maxabs(lse, L)}
    errs.update({k_: maxabs(gr[k_], ref[k_]) for k_ in ("dq", "dk", "dv")})
    _say("%s errors %s" % (w.name, {k_: "%.2e" % e for k_, e in errs.items()}))
    for key, e in errs.items():
        assert e <= 2e-2, (key, e)
    return g, xd, o, lse, gr


@pytest.mark.parametrize("score", ["dot", "coord", "uniform"])
def test_decode_explicit_lists(score):
    """Decode on an explicit-list graph: the new token at row t attends to
    row t's list; compared with the oracle's forward at that row."""
    B, H, T, D = 4, 2, 1500, 64
    rp, cols = random_causal_lists(T, 8, 24, 55)
    g = sa_build_graph_csr(T, rp, cols)
    pos = np.array([0, 3, 777, T - 1], dtype=np.int32)
    gen = torch.Generator().manual_seed(808)
    v = torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)
    posd = torch.from_numpy(pos).to(DEV)
    O, L = np.empty((B, H, D)), np.empty((B, H))
    if score == "dot":
        q = torch.randn((B, H, D), generator=gen).to(torch.bfloat16)
        k = torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)
        o, lse = sa_decode(g, q.to(DEV), k.to(DEV), v.to(DEV), positions=posd)
    elif score == "coord":
        cq = torch.randn((B, H, 3), generator=gen)
        ck = torch.randn((B, H, T, 3), generator=gen)
        gamma = torch.rand((H,), generator=gen) + 0.5
        beta = torch.randn((H,), generator=gen) * 0.1
        o, lse = sa_decode(g, v=v.to(DEV), positions=posd, cq=cq.to(DEV), ck=ck.to(DEV), gamma=gamma.to(DEV),
                           beta=beta.to(DEV))
    else:
        o, lse = sa_decode(g, v=v.to(DEV), positions=posd)
    torch.cuda.synchronize()
    hvv = host_view(v)
    for b in range(B):
        t = int(pos[b])
        for h in range(H):
            if score == "dot":
                qf = np.zeros((T, D), dtype=host_view(q).dtype)
                qf[t] = host_view(q)[b, h]
                kw = dict(q=qf, k=host_view(k)[b, h])
            elif score == "coord":
                cqf = np.zeros((T, 3))
                cqf[t] = cq[b, h].double().numpy()
                kw = dict(cq=cqf, ck=ck[b, h].double().numpy(), gamma=float(gamma[h]), beta=float(beta[h]))
            else:
                kw = {}
            Of, Lf = oracle.fwd_csr(rp, cols, hvv[b, h], **kw)
            O[b, h], L[b, h] = Of[t], Lf[t]
    eo, el = maxabs(o, O), maxabs(lse, L)
    _say("decode lists %s errors o %.2e lse %.2e" % (score, eo, el))
    assert eo <= 2e-2 and el <= 2e-2


def test_explicit_lists_edge_cases():
    """T = 1 (one row listing itself); strided [B, T, H, D] storage; bf16
    gradients; bitwise run-to-run determinism of every output."""
    # T = 1
    rp, cols = np.array([0, 1]), np.array([0])
    run_csr(rp, cols, 2, 2, 2, 32, torch.float32, "dot", seed=1)
    # strided storage and bf16 gradients
    B, H, T, D = 2, 3, 400, 64
    rp, cols = random_causal_lists(T, 6, 20, 77)
    g = sa_build_graph_csr(T, rp, cols)
    gen = torch.Generator().manual_seed(2024)
    base = {k_: torch.randn((B, T, H, D), generator=gen).to(torch.bfloat16) for k_ in ("q", "k", "v", "do")}
    xd = {k_: t.to(DEV).transpose(1, 2) for k_, t in base.items()}  # [B, H, T, D] views, t stride H*D
    assert not xd["q"].is_contiguous()
    o, lse = sa_fwd(g, xd["q"], xd["k"], xd["v"])
    gr = sa_bwd(g, xd["q"], xd["k"], xd["v"], o, lse, xd["do"], grad_dtype=torch.bfloat16)
    o2, lse2 = sa_fwd(g, xd["q"], xd["k"], xd["v"])
    gr2 = sa_bwd(g, xd["q"], xd["k"], xd["v"], o2, lse2, xd["do"], grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert all(torch.equal(gr[k_], gr2[k_]) for k_ in gr)
    hv = {k_: host_view(t.transpose(1, 2).contiguous()) for k_, t in base.items()}
    O, L, ref = csr_reference(rp, cols, 1, hv["v"], hv["do"], q=hv["q"], k=hv["k"])
    errs = {"o": maxabs(o, O), "lse": maxabs(lse, L)}
    errs.update({k_: grad_err(gr[k_], ref[k_], 2e-2, torch.bfloat16) for k_ in ("dq", "dk", "dv")})
    _say("csr strided / bf16 gradients errors %s (gradients: beyond their bf16 rounding)"
         % {k_: "%.2e" % e for k_, e in errs.items()})
    assert all(e <= 2e-2 for e in errs.values()), errs


@pytest.mark.parametrize("kind", ["band", "dilated", "lists"])
def test_graph_capture_replays_match_eager(kind):
    """sa_fwd + sa_bwd captured in a HIP graph (they allocate, clear and
    synchronise nothing): several replays, with eager work and
    synchronisation between them, each bitwise equal to the eager result."""
    B, H, T, D = 1, 2, 1024, 64
    if kind == "band":
        g = sa_build_graph(T, 128, ())
    elif kind == "dilated":
        g = sa_build_graph(T, 4, tuple(2 ** k for k in range(10)))
    else:
        rp, cols = random_causal_lists(T, 4, 12, 99)
        g = sa_build_graph_csr(T, rp, cols)
    gen = torch.Generator().manual_seed(5150)
    x = {k_: torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16).to(DEV) for k_ in ("q", "k", "v", "do")}
    s = torch.cuda.Stream()
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, H, T), dtype=torch.float32, device=DEV)
    grads = {k_: torch.empty((B, H, T, D), dtype=torch.float32, device=DEV) for k_ in ("dq", "dk", "dv")}
    with torch.cuda.stream(s):
        sa_fwd(g, x["q"], x["k"], x["v"], o=o, lse=lse, stream=s)  # eager (uploads explicit lists)
        sa_bwd(g, x["q"], x["k"], x["v"], o, lse, x["do"], stream=s, **grads)
    torch.cuda.synchronize()
    ref = {"o": o.clone(), "lse": lse.clone(), **{k_: t.clone() for k_, t in grads.items()}}
    ws = torch.empty(max(sa_bwd_workspace_size_of(g, x["v"]), 256), dtype=torch.uint8, device=DEV)
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg, stream=s):
        sa_fwd(g, x["q"], x["k"], x["v"], o=o, lse=lse, stream=s)
        sa_bwd(g, x["q"], x["k"], x["v"], o, lse, x["do"], workspace=ws, stream=s, **grads)
    outs = {"o": o, "lse": lse, **grads}
    for rep in range(4):
        for t in outs.values():
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        cg.replay()
        torch.cuda.synchronize()
        for k_, t in outs.items():
            assert torch.equal(t, ref[k_]), (kind, rep, k_)
    _say("graph capture %s: %d replays equal to eager" % (kind, 4))


def sa_bwd_workspace_size_of(g, v):
    from sparse_causal_attention_amd import sa_bwd_workspace_size
    return sa_bwd_workspace_size(g, v)


def test_side_stream_and_fixed_upload():
    """Calls on a stream other than torch's current one give the same bits as
    on the current stream (the binding makes the launch stream wait for the
    current one and allocates outputs and workspace on it), and an explicit-list
    graph's device lists are fixed by its first upload: the library refuses a
    second sa_graph_upload, with nothing copied."""
    import ctypes

    from sparse_causal_attention_amd import _abi

    B, H, T, D = 1, 2, 700, 64
    rp, cols = random_causal_lists(T, 4, 12, 4242)
    for g in (sa_build_graph(T, 64, (128, 256)), sa_build_graph_csr(T, rp, cols)):
        gen = torch.Generator().manual_seed(31337)
        x = {k_: torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16).to(DEV)
             for k_ in ("q", "k", "v", "do")}
        o, lse = sa_fwd(g, x["q"], x["k"], x["v"])
        gr = sa_bwd(g, x["q"], x["k"], x["v"], o, lse, x["do"])
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        # inputs produced on the current stream just before the side-stream call
        xs = {k_: t * 1 for k_, t in x.items()}
        o2, lse2 = sa_fwd(g, xs["q"], xs["k"], xs["v"], stream=s)
        gr2 = sa_bwd(g, xs["q"], xs["k"], xs["v"], o2, lse2, xs["do"], stream=s)
        s.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2)
        assert all(torch.equal(gr[k_], gr2[k_]) for k_ in gr)
        if g.is_csr:
            n = g.device_bytes()
            other = torch.empty(n + 256, dtype=torch.uint8, device=DEV)
            ptr = other.data_ptr() + (-other.data_ptr()) % 256
            st = _abi.lib().sa_graph_upload(g.handle, ctypes.c_void_p(ptr), n, None)
            assert st == _abi.SA_ERR_INVALID_ARG
            o3, _ = sa_fwd(g, x["q"], x["k"], x["v"])  # still reads the first upload
            torch.cuda.synchronize()
            assert torch.equal(o3, o)
    _say("side stream: bitwise equal to the current stream; second upload refused")

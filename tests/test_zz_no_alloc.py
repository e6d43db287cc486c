"""The allocation-free backward (sa_bwd_noalloc) against sa_bwd, through the
C ABI: bitwise equal gradients on two calls in a row, the second with a
smaller input (the built-in scratch keeps the first call's contents), on the
band, gather, coordinate and explicit-list paths; and no device allocation
during the call when every output is given."""
import sys

import pytest
import torch

from sparse_causal_attention_amd import (_abi, sa_build_graph, sa_build_graph_csr, sa_bwd, sa_bwd_noalloc,
                                        sa_describe_plan, sa_fwd)
from sparse_causal_attention_amd.inputs import random_causal_lists

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print("\n[no-alloc] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _abi.lib()


def _inputs(B, H, T, D, score, seed):
    gen = torch.Generator().manual_seed(seed)
    x = {"v": torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16),
         "do": torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)}
    if score == "coord":
        x["cq"] = torch.randn((B, H, T, 3), generator=gen)
        x["ck"] = torch.randn((B, H, T, 3), generator=gen)
        x["gamma"] = torch.rand((H,), generator=gen) * 1.5 + 0.5
        x["beta"] = torch.randn((H,), generator=gen) * 0.1
    else:
        x["q"] = torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)
        x["k"] = torch.randn((B, H, T, D), generator=gen).to(torch.bfloat16)
    return {k: t.to(DEV) for k, t in x.items()}


def _graph(kind, T):
    if kind == "band":
        return sa_build_graph(T, 256, ())
    if kind in ("dilated", "coord"):
        return sa_build_graph(T, 4, tuple(2 ** k for k in range(14)))
    rp, cols = random_causal_lists(T, 4, 12, 2718)
    return sa_build_graph_csr(T, rp, cols)


def _one(kind, B, H, T, seed):
    score = "coord" if kind == "coord" else "dot"
    g = _graph(kind, T)
    x = _inputs(B, H, T, 64, score, seed)
    if score == "coord":
        cw = dict(cq=x["cq"], ck=x["ck"], gamma=x["gamma"], beta=x["beta"])
        o, lse = sa_fwd(g, v=x["v"], **cw)
        ref = sa_bwd(g, v=x["v"], o=o, lse=lse, dout=x["do"], **cw)
        outs = {k: torch.full_like(t, float("nan")) for k, t in ref.items()}
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        got = sa_bwd_noalloc(g, v=x["v"], o=o, lse=lse, dout=x["do"], **cw, **outs)
    else:
        o, lse = sa_fwd(g, x["q"], x["k"], x["v"])
        ref = sa_bwd(g, x["q"], x["k"], x["v"], o, lse, x["do"])
        outs = {k: torch.full_like(t, float("nan")) for k, t in ref.items()}
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        got = sa_bwd_noalloc(g, x["q"], x["k"], x["v"], o, lse, x["do"], **outs)
    after = torch.cuda.memory_allocated()
    torch.cuda.synchronize()
    plan = sa_describe_plan(g, x["v"], score=score, which="bwd")
    _say("%s B=%d H=%d T=%d plan %s" % (kind, B, H, T, plan))
    assert after == before, "the call allocated device memory through torch"
    for k, t in ref.items():
        assert got[k] is outs[k]
        assert torch.equal(got[k], t), (kind, T, k)
    return plan


@pytest.mark.parametrize("kind", ["band", "dilated", "coord", "lists"])
def test_noalloc_matches_sa_bwd_twice_then_smaller(kind):
    plan1 = _one(kind, 2, 4, 4096, 11)
    plan2 = _one(kind, 1, 2, 1000, 12)  # smaller: the scratch still holds the first call's values
    if kind == "band":
        assert plan1.startswith("band_bwd") and plan2.startswith("band_bwd")


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    # 40 x 65536 rows: 21 MB of workspace against the 16 MiB scratch
    g = sa_build_graph(1 << 16, 4, ())
    x = {k: torch.zeros((1, 40, 1 << 16, 64), dtype=torch.bfloat16, device=DEV) for k in ("q", "k", "v", "do")}
    lse = torch.zeros((1, 40, 1 << 16), dtype=torch.float32, device=DEV)
    with pytest.raises(_abi.SaError) as e:
        sa_bwd_noalloc(g, x["q"], x["k"], x["v"], x["v"], lse, x["do"])
    assert e.value.status == _abi.SA_ERR_WORKSPACE

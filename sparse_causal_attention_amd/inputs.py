"""Seeded synthetic workloads.

This module holds the workload shapes and the seeded random inputs that both
the HIP path's tests/benchmark and the CPU oracle consume.  It holds none of
the method's arithmetic: only shapes, graph parameters (T, W, offsets) and
random draws.  It imports nothing from the rest of the package.

Shapes stand in for the pages' workloads (no corpus or trained weight is
available or needed): the 16,384-token training context of the SpatialLM-Mini
news page ("What the comparison on 8 GB showed"), the 256-token chunked window
at the longest context MiniGPT (Part 6) trained ("The raw numbers" table), and
the very long single-GPU sequences of the sparse-graph-processing abstract
(arXiv 2502.01659).  Values are i.i.d. N(0, 1) drawn in fp32 and rounded to
bf16 (round-to-nearest-even) where the workload is bf16.

Seed of tensor t of workload c: 1000 * c + t with t = 0 q, 1 k, 2 v, 3 dO,
4 c_q, 5 c_k, 6 gamma, 7 beta, 8 sampled rows, 9 random neighbour lists.

Explicit-list workloads carry their graph as per-row key lists: either the
window + distances graph written out row by row (`graph="lists"`, the same
edges through the indexed kernels) or random causal lists (`graph="random"`:
row i keeps its `window` nearest keys i-window+1 .. i plus `extra` distinct
earlier keys drawn uniformly, the same degree as the dilated workload with no
regular structure).  The pages name no particular mask, so this random
pattern is a stand-in.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SEED_Q, SEED_K, SEED_V, SEED_DO, SEED_CQ, SEED_CK, SEED_GAMMA, SEED_BETA, SEED_ROWS, SEED_LISTS = range(10)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int  # c in the seed formula
    B: int
    H: int
    T: int
    D: int
    dtype: torch.dtype
    window: int
    offsets: tuple = field(default_factory=tuple)
    coord: bool = False
    backward: bool = True
    uniform: bool = False  # fixed equal weights (v alone)
    decode: bool = False   # one new token per sequence at row T - 1 of a T-row cache
    Hkv: int = 0           # key/value heads (0: H)
    graph: str = "distance"  # "distance", "lists" (same graph as lists) or "random" lists
    extra: int = 0           # random lists: distinct earlier keys per row beyond the window
    grad_bf16: bool = False  # gradients stored in bf16 (else fp32)

    @property
    def kv_heads(self) -> int:
        return self.Hkv if self.Hkv > 0 else self.H

    @property
    def dtype_name(self) -> str:
        return {torch.float32: "f32", torch.bfloat16: "bf16"}[self.dtype]


def _pow2(lo: int, hi: int) -> tuple:
    return tuple(2 ** k for k in range(lo, hi + 1))


WORKLOADS = {
    # tiny fp32 forward/backward: window 8 + distances 16..128
    "tiny": Workload("tiny", 1, 1, 2, 256, 32, torch.float32, 8, (16, 32, 64, 128)),
    "tiny_dense": Workload("tiny_dense", 1, 1, 2, 256, 32, torch.float32, 256, ()),
    # sliding window only, W = 256, T = 16384
    "band": Workload("band", 2, 1, 8, 16384, 64, torch.bfloat16, 256, ()),
    "band_dense": Workload("band_dense", 2, 1, 8, 2048, 64, torch.bfloat16, 2048, ()),
    # local window 4 + distances 2^0..2^13, training shape B=4, H=8, T=16384
    "dilated": Workload("dilated", 3, 4, 8, 16384, 64, torch.bfloat16, 4, _pow2(0, 13)),
    # coordinate-distance score on the dilated graph
    "coord": Workload("coord", 4, 4, 8, 16384, 64, torch.bfloat16, 4, _pow2(0, 13), coord=True),
    # coordinate-distance score on the W = 256 band graph (secondary)
    "coord_band": Workload("coord_band", 4, 1, 8, 16384, 64, torch.bfloat16, 256, (), coord=True),
    # the dilated graph with fixed equal weights (the same-graph comparison
    # that isolates the scores)
    "uniform": Workload("uniform", 6, 4, 8, 16384, 64, torch.bfloat16, 4, _pow2(0, 13), uniform=True),
    # grouped key/value heads: 8 query heads sharing 2 key/value heads, on the
    # band graph and on the dilated graph
    "band_gqa": Workload("band_gqa", 9, 1, 8, 16384, 64, torch.bfloat16, 256, (), Hkv=2),
    "dilated_gqa": Workload("dilated_gqa", 10, 4, 8, 16384, 64, torch.bfloat16, 4, _pow2(0, 13), Hkv=2),
    # decode steps: 64 sequences x 8 heads, one new token each at the end of a
    # 16,384-row key/value cache, on the band graph and on the dilated graph
    "decode_band": Workload("decode_band", 7, 64, 8, 16384, 64, torch.bfloat16, 256, (), backward=False,
                            decode=True),
    "decode_dilated": Workload("decode_dilated", 8, 64, 8, 16384, 64, torch.bfloat16, 4, _pow2(0, 13),
                               backward=False, decode=True),
    # explicit per-row lists: the dilated graph written out, and random causal
    # lists of the same degree (window 4 + 12 random earlier keys)
    "csr_dilated": Workload("csr_dilated", 11, 4, 8, 16384, 64, torch.bfloat16, 4, _pow2(0, 13),
                            graph="lists"),
    "csr_random": Workload("csr_random", 12, 4, 8, 16384, 64, torch.bfloat16, 4, (), graph="random",
                           extra=12),
    # ultra-long single head, forward only: window 64 + distances 2^6..2^25
    "ultra": Workload("ultra", 5, 1, 1, 2 ** 26, 64, torch.bfloat16, 64, _pow2(6, 25),
                      backward=False),
    # the same inputs with the window alone (the ultra workload's time and
    # traffic split into its window and long-range parts)
    "ultra_band": Workload("ultra_band", 5, 1, 1, 2 ** 26, 64, torch.bfloat16, 64, (), backward=False),
    # the band workload with gradients stored in bf16 (the gradient dtype of
    # a bf16 model); the fp32-gradient band workload stays the reference
    "band_bf16grad": Workload("band_bf16grad", 2, 1, 8, 16384, 64, torch.bfloat16, 256, (), grad_bf16=True),
}


def seed_of(w: Workload, t: int) -> int:
    return 1000 * w.index + t


def _randn(shape, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32)


def _uniform(shape, lo: float, hi: float, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def random_causal_lists(T: int, window: int, extra: int, seed: int):
    """Seeded random causal lists (int64 numpy row_ptr [T+1], cols): row i
    holds max(0, i-window+1) .. i and min(extra, i-window+1) distinct keys
    drawn uniformly from 0 .. i-window, ascending."""
    import numpy as np

    rng = np.random.default_rng(seed)
    rp = np.zeros(T + 1, dtype=np.int64)
    rows = []
    for i in range(T):
        lo = max(0, i - window + 1)
        pool = lo  # keys 0 .. lo-1 lie outside the window
        n = min(extra, pool)
        if n == 0:
            far = np.empty(0, dtype=np.int64)
        elif n * 4 >= pool:
            far = np.sort(rng.permutation(pool)[:n])
        else:
            picked = set()
            while len(picked) < n:
                picked.update(int(x) for x in rng.integers(0, pool, size=n - len(picked)))
            far = np.array(sorted(picked), dtype=np.int64)
        row = np.concatenate([far, np.arange(lo, i + 1, dtype=np.int64)])
        rows.append(row)
        rp[i + 1] = rp[i] + len(row)
    return rp, np.concatenate(rows)


def workload_lists(w: Workload):
    """The explicit lists of a random-list workload (row_ptr, cols)."""
    assert w.graph == "random", w.name
    return random_causal_lists(w.T, w.window, w.extra, seed_of(w, SEED_LISTS))


def make_inputs(w: Workload, device="cpu", backward: bool | None = None,
                B: int | None = None, H: int | None = None, T: int | None = None,
                D: int | None = None) -> dict:
    """CPU-generated seeded inputs, moved to `device`.  Shape overrides allow
    small variants of a workload with the same recipe."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    D = w.D if D is None else D
    backward = w.backward if backward is None else backward
    shp = (B, H, T, D)
    kv_shp = (B, w.kv_heads if H == w.H else H, T, D)  # shape overrides keep one head per query head
    out = {}
    if w.coord:
        out["cq"] = _randn((B, H, T, 3), seed_of(w, SEED_CQ))
        out["ck"] = _randn((B, H, T, 3), seed_of(w, SEED_CK))
        out["gamma"] = _uniform((H,), 0.5, 2.0, seed_of(w, SEED_GAMMA))
        out["beta"] = _randn((H,), seed_of(w, SEED_BETA)) * 0.1
    elif w.uniform:
        pass  # v alone
    else:
        out["q"] = _randn((B, H, D) if w.decode else shp, seed_of(w, SEED_Q)).to(w.dtype)
        out["k"] = _randn(kv_shp, seed_of(w, SEED_K)).to(w.dtype)
    out["v"] = _randn(kv_shp, seed_of(w, SEED_V)).to(w.dtype)
    if backward:
        out["do"] = _randn(shp, seed_of(w, SEED_DO)).to(w.dtype)
    return {k: t.to(device) for k, t in out.items()}


def make_decode_inputs(w: Workload, device) -> dict:
    """Decode inputs drawn on the device (the caches are too large to draw on
    the host quickly): q [B, H, D], k and v caches [B, H, T, D], fp32 normal
    draws from seeded device generators rounded to the workload dtype."""
    out = {}
    for name, t, shp in (("q", SEED_Q, (w.B, w.H, w.D)), ("k", SEED_K, (w.B, w.H, w.T, w.D)),
                         ("v", SEED_V, (w.B, w.H, w.T, w.D))):
        g = torch.Generator(device=device).manual_seed(seed_of(w, t))
        out[name] = torch.randn(shp, generator=g, device=device, dtype=torch.float32).to(w.dtype)
    return out


def make_device_inputs_chunked(w: Workload, device, chunk_rows: int = 1 << 22) -> dict:
    """Device-generated inputs for workloads too large to draw on the host
    (the 2^26-token single head): fp32 normal draws from a seeded device
    generator, chunk by chunk, rounded to the workload dtype."""
    assert w.B == 1 and w.H == 1
    out = {}
    for name, t in (("q", SEED_Q), ("k", SEED_K), ("v", SEED_V)):
        x = torch.empty((1, 1, w.T, w.D), dtype=w.dtype, device=device)
        g = torch.Generator(device=device).manual_seed(seed_of(w, t))
        for r0 in range(0, w.T, chunk_rows):
            r1 = min(w.T, r0 + chunk_rows)
            x[0, 0, r0:r1].copy_(torch.randn((r1 - r0, w.D), generator=g, device=device,
                                             dtype=torch.float32))
        out[name] = x
    return out


def sample_rows(w: Workload, n: int = 4096, boundary=None) -> torch.Tensor:
    """n rows uniform in [0, T) from the workload's row seed, plus boundary rows."""
    g = torch.Generator().manual_seed(seed_of(w, SEED_ROWS))
    r = torch.randint(0, w.T, (n,), generator=g, dtype=torch.int64)
    if boundary:
        r = torch.cat([r, torch.tensor([b for b in boundary if 0 <= b < w.T], dtype=torch.int64)])
    return torch.unique(r)


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 CPU tensor (exact stored bits)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def host_view(t: torch.Tensor):
    """numpy view with exact stored values: fp32 stays fp32, bf16 becomes bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.numpy()

"""Throughput of the sparse causal attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads band,dilated,coord,ultra]

One step = one forward (sa_fwd) plus one backward (sa_bwd) over one batch of
seeded synthetic inputs already resident in HBM (the 2^26-token workload is
forward only).  The headline line is the sliding-window workload (B=1, H=8,
T=16384, D=64, W=256, bf16); the other workloads are measured in the same run
and reported under "extra".  Prints exactly one JSON line.

Roofline: algorithmic bytes per call (each tensor once: q, k, v, o, lse
forward; q, k, v, o, dout, lse, dq, dk, dv backward; plus a K and V row per
long-range edge forward and q, dout, k, v rows plus lse, Delta per long-range
edge backward) divided by the call's average duration, measured with HIP
events recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16 MFMA
METRIC = "attention edges/s and tokens/s fwd+bwd at T=16384; % of HBM/MFMA roofline"
SAMPLE = 10                  # per-call HIP events on every SAMPLE-th timed step
COLD_REPS = 10               # cold-cache repetitions per call
FLUSH_BYTES = 1 << 30        # written before each cold call: more than the L2s and the 256 MB MALL


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads",
                    default="band,band_bf16grad,uniform,band_gqa,dilated_gqa,csr_dilated,csr_random,decode_band,"
                            "decode_dilated,ultra_band,dilated,coord,ultra")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample length")
    ap.add_argument("--algo", default="auto")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache repetitions (profiled runs: keeps per-kernel averages warm)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (scales profiler byte counters)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured copy / MFMA-loop / empty-launch denominators")
    ap.add_argument("--probe-rates", action="store_true",
                    help="only run the issue-rate probes (MFMA and vector-ALU overlap on one SIMD) and print "
                         "one JSON line")
    ap.add_argument("--sweep", action="store_true",
                    help="only time forward + backward across window sizes (band graph) and sequence lengths "
                         "(dilated graph), per edge, and print one JSON line")
    ap.add_argument("--record-profiles", metavar="DIR",
                    help="write profiles/ from the rocprofv3 CSV output under DIR/<workload>/<pass> (no GPU)")
    return ap.parse_args()


# ------------------------------------------------------------------ byte and flop models
_LISTS = {}


def random_lists(w):
    """The seeded lists of a random-list workload (drawn once per process)."""
    if w.name not in _LISTS:
        from sparse_causal_attention_amd.inputs import workload_lists
        _LISTS[w.name] = workload_lists(w)
    return _LISTS[w.name]


def edge_counts(w):
    """(total edges per (b, h), edges outside the window per (b, h)).  For
    random lists every edge past the row's `window` nearest keys counts as a
    long-range (gathered) edge."""
    T, Wc = w.T, min(w.window, w.T)
    band = Wc * (Wc + 1) // 2 + Wc * (T - Wc)
    if w.graph == "random":
        E = int(random_lists(w)[0][-1])
        return E, E - band
    dil = sorted({d for d in w.offsets if Wc <= d < T})
    long_range = sum(T - d for d in dil)
    return band + long_range, long_range


def models(w, grad_bytes=4):
    """Algorithmic bytes and flops per call for workload w (all heads).

    Two byte models: "compulsory" reads and writes every tensor once (the
    floor); "gather" adds the K/V (forward) and K, V, Q, dO, LSE, Delta
    (backward) rows fetched per long-range edge, with no credit for cache
    reuse across queries.  Window edges are charged as compulsory: their rows
    are contiguous and reused on chip.  Explicit lists add their int32 arrays
    once per call (row pointers and keys; the backward reads the reverse lists
    too): they are shared by every (batch, head) and stay in cache."""
    E, Ed = edge_counts(w)
    lists = 4 * (w.T + 1) + 4 * E if w.graph != "distance" else 0
    rows = w.B * w.H * w.T
    eb = 2 if w.dtype_name == "bf16" else 4
    D = w.D
    if w.decode:
        # one token per (b, h) at row T - 1: its k and v rows per edge, q, o, lse
        deg = min(w.T, w.window) + sum(1 for d in sorted(set(w.offsets)) if min(w.T, w.window) <= d <= w.T - 1)
        bh = w.B * w.H
        byt = bh * (deg * 2 * D * eb + 2 * D * eb + 4) + 4 * w.B
        return {"edges": bh * deg, "fwd_bytes": byt, "bwd_bytes": 0, "fwd_bytes_compulsory": byt,
                "bwd_bytes_compulsory": 0, "fwd_flops": bh * deg * 4 * D, "bwd_flops": 0}
    if w.uniform:
        # forward: v, o rows, lse; backward: dout, lse, dv; per long-range edge
        # the v row (forward) or the dout row and lse (backward)
        fwd_c = rows * (2 * D * eb + 4)
        fwd_e = Ed * D * eb
        bwd_c = rows * (D * eb + 4 + D * grad_bytes)
        bwd_e = Ed * (D * eb + 4)
        ffl = w.B * w.H * E * 2 * D
        bfl = w.B * w.H * E * 2 * D
    elif w.coord:
        # forward: c_q, c_k (12 B), v, o rows, lse; backward: + dout, dv, dcq, dck
        fwd_c = rows * (12 + 12 + 2 * D * eb + 4)
        fwd_e = Ed * (12 + D * eb)
        bwd_c = rows * (12 + 12 + D * eb + D * eb + D * eb + 4 + D * grad_bytes + 12 + 12)
        bwd_e = Ed * 2 * (12 + D * eb + 8)
        ffl = w.B * w.H * E * (2 * D + 11)
        bfl = w.B * w.H * E * (4 * D + 35)
    else:
        # q, o, dO, dq, lse per query-head row; k, v, dk, dv per key/value-head row
        kv_rows = w.B * w.kv_heads * w.T
        fwd_c = rows * (2 * D * eb + 4) + kv_rows * 2 * D * eb
        fwd_e = Ed * 2 * D * eb
        bwd_c = rows * (3 * D * eb + 4 + D * grad_bytes) + kv_rows * (2 * D * eb + 2 * D * grad_bytes)
        bwd_e = Ed * (4 * D * eb + 8)
        ffl = w.B * w.H * E * 4 * D
        bfl = w.B * w.H * E * 10 * D
    bh = w.B * w.H
    fwd_c += lists
    bwd_c += 2 * lists
    return {"edges": bh * E, "fwd_bytes": fwd_c + bh * fwd_e, "bwd_bytes": bwd_c + bh * bwd_e,
            "fwd_bytes_compulsory": fwd_c, "bwd_bytes_compulsory": bwd_c,
            "fwd_flops": ffl, "bwd_flops": bfl}


# ------------------------------------------------------------------ timing
def score_name(w):
    return "coord" if w.coord else ("uniform" if w.uniform else "dot")


def make_graph(w):
    """The workload's graph: the window + distances descriptor, the same graph
    as explicit lists (the library's own row export), or random lists."""
    from sparse_causal_attention_amd import sa_build_graph, sa_build_graph_csr

    if w.graph == "distance":
        return sa_build_graph(w.T, w.window, w.offsets)
    if w.graph == "lists":
        return sa_build_graph_csr(w.T, *sa_build_graph(w.T, w.window, w.offsets).rows())
    return sa_build_graph_csr(w.T, *random_lists(w))


def run_workload(w, steps, warmup, algo, with_backward=True, no_cold=False):
    import torch

    from sparse_causal_attention_amd import sa_bwd_prepared, sa_describe_plan, sa_fwd_prepared
    from sparse_causal_attention_amd.inputs import make_device_inputs_chunked, make_inputs

    dev = "cuda"
    if w.T * w.D * w.B * w.H > (1 << 30):
        x = make_device_inputs_chunked(w, dev)
    else:
        x = {k: t.to(dev) for k, t in make_inputs(w, backward=with_backward and w.backward).items()}
    g = make_graph(w)
    bwd = with_backward and w.backward
    coord = w.coord
    o = torch.empty((w.B, w.H, w.T, w.D), dtype=x["v"].dtype, device=dev)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    fkw = dict(v=x["v"], cq=x.get("cq"), ck=x.get("ck"), gamma=x.get("gamma"), beta=x.get("beta"),
               o=o, lse=lse, algo=algo)
    if not coord and not w.uniform:
        fkw.update(q=x["q"], k=x["k"])
    grads = None
    if bwd:
        gshape = (w.B, w.H, w.T, w.D)
        kvshape = (w.B, w.kv_heads, w.T, w.D)
        gdt = torch.bfloat16 if w.grad_bf16 else torch.float32
        grads = {"dv": torch.empty(kvshape, dtype=gdt, device=dev)}
        if coord:
            grads.update(dcq=torch.empty((w.B, w.H, w.T, 3), dtype=torch.float32, device=dev),
                         dck=torch.empty((w.B, w.H, w.T, 3), dtype=torch.float32, device=dev),
                         dgamma=torch.empty((w.H,), dtype=torch.float32, device=dev),
                         dbeta=torch.empty((w.H,), dtype=torch.float32, device=dev))
        elif not w.uniform:
            grads.update(dq=torch.empty(gshape, dtype=gdt, device=dev),
                         dk=torch.empty(kvshape, dtype=gdt, device=dev))
        from sparse_causal_attention_amd import sa_bwd_workspace_size
        ws = torch.empty(sa_bwd_workspace_size(g, x["v"], heads=w.H), dtype=torch.uint8, device=dev)
        bkw = dict(v=x["v"], o=o, lse=lse, dout=x["do"], cq=x.get("cq"), ck=x.get("ck"),
                   gamma=x.get("gamma"), beta=x.get("beta"), workspace=ws, algo=algo,
                   grad_dtype=gdt, **grads)
        if not coord and not w.uniform:
            bkw.update(q=x["q"], k=x["k"])

    fwd_call = sa_fwd_prepared(g, **fkw)
    bwd_call = sa_bwd_prepared(g, **bkw) if bwd else None

    def step(start=None, mid=None):
        if start is not None:
            start.record()
        fwd_call()
        if mid is not None:
            mid.record()
        if bwd:
            bwd_call()

    for _ in range(warmup):
        step()
    # HIP events on the kernels' stream.  An event between two kernels holds
    # the second back until the first has drained, so the per-call events are
    # recorded on every SAMPLE-th step only (its forward runs from ev[s][0] to
    # ev[s][1], its backward from ev[s][1] to ev[s][2]); the other steps run
    # back to back, as they would in training, and the whole timed region is
    # bracketed by its own pair of events.
    sampled = list(range(0, steps, SAMPLE))
    ev = {s: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for s in sampled}
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record()
    for s in range(steps):
        e = ev.get(s)
        if e is None:
            step()
        else:
            step(e[0], e[1])
            e[2].record()
    region[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = [ev[s][0].elapsed_time(ev[s][1]) for s in sampled]
    b_ms = [ev[s][1].elapsed_time(ev[s][2]) for s in sampled] if bwd else [0.0]
    cold = None if no_cold else cold_cache(fwd_call, bwd_call, COLD_REPS if steps >= COLD_REPS else 1)
    res = {
        "wall_s": wall, "ms_per_step": 1e3 * wall / steps,
        "event_ms_per_step": region[0].elapsed_time(region[1]) / steps, "sampled_steps": len(sampled),
        "fwd_ms": sum(f_ms) / len(f_ms), "bwd_ms": sum(b_ms) / len(b_ms),
        "fwd_ms_min": min(f_ms), "bwd_ms_min": min(b_ms),
        "fwd_ms_median": median(f_ms), "bwd_ms_median": median(b_ms), "cold": cold,
        "plan_fwd": sa_describe_plan(g, x["v"], score=score_name(w), algo=algo, which="fwd", heads=w.H),
        "plan_bwd": sa_describe_plan(g, x["v"], score=score_name(w), algo=algo, which="bwd",
                                     heads=w.H) if bwd else None,
        "inputs": {k: t for k, t in x.items()},
    }
    del o, lse, grads
    return res


def sweep_workloads():
    """The scaling sweep: the band graph (B = 1, H = 8, T = 16,384, D = 64
    bf16) at windows 32 .. 2,048 and at W = T (dense causal attention), and
    the dilated graph (B = 1, H = 8, window 4 plus distances 2^0 .. < T) at
    T = 4,096 .. 65,536.  Seeded inputs of the same recipe as the named
    workloads."""
    import dataclasses

    from sparse_causal_attention_amd.inputs import WORKLOADS
    band, dil = WORKLOADS["band"], WORKLOADS["dilated"]
    out = [dataclasses.replace(band, name="band_W%d" % W, window=W) for W in (32, 64, 128, 256, 512, 1024, 2048)]
    out.append(dataclasses.replace(band, name="band_dense_causal", window=band.T))
    for T in (4096, 8192, 16384, 32768, 65536):
        offs = tuple(2 ** k for k in range(T.bit_length() - 1))
        out.append(dataclasses.replace(dil, name="dilated_T%d" % T, B=1, T=T, offsets=offs))
    return out


def sweep(steps=50, warmup=10):
    """Forward + backward time per workload of sweep_workloads() and per edge
    (the work of a sparse graph should follow its edge count, not T^2)."""
    rows = []
    for w in sweep_workloads():
        print("[bench] sweep %s" % w.name, file=sys.stderr, flush=True)
        r = run_workload(w, steps, warmup, "auto", no_cold=True)
        E, _ = edge_counts(w)
        edges = E * w.B * w.H
        fb_ms = r["fwd_ms"] + r["bwd_ms"]
        rows.append({"workload": w.name, "T": w.T, "window": min(w.window, w.T), "n_offsets": len(w.offsets),
                     "edges": edges, "fwd_us": round(1e3 * r["fwd_ms"], 1), "bwd_us": round(1e3 * r["bwd_ms"], 1),
                     "ps_per_edge_fwd_bwd": round(1e9 * fb_ms / edges, 2),
                     "plan": "%s | %s" % (r["plan_fwd"], r["plan_bwd"])})
        del r
    return {"sweep": "forward + backward per edge", "B": 1, "H": 8, "D": 64, "dtype": "bf16",
            "steps": steps, "rows": rows}


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def cold_cache(fwd_call, bwd_call, reps):
    """Each call timed alone after FLUSH_BYTES of unrelated writes (a fill
    kernel) have evicted the inputs from the L2s and the MALL: median and
    minimum over `reps` repetitions.  The backward reads the o and lse of the
    forward just before it, as in a training step."""
    import torch

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    f_ms, b_ms = [], []
    for r in range(reps):
        for call, out in ((fwd_call, f_ms), (bwd_call, b_ms)):
            if call is None:
                continue
            flush.fill_(r & 0xFF)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            call()
            e[1].record()
            torch.cuda.synchronize()
            out.append(e[0].elapsed_time(e[1]))
    del flush
    res = {"reps": reps, "flush_bytes": FLUSH_BYTES,
           "fwd_ms_median": median(f_ms), "fwd_ms_min": min(f_ms)}
    if b_ms:
        res.update(bwd_ms_median=median(b_ms), bwd_ms_min=min(b_ms))
    return res


def run_decode(w, steps, warmup, no_cold=False):
    """Decode steps: sa_decode of B new tokens (every head) at row T - 1."""
    import torch

    from sparse_causal_attention_amd import sa_build_graph, sa_decode_prepared
    from sparse_causal_attention_amd.inputs import make_decode_inputs

    dev = "cuda"
    x = make_decode_inputs(w, dev)
    g = sa_build_graph(w.T, w.window, w.offsets)
    call = sa_decode_prepared(g, x["q"], x["k"], x["v"])
    for _ in range(warmup):
        call()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f_ms = [e[0].elapsed_time(e[1]) for e in evs]
    cold = None if no_cold else cold_cache(call, None, COLD_REPS)
    return {"wall_s": wall, "ms_per_step": 1e3 * wall / steps, "fwd_ms": sum(f_ms) / len(f_ms), "bwd_ms": 0.0,
            "fwd_ms_min": min(f_ms), "bwd_ms_min": 0.0, "fwd_ms_median": median(f_ms), "bwd_ms_median": 0.0,
            "cold": cold, "plan_fwd": "decode_kernel(dot)", "plan_bwd": None, "inputs": x}


def summarize(w, r, steps):
    m = models(w, grad_bytes=2 if w.grad_bf16 else 4)
    tokens = w.B if w.decode else w.B * w.T  # a decode step makes one token per sequence
    fb = r["fwd_ms"] + r["bwd_ms"]
    wall = r["wall_s"]
    out = {
        "workload": w.name,
        "shape": {"B": w.B, "H": w.H, "H_kv": w.kv_heads, "T": w.T, "D": w.D, "window": w.window,
                  "offsets": list(w.offsets), "graph": w.graph, "dtype": w.dtype_name,
                  "score": score_name(w), "backward": w.backward,
                  "grad_dtype": ("bf16" if w.grad_bf16 else "f32") if w.backward else None},
        # decode steps last microseconds: their rate comes from the kernel events
        "tokens_per_s": tokens / (r["fwd_ms"] * 1e-3) if w.decode else tokens * steps / wall,
        "edges_per_s": m["edges"] / (r["fwd_ms"] * 1e-3) if w.decode else m["edges"] * steps / wall,
        "ms_per_step": r["ms_per_step"],
        "fwd_ms": r["fwd_ms"], "bwd_ms": r["bwd_ms"],
        "fwd_GBs": m["fwd_bytes"] / (r["fwd_ms"] * 1e6),
        "bwd_GBs": m["bwd_bytes"] / (r["bwd_ms"] * 1e6) if r["bwd_ms"] > 0 else None,
        "fwd_TFLOPs": m["fwd_flops"] / (r["fwd_ms"] * 1e9),
        "bwd_TFLOPs": m["bwd_flops"] / (r["bwd_ms"] * 1e9) if r["bwd_ms"] > 0 else None,
        "kernels": {"fwd": r["plan_fwd"], "bwd": r["plan_bwd"]},
        "event_ms_fwd_plus_bwd": fb,
    }
    if "fwd_ms_median" in r:
        out["warm_median_min_ms"] = {"fwd": [r["fwd_ms_median"], r["fwd_ms_min"]],
                                     "bwd": [r["bwd_ms_median"], r["bwd_ms_min"]] if r["bwd_ms"] > 0 else None}
    if r.get("cold") is not None:
        c = r["cold"]
        out["cold_cache"] = {"fwd_ms_median": c["fwd_ms_median"], "fwd_ms_min": c["fwd_ms_min"],
                             "bwd_ms_median": c.get("bwd_ms_median"), "bwd_ms_min": c.get("bwd_ms_min"),
                             "reps": c["reps"],
                             "how": "each call alone after a %d MiB fill evicts the L2s and the MALL"
                                    % (c["flush_bytes"] >> 20)}
    if "event_ms_per_step" in r:
        out["event_ms_per_step"] = r["event_ms_per_step"]
        out["per_call_events"] = "every %dth timed step (%d steps)" % (SAMPLE, r["sampled_steps"])
    return out, m


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "traffic.json")


def measured_traffic(workload, kernel):
    """HBM bytes per call of `kernel` (a plan name; "a+b" for a call of two
    launches) on `workload` from the committed rocprofv3 --pmc record
    (FETCH_SIZE and WRITE_SIZE in KiB per dispatch, each scaled by what the same
    counter reads for a plain 1 GiB device copy), or None when there is no
    record or the kernels changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        from sparse_causal_attention_amd.build import source_digest
        if rec.get("source_sha256") != source_digest():
            return None
        cf = rec["copy"]["bytes"] / (rec["copy"]["fetch_kib"] * 1024.0)
        cw = rec["copy"]["bytes"] / (rec["copy"]["write_kib"] * 1024.0)
        total = 0.0
        for name in kernel.split("+"):  # a call of several launches: their sum
            e = rec["kernels"][workload][name]
            total += (e["fetch_kib"] * cf + e["write_kib"] * cw) * 1024.0
        return int(round(total))
    except (OSError, KeyError, ValueError, TypeError, ZeroDivisionError):
        return None


COUNTER_RECORD = os.path.join(ROOT, "profiles", "counters.json")


def counter_mfma(workload, kernel, avg_ms):
    """Matrix-core work of `kernel` (a plan name, "a+b" for several launches)
    on `workload` from the committed rocprofv3 --pmc record: bf16 MFMA flops
    per call (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, per dispatch), those flops
    over `avg_ms` against the spec peak, and rocprofv3's own MfmaUtil and
    VALUBusy (percent of the kernel's time the matrix cores / vector ALUs are
    busy; for a call of several launches, the launch with the most MFMA work).
    None when there is no record or the kernels changed since."""
    try:
        rec = json.load(open(COUNTER_RECORD))
        from sparse_causal_attention_amd.build import source_digest
        if rec.get("source_sha256") != source_digest():
            return None
        ents = [rec["kernels"][workload][name] for name in kernel.split("+")]
        flops = 512.0 * sum(e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for e in ents)
        main = max(ents, key=lambda e: e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0))
        out = {"flops_per_call": flops,
               "mfma_bf16_frac": round(flops / (avg_ms * 1e9) / MFMA_BF16_PEAK_TFS, 4)}
        for key in ("MfmaUtil", "VALUBusy"):
            if key in main:
                out[key + "_pct"] = round(main[key], 2)
        return out
    except (OSError, KeyError, ValueError, TypeError, ZeroDivisionError):
        return None


RIDGE = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)  # flop per byte where the two roofs meet


def roofline_for(w, r, m, peaks=None):
    """Roofline entry for the longer of the two calls.  The bound is the roof
    the call's algorithmic intensity (flops over compulsory bytes) falls under:
    HBM below the ridge (MFMA peak / HBM peak = 312.5 flop/B), the bf16 matrix
    cores above it.  Against HBM the fraction is taken with the gather byte
    model; where that exceeds 1 (rows reused from cache), with the compulsory
    bytes instead, and `model` says which.  `peaks`: measured denominators
    (copy bandwidth, MFMA loop), reported beside the spec fractions."""
    use_bwd = r["bwd_ms"] > r["fwd_ms"]
    ms = r["bwd_ms"] if use_bwd else r["fwd_ms"]
    call = "bwd" if use_bwd else "fwd"
    byt_g = m[call + "_bytes"]
    byt_c = m[call + "_bytes_compulsory"]
    fl = m[call + "_flops"]
    kernel = r["plan_" + call]
    frac_g = byt_g / (ms * 1e6) / HBM_PEAK_GBS
    frac_c = byt_c / (ms * 1e6) / HBM_PEAK_GBS
    model = "gather" if frac_g <= 1.0 else "compulsory"
    byt = byt_g if model == "gather" else byt_c
    gbs = byt / (ms * 1e6)
    tfs = fl / (ms * 1e9)
    dot_mfma = kernel.startswith("band_")  # the band kernels run their products on the matrix cores
    intensity = fl / byt_c if byt_c else 0.0
    bound = "mfma" if dot_mfma and intensity > RIDGE else "hbm"
    if bound == "mfma":
        head = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(tfs / MFMA_BF16_PEAK_TFS, 4)}
    else:
        head = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    traffic = measured_traffic(w.name, kernel)
    out = dict(head)
    out.update({
        "traffic": traffic,
        "kernel": kernel,
        "call": "sa_" + call,
        "avg_ms": round(ms, 5), "algorithmic_bytes": byt, "model": model,
        "intensity_flop_per_byte": round(intensity, 1),
        "frac_gather_model": round(frac_g, 4), "frac_compulsory": round(frac_c, 4),
        "mfma_bf16_frac": round(tfs / MFMA_BF16_PEAK_TFS, 4) if dot_mfma else None,
    })
    if traffic:
        out["traffic_over_algorithmic"] = round(traffic / byt, 3)
        out["traffic_GBs"] = round(traffic / (ms * 1e6), 1)
    cm = counter_mfma(w.name, kernel, ms) if dot_mfma else None
    if cm:
        out["mfma_counters"] = cm
    if peaks:
        out["frac_of_measured_copy"] = round(gbs / peaks["copy_GBs"], 4)
        if dot_mfma:
            out["mfma_frac_of_measured_loop"] = round(tfs / peaks["mfma_bf16_TFs"], 4)
    return out


# ------------------------------------------------------------------ CPU baseline (oracle)
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inputs, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same inputs:
    whole (b, h) slices (forward + backward) until target_s seconds elapse on
    every host thread, then one slice on a single thread.  Scaled to tokens/s
    of the full workload."""
    import oracle
    from sparse_causal_attention_amd.inputs import host_view

    hv = {k: host_view(t) for k, t in inputs.items()}
    slices = [(b, h) for b in range(w.B) for h in range(w.H)]
    lists = None
    if w.graph == "lists":
        lists = oracle.graph_csr(w.T, w.window, w.offsets)
    elif w.graph == "random":
        lists = random_lists(w)

    def one_slice(b, h):
        if lists is not None:  # dot score over explicit lists
            oracle.fwd_csr(*lists, hv["v"][b, h], q=hv["q"][b, h], k=hv["k"][b, h])
            oracle.bwd_csr(*lists, hv["v"][b, h], hv["do"][b, h], q=hv["q"][b, h], k=hv["k"][b, h])
        elif w.uniform:
            oracle.fwd(w.T, w.window, w.offsets, hv["v"][b, h])
            oracle.bwd(w.T, w.window, w.offsets, hv["v"][b, h], hv["do"][b, h])
        elif w.coord:
            oracle.fwd(w.T, w.window, w.offsets, hv["v"][b, h], cq=hv["cq"][b, h], ck=hv["ck"][b, h],
                       gamma=float(hv["gamma"][h]), beta=float(hv["beta"][h]))
            oracle.bwd(w.T, w.window, w.offsets, hv["v"][b, h], hv["do"][b, h], cq=hv["cq"][b, h],
                       ck=hv["ck"][b, h], gamma=float(hv["gamma"][h]), beta=float(hv["beta"][h]))
        else:
            oracle.fwd(w.T, w.window, w.offsets, hv["v"][b, h], q=hv["q"][b, h], k=hv["k"][b, h])
            oracle.bwd(w.T, w.window, w.offsets, hv["v"][b, h], hv["do"][b, h], q=hv["q"][b, h],
                       k=hv["k"][b, h])

    threads = oracle.num_threads()
    done = 0
    t0 = time.perf_counter()
    while True:  # whole passes over the (batch, head) slices until target_s
        one_slice(*slices[done % len(slices)])
        done += 1
        if time.perf_counter() - t0 >= target_s:
            break
    el = time.perf_counter() - t0
    frac = done / len(slices)
    tokens_per_s = w.B * w.T * frac / el
    # one slice on one thread: how the oracle's rate scales with the host's cores
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    one_slice(*slices[0])
    el1 = time.perf_counter() - t1
    oracle.set_num_threads(threads)
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d (batch, head) slices (%.2f passes over the %d slices of the %s workload), "
                      "forward + backward, fp64, %.1f s; tokens/s scaled by the slice fraction"
                      % (done, frac, len(slices), w.name, el),
            "edges_per_s": edge_counts(w)[0] * done / el,
            "single_thread": {"value": w.B * w.T / len(slices) / el1, "unit": "tokens/s",
                              "sample": "1 slice, %.1f s" % el1},
            "cpu_model": cpu_model()}


_PROBE = None


def probe_lib():
    """libsa_probe.so (include/sa_probe.h): copy, MFMA-loop and empty-launch
    probes built beside libsa.so."""
    global _PROBE
    if _PROBE is None:
        import ctypes
        path = os.path.join(ROOT, "sparse_causal_attention_amd", "libsa_probe.so")
        if not os.path.exists(path):
            raise ImportError("libsa_probe.so is not built; run python -m sparse_causal_attention_amd.build")
        L = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        L.sa_probe_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        L.sa_probe_mfma.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
        L.sa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
        L.sa_probe_empty.argtypes = [vp]
        ip = ctypes.POINTER(ctypes.c_int)
        L.sa_probe_mix_variants.argtypes = []
        L.sa_probe_mix_counts.argtypes = [ctypes.c_int, ip, ip, ip]
        L.sa_probe_mix.argtypes = [ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp]
        _PROBE = L
    return _PROBE


def _stream_handle():
    import ctypes
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


COPY_PROBE_BYTES = 1 << 30


def probe_rates(iters=512, reps=5):
    """The issue-rate probes (include/sa_probe.h), four workgroups of four
    wavefronts per compute unit, so each SIMD processes four wavefronts'
    rounds.  Per variant: the launch's HIP-event time per round (median of
    `reps` launches after one warm-up launch), i.e. one SIMD's time for four
    rounds, and the shader clock from the wavefronts' s_memtime against
    s_memrealtime (100 MHz) ticks; cycles = time x clock.  Comparing the
    MFMA-only, FMA-only and mixed rounds shows how far the matrix core and the
    vector ALU overlap; the per-instruction figures are cycles / (4 x count)
    for the single-kind rounds.  (The wavefronts of a SIMD do not all run
    side by side for the whole launch, so per-wavefront spans are not used.)"""
    import ctypes
    import torch
    L = probe_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 4 * cus
    out = torch.empty(16 * blocks, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def launch(v):
        assert L.sa_probe_mix(v, ctypes.c_void_p(out.data_ptr()), blocks, iters, _stream_handle()) == 0

    rows = []
    for v in range(L.sa_probe_mix_variants()):
        nm, nf, ne = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        assert L.sa_probe_mix_counts(v, ctypes.byref(nm), ctypes.byref(nf), ctypes.byref(ne)) == 0
        launch(v)
        torch.cuda.synchronize()
        ns, ghz = [], []
        for _ in range(reps):
            e0.record()
            launch(v)
            e1.record()
            torch.cuda.synchronize()
            ns.append(e0.elapsed_time(e1) * 1e6 / iters)
            w = out.view(-1, 4).double()
            ghz.append(float((w[:, 0] / (w[:, 1] * 10.0)).median()))  # memtime ticks per ns
        ns.sort()
        ghz.sort()
        t, f = ns[len(ns) // 2], ghz[len(ghz) // 2]
        rows.append({"mfma": nm.value, "fma": nf.value, "exp": ne.value, "ns_per_round": round(t, 1),
                     "shader_ghz": round(f, 3), "simd_cycles_per_round": round(t * f, 1)})
    per = {}
    for r in rows:
        kinds = [k for k in ("mfma", "fma", "exp") if r[k]]
        if len(kinds) == 1:
            per[kinds[0]] = round(r["simd_cycles_per_round"] / (4 * r[kinds[0]]), 2)
    return {"probe": "issue rates", "workgroups_per_cu": 4, "wavefronts_per_simd": 4, "iters": iters,
            "rounds": rows, "simd_cycles_per_wavefront_instruction": per}


def copy_probe(reps=3):
    """The probe's plain 1 GiB device copy (the counters' scale reference):
    returns the median copy time in ms over `reps` launches."""
    import ctypes
    import torch
    L = probe_lib()
    a = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        assert L.sa_probe_copy(ctypes.c_void_p(b.data_ptr()), ctypes.c_void_p(a.data_ptr()), COPY_PROBE_BYTES,
                               _stream_handle()) == 0
        e[1].record()
        torch.cuda.synchronize()
        ms.append(e[0].elapsed_time(e[1]))
    del a, b
    return median(ms)


def measured_peaks():
    """Measured denominators beside the published peaks: a plain device copy
    (read + write bytes over its time), a loop of independent bf16 MFMAs, and
    an empty launch (alone between two events, and back to back)."""
    import ctypes
    import torch
    L = probe_lib()
    copy_probe(2)  # warm
    copy_ms = copy_probe(5)
    blocks, iters = 256 * 8, 2000
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    fl = ctypes.c_double()
    L.sa_probe_mfma_flops(blocks, iters, ctypes.byref(fl))
    ms = []
    for r in range(6):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        assert L.sa_probe_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, _stream_handle()) == 0
        e[1].record()
        torch.cuda.synchronize()
        if r:
            ms.append(e[0].elapsed_time(e[1]))
    mfma_ms = median(ms)
    alone = []
    for _ in range(50):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        L.sa_probe_empty(_stream_handle())
        e[1].record()
        torch.cuda.synchronize()
        alone.append(e[0].elapsed_time(e[1]))
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    for _ in range(200):
        L.sa_probe_empty(_stream_handle())
    e[1].record()
    torch.cuda.synchronize()
    return {"copy_GBs": round(2 * COPY_PROBE_BYTES / (copy_ms * 1e6), 1),
            "copy_how": "probe copy kernel, 1 GiB read + 1 GiB written, median of 5",
            "mfma_bf16_TFs": round(fl.value / (mfma_ms * 1e9), 1),
            "mfma_how": "%d workgroups x 4 wavefronts x 4 independent chains x %d v_mfma_f32_32x32x16_bf16, "
                        "median of 5" % (blocks, iters),
            "empty_launch_us": round(1e3 * median(alone), 2),
            "empty_launch_us_back_to_back": round(1e3 * e[0].elapsed_time(e[1]) / 200, 2),
            "spec": {"hbm_GBs": HBM_PEAK_GBS, "mfma_bf16_TFs": MFMA_BF16_PEAK_TFS}}


# ------------------------------------------------------------------ profile records
# The rocprofv3 runs behind profiles/ (each from /tmp with TMPDIR=/tmp, one
# bench process per workload, into <dir>/<workload>/<pass>), and the bench
# command each profiles.  `python bench.py --record-profiles <dir>` turns their
# CSV output into profiles/<family>__<workload>.txt (kernel-trace statistics),
# profiles/counters__<workload>.txt and the JSON records bench.py reads back
# (profiles/traffic.json, profiles/counters.json).
PROFILE_PASSES = {
    "trace": ("rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/<workload>/trace -o run --",
              "--steps 10 --warmup 2 --no-cpu-baseline --no-cold --no-peaks"),
    "fetch": ("rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/<workload>/fetch -o run --",
              "--steps 3 --warmup 1 --no-cpu-baseline --no-cold --no-peaks --copy-probe"),
    "write": ("rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/<workload>/write -o run --",
              "--steps 3 --warmup 1 --no-cpu-baseline --no-cold --no-peaks --copy-probe"),
    "mfma": ("rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 MfmaUtil VALUBusy --output-format csv "
             "-d <dir>/<workload>/mfma -o run --",
             "--steps 3 --warmup 1 --no-cpu-baseline --no-cold --no-peaks"),
    "insts": ("rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INSTS_LDS SQ_INSTS_SALU SQ_INSTS_MFMA SQ_WAVES "
              "--output-format csv -d <dir>/<workload>/insts -o run --",
              "--steps 3 --warmup 1 --no-cpu-baseline --no-cold --no-peaks"),
    "loadpath": ("rocprofv3 --pmc TA_TA_BUSY_sum TA_DATA_STALLED_BY_TC_CYCLES_sum TCC_HIT_sum TCC_MISS_sum "
                 "GRBM_GUI_ACTIVE --output-format csv -d <dir>/<workload>/loadpath -o run --",
                 "--steps 3 --warmup 1 --no-cpu-baseline --no-cold --no-peaks"),
}
# Per-dispatch counters kept in profiles/counters.json (besides FETCH_SIZE and
# WRITE_SIZE, which go to profiles/traffic.json).
COUNTER_KEYS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "MfmaUtil", "VALUBusy", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD",
                "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_INSTS_MFMA", "SQ_WAVES", "TA_TA_BUSY_sum",
                "TA_DATA_STALLED_BY_TC_CYCLES_sum", "TCC_HIT_sum", "TCC_MISS_sum", "GRBM_GUI_ACTIVE")
CUS, XCDS, SIMDS = 256, 8, 1024  # MI355X: compute units, accelerator dies, SIMDs


def profile_command(pass_name, workload):
    tool, args = PROFILE_PASSES[pass_name]
    return "%s python3 <repo>/bench.py %s --workloads %s" % (tool.replace("<workload>", workload), args, workload)


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _plain_name(full):
    """'void sa::(anonymous namespace)::band_fwd_kernel<false, 1>(sa::Params)'
    -> 'band_fwd_kernel<false, 1>' (the name with its template arguments and
    without namespaces, return type or parameter list)."""
    name = full.replace("(anonymous namespace)", "")
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # the parameter list starts at the first '(' outside <...>
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = i
            break
    name = name[:cut]
    head = name.split("<", 1)[0]
    return head.split("::")[-1] + (name[len(head):] if "<" in name else "")


def _plan_names(workload):
    """Plan names of the workload's calls, each with the symbol prefix of its
    kernel, in launch order (forward first)."""
    from sparse_causal_attention_amd.inputs import WORKLOADS
    w = WORKLOADS[workload]
    if w.decode:
        return ["decode_kernel(dot)"]
    import torch

    from sparse_causal_attention_amd import sa_describe_plan
    g = make_graph(w)
    v = torch.empty((w.B, w.kv_heads, w.T, w.D), dtype=w.dtype, device="meta")  # shape only, no memory
    plans = sa_describe_plan(g, v, score=score_name(w), which="fwd", heads=w.H).split("+")
    if w.backward:
        plans += sa_describe_plan(g, v, score=score_name(w), which="bwd", heads=w.H).split("+")
    return plans


def _symbol_plan(symbol, plans):
    """The plan name a kernel symbol belongs to: the plan whose kernel name
    the symbol starts with (for a family launched once per call)."""
    base = symbol.split("<")[0]
    for pl in plans:
        if pl.split("(")[0] == base:
            return pl
    return None


def record_profiles(root):
    """Reads <root>/<workload>/{trace,fetch,write,mfma}/run_*.csv and writes
    the profile summaries and records under profiles/."""
    from sparse_causal_attention_amd.build import source_digest
    from sparse_causal_attention_amd.inputs import WORKLOADS
    prof = os.path.join(ROOT, "profiles")
    digest = source_digest()
    traffic = {"source_sha256": digest,
               "note": "FETCH_SIZE and WRITE_SIZE in KiB per dispatch (mean over dispatches), from two rocprofv3 "
                       "--pmc runs per workload; copy = the probe's plain 1 GiB device copy in the same process, "
                       "used to scale each counter to bytes",
               "commands": {p: profile_command(p, "<workload>") for p in ("fetch", "write")},
               "copy": None, "kernels": {}}
    counters = {"source_sha256": digest,
                "note": "per dispatch means: SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 MFMA flops / 512), MfmaUtil and "
                        "VALUBusy (rocprofv3 derived metrics, percent), instruction counts (wavefront "
                        "instructions, summed over the GPU), TA_TA_BUSY_sum (texture-addresser busy cycles "
                        "summed over the 256 compute units), TCC hits and misses, GRBM_GUI_ACTIVE (GPU-busy "
                        "cycles summed over the 8 dies)",
                "commands": {p: profile_command(p, "<workload>") for p in ("mfma", "insts", "loadpath")},
                "kernels": {}}
    for workload in sorted(os.listdir(root)):
        wdir = os.path.join(root, workload)
        if workload not in WORKLOADS or not os.path.isdir(wdir):
            continue
        w = WORKLOADS[workload]
        plans = _plan_names(workload)
        # kernel trace statistics
        stats = os.path.join(wdir, "trace", "run_kernel_stats.csv")
        if os.path.exists(stats):
            rows = [r for r in _csv_rows(stats) if "sa::" in r["Name"]]
            fam = {"band": "band_kernels", "gather": "gather_kernels", "csr": "csr_kernels",
                   "decode": "decode_kernel"}[plans[0].split("_")[0]]
            lines = ["# rocprofv3 kernel-trace statistics, %s: B=%d H=%d H_kv=%d T=%d D=%d W=%d offsets=%s %s %s "
                     "score, %s" % (workload, w.B, w.H, w.kv_heads, w.T, w.D, w.window, list(w.offsets),
                                    w.dtype_name, score_name(w), "fwd+bwd" if w.backward else "fwd"),
                     "# one MI355X (gfx950); calls per kernel = warm-up + timed steps of bench.py",
                     "# command, run from /tmp with TMPDIR=/tmp on the repository as committed:",
                     "#   " + profile_command("trace", workload),
                     "# libsa.so source sha256: " + digest,
                     "%-64s %6s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
            for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
                lines.append("%-64s %6d %12.2f %12.2f %12.2f" % (
                    _plain_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                    float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
            open(os.path.join(prof, "%s__%s.txt" % (fam, workload)), "w").write("\n".join(lines) + "\n")
        # counters: mean per dispatch of each counter per kernel symbol
        per = {}
        for pass_name in ("fetch", "write", "mfma", "insts", "loadpath"):
            path = os.path.join(wdir, pass_name, "run_counter_collection.csv")
            if not os.path.exists(path):
                continue
            acc = {}
            for r in _csv_rows(path):
                key = (_plain_name(r["Kernel_Name"]), r["Counter_Name"])
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
            for (sym, cname), vals in acc.items():
                per.setdefault(sym, {})[cname] = sum(vals) / len(vals)
        copy = per.get("probe_copy_kernel")
        if copy and "FETCH_SIZE" in copy and "WRITE_SIZE" in copy and traffic["copy"] is None:
            traffic["copy"] = {"bytes": COPY_PROBE_BYTES, "fetch_kib": copy["FETCH_SIZE"],
                               "write_kib": copy["WRITE_SIZE"], "workload_run": workload}
        for sym, vals in per.items():
            plan = _symbol_plan(sym, plans)
            if plan is None:
                continue
            if "FETCH_SIZE" in vals and "WRITE_SIZE" in vals:
                traffic["kernels"].setdefault(workload, {})[plan] = {
                    "fetch_kib": vals["FETCH_SIZE"], "write_kib": vals["WRITE_SIZE"], "symbol": sym}
            m = {k: vals[k] for k in COUNTER_KEYS if k in vals}
            if m:
                counters["kernels"].setdefault(workload, {})[plan] = dict(m, symbol=sym)
    json.dump(traffic, open(os.path.join(prof, "traffic.json"), "w"), indent=1)
    json.dump(counters, open(os.path.join(prof, "counters.json"), "w"), indent=1)
    # a readable summary per workload
    cf = cw = None
    if traffic["copy"]:
        cf = traffic["copy"]["bytes"] / (traffic["copy"]["fetch_kib"] * 1024.0)
        cw = traffic["copy"]["bytes"] / (traffic["copy"]["write_kib"] * 1024.0)
    for workload in sorted(set(traffic["kernels"]) | set(counters["kernels"])):
        lines = ["# rocprofv3 --pmc counters per dispatch, workload %s, one MI355X (gfx950)" % workload,
                 "# commands (from /tmp, TMPDIR=/tmp, on the repository as committed):"]
        for p in ("fetch", "write", "mfma", "insts", "loadpath"):
            lines.append("#   " + profile_command(p, workload))
        lines.append("# libsa.so source sha256: " + digest)
        if cf:
            lines.append("# bytes = FETCH_SIZE KiB x 1024 x %.4f + WRITE_SIZE KiB x 1024 x %.4f (the probe's 1 GiB "
                         "copy reads %.1f / %.1f KiB on these counters)" % (
                             cf, cw, traffic["copy"]["fetch_kib"], traffic["copy"]["write_kib"]))
        lines.append("%-34s %14s %14s %12s %16s %10s %10s" % ("kernel (plan name)", "FETCH_SIZE_KiB",
                                                             "WRITE_SIZE_KiB", "HBM_MB", "MFMA_bf16_GFLOP",
                                                             "MfmaUtil%", "VALUBusy%"))
        names = sorted(set(traffic["kernels"].get(workload, {})) | set(counters["kernels"].get(workload, {})))
        for plan in names:
            t = traffic["kernels"].get(workload, {}).get(plan, {})
            c = counters["kernels"].get(workload, {}).get(plan, {})
            hbm = (t["fetch_kib"] * cf + t["write_kib"] * cw) * 1024 / 1e6 if (t and cf) else float("nan")
            lines.append("%-34s %14.1f %14.1f %12.2f %16.3f %10.2f %10.2f" % (
                plan, t.get("fetch_kib", float("nan")), t.get("write_kib", float("nan")), hbm,
                512 * c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", float("nan")) / 1e9,
                c.get("MfmaUtil", float("nan")), c.get("VALUBusy", float("nan"))))
        # issue and load-path figures: per SIMD instruction counts, and the texture addresser's
        # busy fraction = TA_TA_BUSY_sum / CUs over GRBM_GUI_ACTIVE / dies
        # TA_floor%: the share of the kernel's time the texture addresser would need at its nominal
        # 16 cycles per 64-lane load instruction (64 B per cycle for 16-byte lanes)
        lines.append("%-34s %12s %12s %10s %10s %10s %9s %9s %9s" % (
            "kernel (plan name)", "VALU/SIMD", "VMEM_RD/SIMD", "LDS/SIMD", "SALU/SIMD", "MFMA/SIMD",
            "TA_busy%", "TA_floor%", "L2_hit%"))
        for plan in names:
            c = counters["kernels"].get(workload, {}).get(plan, {})
            if "SQ_INSTS_VALU" not in c:
                continue
            ta = (100.0 * c["TA_TA_BUSY_sum"] / CUS / (c["GRBM_GUI_ACTIVE"] / XCDS)
                  if c.get("GRBM_GUI_ACTIVE") and "TA_TA_BUSY_sum" in c else float("nan"))
            floor = (100.0 * c.get("SQ_INSTS_VMEM_RD", 0.0) * 16 / CUS / (c["GRBM_GUI_ACTIVE"] / XCDS)
                     if c.get("GRBM_GUI_ACTIVE") else float("nan"))
            hm = c.get("TCC_HIT_sum", 0.0) + c.get("TCC_MISS_sum", 0.0)
            l2 = 100.0 * c["TCC_HIT_sum"] / hm if hm else float("nan")
            lines.append("%-34s %12.0f %12.0f %10.0f %10.0f %10.0f %9.1f %9.1f %9.1f" % (
                plan, c["SQ_INSTS_VALU"] / SIMDS, c.get("SQ_INSTS_VMEM_RD", 0.0) / SIMDS,
                c.get("SQ_INSTS_LDS", 0.0) / SIMDS, c.get("SQ_INSTS_SALU", 0.0) / SIMDS,
                c.get("SQ_INSTS_MFMA", 0.0) / SIMDS, ta, floor, l2))
        open(os.path.join(prof, "counters__%s.txt" % workload), "w").write("\n".join(lines) + "\n")


# Workloads the oracle is also timed on (besides the headline): the dilated
# training shape, its coordinate-score variant and the tiny fp32 case (CPU
# only), each with a single-thread slice.
CPU_EXTRA = ("dilated", "coord", "tiny")
CPU_EXTRA_SECONDS = 6.0

# Order of the compact per-workload summary that closes the JSON line: the
# configurations the metric is quoted on come last.
SUMMARY_LAST = ("band", "dilated", "coord", "ultra")


def summary_order(names):
    """Workload names with the configurations the metric is quoted on last."""
    return [n for n in names if n not in SUMMARY_LAST] + [n for n in SUMMARY_LAST if n in names]


def compact(s):
    """One short entry per workload for the end of the line."""
    rf = s["roofline"]
    e = {"tok_s": round(s["tokens_per_s"], 1), "edges_s": round(s["edges_per_s"], 1),
         "fwd_us": round(1e3 * s["fwd_ms"], 1), "bwd_us": round(1e3 * s["bwd_ms"], 1),
         "bound": rf["bound"], "frac": rf["frac"], "model": rf["model"],
         "frac_compulsory": rf["frac_compulsory"]}
    if rf.get("traffic"):
        e["traffic_ratio"] = rf["traffic_over_algorithmic"]
    if rf.get("mfma_bf16_frac") is not None:
        e["mfma_frac"] = rf["mfma_bf16_frac"]
    if rf.get("mfma_counters"):
        e["mfma_frac_counters"] = rf["mfma_counters"]["mfma_bf16_frac"]
        if "MfmaUtil_pct" in rf["mfma_counters"]:
            e["MfmaUtil_pct"] = rf["mfma_counters"]["MfmaUtil_pct"]
    return e


def main():
    args = parse()
    if args.record_profiles:
        record_profiles(args.record_profiles)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.stderr.write("bench.py measures one GPU only: the library has no multi-GPU path "
                         "(independent (batch, head) slices would shard without communication; "
                         "see the sharding notes in the design document).\n")
        sys.exit(2)
    import torch

    from sparse_causal_attention_amd import _abi
    from sparse_causal_attention_amd.inputs import WORKLOADS, make_inputs

    _abi.lib()
    if args.probe_rates:
        print(json.dumps(probe_rates()))
        return
    if args.sweep:
        print(json.dumps(sweep()))
        return
    if args.copy_probe:
        copy_probe()
    peaks = None
    if not args.no_peaks:
        print("[bench] measured peaks (copy, MFMA loop, empty launch)", file=sys.stderr, flush=True)
        peaks = measured_peaks()
    names = [n for n in args.workloads.split(",") if n]
    headline = names[0]
    results = {}
    host_inputs = {}
    for name in names:
        w = WORKLOADS[name]
        long_t = w.T > (1 << 24)  # the 2^26-token workloads: tens of ms per call
        steps = args.steps if not long_t else max(2, min(args.steps, 5))
        warm = args.warmup if not long_t else min(args.warmup, 2)
        if w.decode:
            steps, warm = max(steps, 200), max(warm, 20)  # microsecond steps
        print("[bench] %s: %d warmup + %d timed steps" % (name, warm, steps), file=sys.stderr, flush=True)
        r = (run_decode(w, steps, warm, args.no_cold) if w.decode
             else run_workload(w, steps, warm, args.algo, no_cold=args.no_cold))
        s, m = summarize(w, r, steps)
        s["roofline"] = roofline_for(w, r, m, peaks)
        s["steps"] = steps
        if w.decode and peaks:
            s["launch_floor_us"] = peaks["empty_launch_us"]
            s["over_launch_floor"] = round(1e3 * r["fwd_ms"] / peaks["empty_launch_us"], 2)
        results[name] = (w, r, s)
        if name != headline:
            if name in CPU_EXTRA and not args.no_cpu_baseline:
                host_inputs[name] = {k: t.cpu() for k, t in r["inputs"].items()}
            del r["inputs"]
            torch.cuda.empty_cache()
    w, r, s = results[headline]
    line = {
        "metric": METRIC,
        "value": s["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": s["steps"],
        "warmup": args.warmup,
        "ms_per_step": s["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype_name,
        "data": "synthetic: seeded N(0,1) inputs shaped like the pages' workloads",
        "config": {"workload": "%s: B=%d H=%d T=%d D=%d W=%d offsets=%s %s, %s" % (
            w.name, w.B, w.H, w.T, w.D, w.window, list(w.offsets), w.dtype_name,
            "fwd+bwd" if w.backward else "fwd"),
            "global_batch": w.B, "seq_len": w.T, "heads": w.H, "head_dim": w.D},
        "edges_per_s": s["edges_per_s"],
        "roofline": s["roofline"],
        "measured_peaks": peaks,
        "detail": {k: v for k, v in s.items() if k not in ("roofline",)},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) on %s" % w.name, file=sys.stderr, flush=True)
        cb = cpu_baseline(w, r["inputs"], args.cpu_seconds)
        others = {}
        for name in CPU_EXTRA:
            wx = WORKLOADS[name]
            xin = host_inputs.get(name)
            if xin is None and name not in results:
                xin = make_inputs(wx)  # a workload the GPU leg did not run (the tiny fp32 case)
            if xin is None:
                continue
            print("[bench] cpu baseline (oracle) on %s" % name, file=sys.stderr, flush=True)
            c = cpu_baseline(wx, xin, CPU_EXTRA_SECONDS)
            if name in results:
                c["gpu_over_cpu"] = round(results[name][2]["tokens_per_s"] / c["value"], 1)
            others[name] = c
        cb["other_workloads"] = others
        line["cpu_baseline"] = cb
    else:
        line["cpu_baseline"] = None
    line["extra"] = {n: s2 for n, (_, _, s2) in results.items() if n != headline}
    line["summary"] = {n: compact(results[n][2]) for n in summary_order(list(results))}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

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
                    default="band,dilated,coord,uniform,band_gqa,dilated_gqa,csr_dilated,csr_random,decode_band,decode_dilated,ultra")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample length")
    ap.add_argument("--algo", default="auto")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache repetitions (profiled runs: keeps per-kernel averages warm)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (scales profiler byte counters)")
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
        grads = {"dv": torch.empty(kvshape, dtype=torch.float32, device=dev)}
        if coord:
            grads.update(dcq=torch.empty((w.B, w.H, w.T, 3), dtype=torch.float32, device=dev),
                         dck=torch.empty((w.B, w.H, w.T, 3), dtype=torch.float32, device=dev),
                         dgamma=torch.empty((w.H,), dtype=torch.float32, device=dev),
                         dbeta=torch.empty((w.H,), dtype=torch.float32, device=dev))
        elif not w.uniform:
            grads.update(dq=torch.empty(gshape, dtype=torch.float32, device=dev),
                         dk=torch.empty(kvshape, dtype=torch.float32, device=dev))
        from sparse_causal_attention_amd import sa_bwd_workspace_size
        ws = torch.empty(sa_bwd_workspace_size(g, x["v"], heads=w.H), dtype=torch.uint8, device=dev)
        bkw = dict(v=x["v"], o=o, lse=lse, dout=x["do"], cq=x.get("cq"), ck=x.get("ck"),
                   gamma=x.get("gamma"), beta=x.get("beta"), workspace=ws, algo=algo, **grads)
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
    m = models(w)
    tokens = w.B if w.decode else w.B * w.T  # a decode step makes one token per sequence
    fb = r["fwd_ms"] + r["bwd_ms"]
    wall = r["wall_s"]
    out = {
        "workload": w.name,
        "shape": {"B": w.B, "H": w.H, "H_kv": w.kv_heads, "T": w.T, "D": w.D, "window": w.window,
                  "offsets": list(w.offsets), "graph": w.graph, "dtype": w.dtype_name,
                  "score": score_name(w), "backward": w.backward},
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


def roofline_for(w, r, m):
    """Roofline entry for the longer of the two calls.  The fraction is taken
    against the gather byte model; where that exceeds 1 (rows reused from
    cache), against the compulsory bytes instead, and `model` says which."""
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
    achieved = byt / (ms * 1e6)
    return {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name, kernel),
        "kernel": kernel,
        "call": "sa_" + call,
        "avg_ms": round(ms, 5), "algorithmic_bytes": byt, "model": model,
        "frac_gather_model": round(frac_g, 4), "frac_compulsory": round(frac_c, 4),
        "mfma_bf16_frac": round(fl / (ms * 1e9) / MFMA_BF16_PEAK_TFS, 4),
    }


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


def copy_probe():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.stderr.write("bench.py measures one GPU only: this build has no multi-GPU path "
                         "(independent (batch, head) slices would shard without communication; "
                         "see the sharding notes in the design document).\n")
        sys.exit(2)
    import torch

    from sparse_causal_attention_amd import _abi
    from sparse_causal_attention_amd.inputs import WORKLOADS

    _abi.lib()
    if args.copy_probe:
        copy_probe()
    names = [n for n in args.workloads.split(",") if n]
    headline = names[0]
    results = {}
    for name in names:
        w = WORKLOADS[name]
        steps = args.steps if name != "ultra" else max(2, min(args.steps, 5))
        warm = args.warmup if name != "ultra" else min(args.warmup, 2)
        if w.decode:
            steps, warm = max(steps, 200), max(warm, 20)  # microsecond steps
        print("[bench] %s: %d warmup + %d timed steps" % (name, warm, steps), file=sys.stderr, flush=True)
        r = (run_decode(w, steps, warm, args.no_cold) if w.decode
             else run_workload(w, steps, warm, args.algo, no_cold=args.no_cold))
        s, m = summarize(w, r, steps)
        s["roofline"] = roofline_for(w, r, m)
        s["steps"] = steps
        results[name] = (w, r, s)
        if name != headline:
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
        "detail": {k: v for k, v in s.items() if k not in ("roofline",)},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) on %s" % w.name, file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, r["inputs"], args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    line["extra"] = {n: s2 for n, (_, _, s2) in results.items() if n != headline}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

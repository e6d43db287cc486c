"""The bench's work models on the CPU: edge counts from the closed form, and
the per-call byte and flop figures at the five workloads (edge set and
algorithmic work as defined by the neighbour graph: window {i-W+1..i} plus
the long-range distances, each tensor once plus the rows fetched per
long-range edge)."""
import bench
from sparse_causal_attention_amd.inputs import WORKLOADS

import oracle


def test_edge_counts_match_set_union_on_small_graph():
    # the oracle's per-row set union, summed, equals the bench's closed form
    from types import SimpleNamespace
    for T, W, offs in [(256, 8, (16, 32, 64, 128)), (100, 3, (1, 2, 4, 8, 16, 32, 64, 128)), (50, 64, ())]:
        w = SimpleNamespace(T=T, window=W, offsets=offs, graph="distance")
        total = sum(len(oracle.row(T, W, offs, i)) for i in range(T))
        long_range = sum(1 for i in range(T) for d in sorted(set(offs)) if min(W, T) <= d < T and i - d >= 0)
        assert bench.edge_counts(w) == (total, long_range)


def test_models_at_the_workloads():
    MB = 1e6
    band = bench.models(WORKLOADS["band"])
    assert band["edges"] == 8 * 4161664
    assert round(band["fwd_bytes"] / MB, 1) == 67.6 and round(band["bwd_bytes"] / MB, 1) == 185.1
    assert band["fwd_bytes"] == band["fwd_bytes_compulsory"]  # no long-range edges
    assert round(band["fwd_flops"] / 1e9, 2) == 8.52 and round(band["bwd_flops"] / 1e9, 2) == 21.31
    dil = bench.models(WORKLOADS["dilated"])
    assert dil["edges"] == 32 * 245758
    assert round(dil["fwd_bytes_compulsory"] / MB, 1) == 270.5
    assert round(dil["bwd_bytes_compulsory"] / MB, 1) == 740.3
    # 32 slices x 180,228 long-range edges x (K + V rows of 128 B)
    assert dil["fwd_bytes"] - dil["fwd_bytes_compulsory"] == 32 * 180228 * 256
    assert dil["bwd_bytes"] - dil["bwd_bytes_compulsory"] == 32 * 180228 * 520
    ultra = bench.models(WORKLOADS["ultra"])
    assert ultra["edges"] == 5570033760


def test_roofline_switches_to_compulsory_above_one():
    w = WORKLOADS["dilated"]
    m = bench.models(w)
    # a forward call fast enough that the gather model would exceed the peak
    r = {"fwd_ms": 0.1, "bwd_ms": 0.0, "plan_fwd": "k", "plan_bwd": None}
    e = bench.roofline_for(w, r, m)
    assert e["model"] == "compulsory" and e["frac_gather_model"] > 1.0
    assert abs(e["frac"] - m["fwd_bytes_compulsory"] / 0.1e6 / bench.HBM_PEAK_GBS) < 1e-4
    r = {"fwd_ms": 1.0, "bwd_ms": 0.0, "plan_fwd": "k", "plan_bwd": None}
    assert bench.roofline_for(w, r, m)["model"] == "gather"


def test_models_uniform_mode():
    """Fixed equal weights read v alone: the forward moves v, o, lse per row
    and one v row per long-range edge; the backward dout, lse, dv per row and
    the dout row and lse per long-range edge; 2D flops per edge each way."""
    m = bench.models(WORKLOADS["uniform"])
    rows = 4 * 8 * 16384
    assert m["fwd_bytes_compulsory"] == rows * (2 * 128 + 4)
    assert m["bwd_bytes_compulsory"] == rows * (128 + 4 + 256)
    assert m["fwd_bytes"] - m["fwd_bytes_compulsory"] == 32 * 180228 * 128
    assert m["fwd_flops"] == m["bwd_flops"] == 32 * 245758 * 2 * 64


def test_models_grouped_heads():
    """With 8 query heads on 2 key/value heads the k, v, dk, dv tensors shrink
    by 4; per long-range edge the rows fetched stay the same."""
    full, gqa = bench.models(WORKLOADS["band"]), bench.models(WORKLOADS["band_gqa"])
    rows, kv_rows = 8 * 16384, 2 * 16384
    assert gqa["fwd_bytes_compulsory"] == rows * (2 * 128 + 4) + kv_rows * 2 * 128
    assert gqa["bwd_bytes_compulsory"] == rows * (3 * 128 + 4 + 256) + kv_rows * (2 * 128 + 2 * 256)
    assert full["fwd_flops"] == gqa["fwd_flops"]
    d, dg = bench.models(WORKLOADS["dilated"]), bench.models(WORKLOADS["dilated_gqa"])
    assert d["fwd_bytes"] - d["fwd_bytes_compulsory"] == dg["fwd_bytes"] - dg["fwd_bytes_compulsory"]


def test_models_explicit_lists():
    """The dilated graph as lists has the dilated edge counts and bytes plus
    the int32 lists (once forward, forward + reverse backward); random lists
    count their own edges, every edge beyond the window being gathered."""
    dil, lst = bench.models(WORKLOADS["dilated"]), bench.models(WORKLOADS["csr_dilated"])
    w = WORKLOADS["csr_dilated"]
    E = 245758
    assert lst["edges"] == dil["edges"]
    assert lst["fwd_bytes"] - dil["fwd_bytes"] == 4 * (w.T + 1) + 4 * E
    assert lst["bwd_bytes"] - dil["bwd_bytes"] == 2 * (4 * (w.T + 1) + 4 * E)
    r = WORKLOADS["csr_random"]
    rp, cols = bench.random_lists(r)
    total, far = bench.edge_counts(r)
    assert total == len(cols) == rp[-1]
    window = sum(min(i + 1, r.window) for i in range(r.T))
    assert far == total - window
    assert bench.models(r)["edges"] == r.B * r.H * total


def test_summary_carries_warm_and_cold_figures():
    """The JSON detail reports warm medians and minima and the cold-cache
    block beside the means; `value` stays on the warm wall-clock rate."""
    w = WORKLOADS["band"]
    r = {"wall_s": 0.02, "ms_per_step": 0.1, "fwd_ms": 0.025, "bwd_ms": 0.075,
         "fwd_ms_min": 0.02, "bwd_ms_min": 0.07, "fwd_ms_median": 0.024, "bwd_ms_median": 0.074,
         "cold": {"reps": 10, "flush_bytes": 1 << 30, "fwd_ms_median": 0.03, "fwd_ms_min": 0.029,
                  "bwd_ms_median": 0.09, "bwd_ms_min": 0.088},
         "plan_fwd": "band_fwd_kernel", "plan_bwd": "band_bwd_prepass_kernel+band_bwd_kernel"}
    s, _ = bench.summarize(w, r, 200)
    assert s["warm_median_min_ms"] == {"fwd": [0.024, 0.02], "bwd": [0.074, 0.07]}
    c = s["cold_cache"]
    assert (c["fwd_ms_median"], c["bwd_ms_min"], c["reps"]) == (0.03, 0.088, 10)
    assert "1024 MiB" in c["how"]
    assert abs(s["tokens_per_s"] - w.B * w.T * 200 / 0.02) < 1e-3
    # a run without the cold leg (profiled runs) reports none
    r["cold"] = None
    s, _ = bench.summarize(w, r, 200)
    assert "cold_cache" not in s


def test_median():
    assert bench.median([3.0, 1.0, 2.0]) == 2.0
    assert bench.median([4.0, 1.0, 2.0, 3.0]) == 2.5


def test_roofline_bound_follows_intensity():
    """The roof is the one the call's intensity (flops over compulsory bytes)
    falls under: the band workload (W = 256, about 115-126 flop/B) sits under
    the HBM roof, the dense W = T = 2048 variant (about 500 flop/B) above the
    ridge of 312.5 flop/B, under the bf16 matrix-core roof; the gather
    kernels report no matrix-core fraction."""
    assert abs(bench.RIDGE - 312.5) < 1e-9
    band = WORKLOADS["band"]
    r = {"fwd_ms": 0.02, "bwd_ms": 0.07, "plan_fwd": "band_fwd_kernel",
         "plan_bwd": "band_bwd_prepass_kernel+band_bwd_kernel"}
    e = bench.roofline_for(band, r, bench.models(band))
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["intensity_flop_per_byte"] < bench.RIDGE
    assert e["mfma_bf16_frac"] is not None
    dense = WORKLOADS["band_dense"]
    e = bench.roofline_for(dense, r, bench.models(dense))
    assert e["bound"] == "mfma" and e["unit"] == "TFLOP/s" and e["peak"] == bench.MFMA_BF16_PEAK_TFS
    assert abs(e["frac"] - bench.models(dense)["bwd_flops"] / 0.07e9 / bench.MFMA_BF16_PEAK_TFS) < 1e-3
    dil = WORKLOADS["dilated"]
    r = {"fwd_ms": 0.09, "bwd_ms": 0.3, "plan_fwd": "gather_fwd_kernel(dot)",
         "plan_bwd": "gather_bwd_q_kernel(dot)+gather_bwd_kv_kernel(dot)"}
    e = bench.roofline_for(dil, r, bench.models(dil), {"copy_GBs": 5500.0, "mfma_bf16_TFs": 1800.0})
    assert e["bound"] == "hbm" and e["mfma_bf16_frac"] is None and "mfma_frac_of_measured_loop" not in e
    assert abs(e["frac_of_measured_copy"] - e["achieved"] / 5500.0) < 1e-3


def test_summary_keeps_the_quoted_configs_last():
    names = ["band", "band_bf16grad", "uniform", "decode_dilated", "ultra_band", "dilated", "coord", "ultra"]
    order = bench.summary_order(names)
    assert order[-4:] == ["band", "dilated", "coord", "ultra"] and sorted(order) == sorted(names)
    assert bench.summary_order(["uniform", "band"]) == ["uniform", "band"]


def test_sweep_workloads_span_windows_and_lengths():
    """The scaling sweep: band windows 32 .. 2,048 and W = T on one shape, the
    dilated graph at T = 4,096 .. 65,536 with every power-of-two distance
    below T; edge counts grow within each family."""
    ws = bench.sweep_workloads()
    band = [w for w in ws if w.name.startswith("band")]
    dil = [w for w in ws if w.name.startswith("dilated")]
    assert [w.window for w in band] == [32, 64, 128, 256, 512, 1024, 2048, 16384]
    assert {(w.B, w.H, w.T, w.D) for w in band} == {(1, 8, 16384, 64)}
    assert [w.T for w in dil] == [4096, 8192, 16384, 32768, 65536]
    for w in dil:
        assert w.window == 4 and w.offsets == tuple(2 ** k for k in range(w.T.bit_length() - 1))
        assert max(w.offsets) < w.T
    for fam in (band, dil):
        edges = [bench.edge_counts(w)[0] for w in fam]
        assert edges == sorted(edges) and len(set(edges)) == len(edges)
    # W = T is dense causal attention: T (T + 1) / 2 edges per (b, h)
    assert bench.edge_counts(band[-1])[0] == 16384 * 16385 // 2

"""Host logic of the measurement scripts (no GPU): the decoder-layer sum of
the crossover sweep, and the CPU-oracle leg of bench.py."""

from affine_quantized_gemm_amd import sweep


def test_layer_table_sums_the_seven_projections():
    def row(shape, M, sel, planned=None):
        r = {"shape": shape, "M": M, "selected": "k", "us": {"k": sel, "other": sel * 10}}
        if planned is not None:
            r["split_us"] = {"planned_ws": planned}
        return r

    rows = [row("verify", 8, 5.0), row("kv", 8, 4.0), row("gateup", 8, 11.0), row("down", 8, 18.0, planned=15.0),
            row("verify", 16, 6.0)]  # M = 16 lacks the other shapes: no layer row
    t = sweep.layer_table(rows)
    assert t == [{"M": 8, "layer_us": 2 * 5.0 + 2 * 4.0 + 2 * 11.0 + 18.0,
                  "layer_ws_us": 2 * 5.0 + 2 * 4.0 + 2 * 11.0 + 15.0}]
    # q, k, v, o, gate, up, down: seven calls
    assert sum(n for _, n in sweep.LAYER) == 7


def test_bench_cpu_baseline_entries():
    """bench.py's CPU-oracle leg for the transposed, batched and
    non-transposed entries (tiny shapes, a few hundredths of a second each)."""
    import bench
    for entry in ("small_m", "batched", "nt"):
        r = bench.cpu_baseline("f16", 4, 64, (4,), 128, 256, 0.02, entry)
        assert r["kind"] == "oracle" and r["value"] > 0 and r["cores"] >= 1, (entry, r)
        assert ("stored [K, N]" in r["sample"]) == (entry == "nt")
        assert ("one entry of a batched call" in r["sample"]) == (entry == "batched")

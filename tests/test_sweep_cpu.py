"""Host logic of the crossover sweep: the decoder-layer sum (no GPU)."""

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

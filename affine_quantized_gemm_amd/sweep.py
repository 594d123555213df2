"""Crossover sweep of the small-M kernel variants on the current GPU.

For each weight shape and each M, every variant that can run the problem is
timed through ``qmm_small_m_forced`` on a stack of distinct quantized
matrices larger than the Infinity Cache (so the weights stream from HBM),
cycled call by call, replayed from a captured HIP graph and timed with HIP
events on the replay stream.  The fastest
variant per (shape, M) is what ``qmm_select_kernel`` should return; the
measured table is the source of the crossovers compiled into the dispatch.

    python -m affine_quantized_gemm_amd.sweep [--json out.json] [--shapes verify,kv,...] [--splits] [--layer]
    python -m affine_quantized_gemm_amd.sweep --formats [--json out.json] [--markdown table.md]

``--layer`` adds a synthetic decoder layer at the page's projection shapes
(hidden 4096, intermediate 14336: q and o 4096 -> 4096, k and v 4096 -> 1024,
gate and up 4096 -> 14336, down 14336 -> 4096; random weights, so only the
shape of the step-time curve over M is reproduced, not a model's numbers):
per M, the sum of the seven calls with the variant qmm_small_m selects, and
with qmm_small_m_ws's plan where it takes a split.

The pages' own dispatch story is a crossover curve in M, measured per shape
(MLX issue #4720: the dispatch rules and the split_k rule under "Describe the
bug", the per-M GB/s of forced qmm_nax and the M = 6-8 crossover under
"Expected behavior").
"""

from __future__ import annotations

import argparse
import json
import os
import sys

import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import affine_quantized_gemm_amd as Q  # noqa: E402
import synth  # noqa: E402

SHAPES = {
    # name: (N, K, dtype, bits, group_size)
    "verify": (4096, 4096, "f16", 4, 64),
    "kv": (1024, 4096, "f16", 4, 64),
    "gateup": (14336, 4096, "f16", 4, 64),
    "down": (4096, 14336, "f16", 4, 64),
    "lmhead": (151936, 4096, "bf16", 4, 64),
    "verify8": (4096, 4096, "f16", 8, 64),
    "verify6": (4096, 4096, "bf16", 6, 128),
}
MS = (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 36, 48, 64)


def weight_bytes(N, K, bits, gs):
    return N * K * bits // 8 + 4 * N * (K // gs)


def time_calls(fn, n_calls, reps=5):
    """Best per-call time of fn's launches, replayed from a HIP graph
    captured from them (so the host's launch cost is not timed)."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n_calls
        best = us if best is None else min(best, us)
    return best


# (kernel id, K split) timed with --splits: the tile kernels, and the
# register kernel on K it takes only split (slices it covers whole)
SPLITS = ((3, 2), (3, 4), (4, 2), (4, 4), (4, 8), (1, 2), (1, 4), (1, 7))


def sweep_shape(name, ms, stack_mib, splits=False, shape=None, kernels=None):
    N, K, dt, bits, gs = shape if shape is not None else SHAPES[name]
    tdt = synth.TORCH_DT[dt]
    B = weight_bytes(N, K, bits, gs)
    S = max(2, -(-(stack_mib << 20) // B))
    stack = []
    for i in range(S):
        w = synth.normal((N, K), 0.02, dt, 7000 + i, device="cuda")
        stack.append(Q.quantize(w, bits, gs))
        del w
    rows = []
    for M in ms:
        x = synth.normal((M, K), 1.0, dt, 7500 + M, device="cuda")
        y = torch.empty((M, N), dtype=tdt, device="cuda")
        res = {}
        for kid in (kernels if kernels is not None else Q.KERNEL_IDS):
            if not Q.kernel_supported(tdt, bits, gs, M, N, K, kid):
                continue

            def run(kid=kid):
                for (wq, sc, bi) in stack:
                    Q.small_m(x, wq, sc, bi, bits, gs, out=y, kernel=kid)

            res[Q.kernel_name(kid)] = round(time_calls(run, len(stack)), 3)
        ws_res = {}
        if splits:
            ws = torch.empty((64 * M * N * 4 + 16,), dtype=torch.uint8, device="cuda")
            for kid, sp in SPLITS:
                try:  # one call decides whether this (kernel, split) runs the shape
                    Q.small_m_ws(x, *stack[0], bits, gs, workspace=ws, out=y, kernel=kid, split=sp)
                except Q.QmmError:
                    continue

                def run_s(kid=kid, sp=sp):
                    for (wq, sc, bi) in stack:
                        Q.small_m_ws(x, wq, sc, bi, bits, gs, workspace=ws, out=y, kernel=kid, split=sp)

                ws_res[f"{Q.kernel_name(kid)}/k{sp}"] = round(time_calls(run_s, len(stack)), 3)
            pk, psplit = Q.split_plan(tdt, bits, gs, M, N, K)
            if psplit > 1:
                def run_p():
                    for (wq, sc, bi) in stack:
                        Q.small_m_ws(x, wq, sc, bi, bits, gs, workspace=ws, out=y)
                ws_res["planned_ws"] = round(time_calls(run_p, len(stack)), 3)
            del ws
        best = min(res, key=res.get)
        sel = Q.kernel_name(Q.select_kernel(tdt, bits, gs, M, N, K))
        row = {"shape": name, "N": N, "K": K, "dt": dt, "bits": bits, "gs": gs, "M": M, "us": res,
               "fastest": best, "selected": sel, "selected_gbs": round(B / (res[sel] * 1e-6) / 1e9, 1)}
        if splits:
            row["split_us"] = ws_res
            row["plan"] = list(Q.split_plan(tdt, bits, gs, M, N, K))
        rows.append(row)
        print(f"{name:8s} M={M:3d}  " + "  ".join(f"{k} {v:8.2f}" for k, v in res.items())
              + f"   fastest {best}   selected {sel}"
              + ("   | " + "  ".join(f"{k} {v:.2f}" for k, v in ws_res.items()) if ws_res else ""), flush=True)
    del stack
    torch.cuda.empty_cache()
    return rows


# --formats: every format of the precision matrix at K = 4096, N = 1024 and
# 4096, and the 6/8-bit formats at wide N (gate/up-like 14336 columns) above
# 16 rows, where the choice among the MFMA variants changes.  The VALU
# variant, which the table never selects, is left out.
FORMAT_MS = (1, 4, 6, 8, 16, 24, 36, 64)
WIDE_MS = (24, 36, 64)
MFMA_KERNELS = (1, 2, 3, 4, 5)


def format_shapes():
    out = []
    for dt in ("f16", "bf16"):
        for bits in (4, 6, 8):
            for gs in (32, 64, 128):
                for N in (1024, 4096):
                    out.append((f"{dt}-{bits}b-gs{gs}-N{N}", (N, 4096, dt, bits, gs), FORMAT_MS))
                if bits != 4:
                    out.append((f"{dt}-{bits}b-gs{gs}-N14336", (14336, 4096, dt, bits, gs), WIDE_MS))
    return out


def selection_margin(rows):
    """Per row, how much slower the selected variant is than the fastest
    (1.0 = the fastest)."""
    return [r["us"][r["selected"]] / r["us"][r["fastest"]] for r in rows]


def markdown_table(rows, title, command):
    """The sweep rows as a markdown table (variants in id order)."""
    names = [Q.kernel_name(k) for k in Q.KERNEL_IDS]
    short = {n: n.replace("mfma_splitfree_", "").replace("valu_splitfree", "valu") for n in names}
    used = [n for n in names if any(n in r["us"] for r in rows)]
    lines = [f"# {title}", "", "Command (from the repository root):", "", f"    {command}", "",
             "us per call, best of 5 replays of a HIP graph cycling a >= 576 MiB stack of distinct quantized "
             "matrices (weights stream from HBM); `-` = the variant cannot run the shape.  `selected` is what "
             "qmm_select_kernel returns, `sel/fastest` its time over the fastest variant's.", "",
             "| shape | N x K | M | " + " | ".join(short[n] for n in used) + " | fastest | selected | sel/fastest |",
             "|---|---|---|" + "---|" * len(used) + "---|---|---|"]
    for r in rows:
        cells = " | ".join(f"{r['us'][n]:.2f}" if n in r["us"] else "-" for n in used)
        lines.append(f"| {r['shape']} | {r['N']} x {r['K']} | {r['M']} | {cells} | {short[r['fastest']]} | "
                     f"{short[r['selected']]} | {r['us'][r['selected']] / r['us'][r['fastest']]:.3f} |")
    m = selection_margin(rows)
    lines += ["", f"{len(rows)} rows; the selection is the fastest in {sum(1 for v in m if v == 1.0)}, within 5 % of "
              f"it in {sum(1 for v in m if v <= 1.05)}, worst {max(m):.3f}.", ""]
    return "\n".join(lines)


# (shape, calls per layer): q, o -> verify; k, v -> kv; gate, up -> gateup; down
LAYER = (("verify", 2), ("kv", 2), ("gateup", 2), ("down", 1))


def layer_table(rows):
    """Per-M sums of one decoder layer's seven projection calls, from the
    measured rows (split-free selection, and with the workspace plan)."""
    by = {(r["shape"], r["M"]): r for r in rows}
    out = []
    for M in sorted({r["M"] for r in rows}):
        if not all((name, M) in by for name, _ in LAYER):
            continue
        sel = ws = 0.0
        for name, n in LAYER:
            r = by[(name, M)]
            t = r["us"][r["selected"]]
            sel += n * t
            ws += n * r.get("split_us", {}).get("planned_ws", t)
        out.append({"M": M, "layer_us": round(sel, 2), "layer_ws_us": round(ws, 2)})
    return out


# (shape, batch entries, M) timed with --batched
BATCHED = (("kv", 8, 1), ("kv", 8, 6), ("kv", 8, 32), ("kv", 32, 4), ("verify", 4, 6), ("verify8", 4, 6), ("gateup", 2, 6))


def sweep_batched(stack_mib):
    """qmm_small_m_batched against one qmm_small_m call per entry, over a
    stack of batched weight sets larger than the caches (graph-replayed)."""
    rows = []
    for name, nb, M in BATCHED:
        N, K, dt, bits, gs = SHAPES[name]
        tdt = synth.TORCH_DT[dt]
        Bw = nb * weight_bytes(N, K, bits, gs)
        S = max(2, -(-(stack_mib << 20) // Bw))
        stack = []
        for i in range(S):
            ents = []
            for b in range(nb):
                w = synth.normal((N, K), 0.02, dt, 7000 + nb * i + b, device="cuda")
                ents.append(Q.quantize(w, bits, gs))
                del w
            stack.append(tuple(torch.stack([e[j] for e in ents]) for j in range(3)))
            del ents
        x = synth.normal((nb, M, K), 1.0, dt, 7600 + M, device="cuda")
        y = torch.empty((nb, M, N), dtype=tdt, device="cuda")

        def run_batched():
            for (wq, sc, bi) in stack:
                Q.small_m_batched(x, wq, sc, bi, bits, gs, out=y)

        def run_each():
            for (wq, sc, bi) in stack:
                for b in range(nb):
                    Q.small_m(x[b], wq[b], sc[b], bi[b], bits, gs, out=y[b])

        tb = round(time_calls(run_batched, len(stack)), 3)
        te = round(time_calls(run_each, len(stack)), 3)
        sel = Q.kernel_name(Q.select_kernel(tdt, bits, gs, M, N, K))
        row = {"shape": name, "N": N, "K": K, "dt": dt, "bits": bits, "gs": gs, "batch": nb, "M": M,
               "kernel": sel, "batched_us": tb, "per_entry_calls_us": te,
               "batched_gbs": round(Bw / (tb * 1e-6) / 1e9, 1)}
        rows.append(row)
        print(f"batched {name:8s} B={nb} M={M:3d}  {sel}  one batched call {tb:8.2f} us ({row['batched_gbs']} GB/s)"
              f"   {nb} calls {te:8.2f} us", flush=True)
        del stack
        torch.cuda.empty_cache()
    return rows


# shapes timed with --nt: the same projections with W stored [K, N]
NT_SHAPES = ("verify", "kv", "gateup", "down")
NT_MS = (1, 6, 16, 64)


def sweep_nt(stack_mib, shapes=NT_SHAPES):
    """qmm_small_m_nt (W stored [K, N], quantized along N) next to the
    transposed call on the same shape, over stacks larger than the caches."""
    rows = []
    for name in shapes:
        N, K, dt, bits, gs = SHAPES[name]
        tdt = synth.TORCH_DT[dt]
        B = weight_bytes(N, K, bits, gs)
        S = max(2, -(-(stack_mib << 20) // B))
        stack = []
        for i in range(S):
            w = synth.normal((K, N), 0.02, dt, 7700 + i, device="cuda")
            stack.append(Q.quantize(w, bits, gs))
            del w
        for M in NT_MS:
            x = synth.normal((M, K), 1.0, dt, 7800 + M, device="cuda")
            y = torch.empty((M, N), dtype=tdt, device="cuda")

            def run():
                for (wq, sc, bi) in stack:
                    Q.small_m_nt(x, wq, sc, bi, bits, gs, out=y)

            t = round(time_calls(run, len(stack)), 3)
            need = Q.nt_workspace_bytes(tdt, bits, gs, M, N, K)
            ws = torch.empty((max(need, 16),), dtype=torch.uint8, device="cuda")

            def run_split():
                for (wq, sc, bi) in stack:
                    Q.small_m_nt(x, wq, sc, bi, bits, gs, out=y, split=True, workspace=ws)

            ts = round(time_calls(run_split, len(stack)), 3)
            row = {"shape": name, "N": N, "K": K, "dt": dt, "bits": bits, "gs": gs, "M": M, "nt_us": t,
                   "nt_gbs": round(B / (t * 1e-6) / 1e9, 1), "nt_split_us": ts,
                   "nt_split_gbs": round(B / (ts * 1e-6) / 1e9, 1), "workspace_bytes": need}
            rows.append(row)
            print(f"nt {name:8s} M={M:3d}  {t:8.2f} us  ({row['nt_gbs']} GB/s)   with the K split {ts:8.2f} us "
                  f"({row['nt_split_gbs']} GB/s)", flush=True)
            del ws
        del stack
        torch.cuda.empty_cache()
    return rows


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--shapes", default=",".join(SHAPES))
    p.add_argument("--ms", default=",".join(map(str, MS)))
    p.add_argument("--stack-mib", type=int, default=576)
    p.add_argument("--json", default=None)
    p.add_argument("--splits", action="store_true", help="also time K splits (workspace path)")
    p.add_argument("--layer", action="store_true", help="also sum one decoder layer's projections per M")
    p.add_argument("--batched", action="store_true", help="also time the batched entry point")
    p.add_argument("--nt", action="store_true", help="also time non-transposed weights")
    p.add_argument("--nt-shapes", default=",".join(NT_SHAPES), help="shapes for --nt")
    p.add_argument("--formats", action="store_true",
                   help="sweep every format of the precision matrix (MFMA variants only) instead of --shapes")
    p.add_argument("--markdown", default=None, help="also write the rows as a markdown table to this path")
    a = p.parse_args()
    ms = [int(m) for m in a.ms.split(",")]
    shapes = [s for s in a.shapes.split(",") if s]
    if a.layer:
        shapes += [name for name, _ in LAYER if name not in shapes]
    rows = []
    if a.formats:
        for name, shape, fms in format_shapes():
            rows += sweep_shape(name, fms, a.stack_mib, shape=shape, kernels=MFMA_KERNELS)
        if a.markdown:
            with open(a.markdown, "w") as f:
                f.write(markdown_table(rows, "Kernel crossover sweep over every format (MI355X)",
                                       "python3 -m affine_quantized_gemm_amd.sweep --formats --json "
                                       "gpurun_out/sweep_formats.json --markdown gpurun_out/dispatch_formats.md"))
        if a.json:
            with open(a.json, "w") as f:
                json.dump(rows, f, indent=1)
        m = selection_margin(rows)
        print(f"{len(rows)} rows: selection fastest in {sum(1 for v in m if v == 1.0)}, within 5 % in "
              f"{sum(1 for v in m if v <= 1.05)}, worst {max(m):.3f}", flush=True)
        return
    for name in shapes:
        rows += sweep_shape(name, ms, a.stack_mib, a.splits)
    out = rows
    if a.layer:
        table = layer_table(rows)
        for t in table:
            print(f"layer  M={t['M']:3d}  {t['layer_us']:8.2f} us  (with the workspace plan {t['layer_ws_us']:8.2f} us)",
                  flush=True)
        out = {"rows": rows, "layer": table}
    if a.batched:
        brows = sweep_batched(a.stack_mib)
        out = dict(out) if isinstance(out, dict) else {"rows": rows}
        out["batched"] = brows
    if a.nt:
        nrows = sweep_nt(a.stack_mib, [s for s in a.nt_shapes.split(",") if s])
        out = dict(out) if isinstance(out, dict) else {"rows": rows}
        out["nt"] = nrows
    if a.json:
        with open(a.json, "w") as f:
            json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()

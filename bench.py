"""Benchmark: effective weight GB/s and us/call of the affine-quantized
small-M matmul y[M,N] = x[M,K] . dequant(Wq[N,K])^T on one GPU.

Workload (default ``verify``): the verify shapes M = 4 and M = 6 with
K = N = 4096 (a q/o-projection shape), 4-bit codes, group size 64, fp16
activations ~N(0, 1), weights ~N(0, 0.02).  A stack of distinct quantized
matrices, more than twice the 256 MiB Infinity Cache, is cycled call by call
so the weights stream from HBM.  One step = one call per matrix of the stack
at M = 4, then one per matrix at M = 6 (several passes over a stack of fewer
than 32 matrices, so that every replayed graph holds at least 32 calls),
issued by replaying a HIP graph captured from those calls (one graph per M;
the launches cost more host time than a verify-shape kernel runs, so issuing
them one by one from Python would time the host).  The one-by-one rate is
reported beside it.  Other workloads (``--workload``) are the batched-decode
shapes and the wide LM head.

Metric: effective weight GB/s = (packed weight bytes + 4 bytes of scale and
bias per group) / time per call, GB = 1e9 bytes -- the byte count of the
MLX issue #4720 reproducer ("To Reproduce").  Printed as one JSON line.

The default run also measures every workload of the method's benchmark
set in one ``configs`` sub-record (``--no-configs`` skips it): the tiny
verify case, verify at the stated 32-matrix stack, the batched-decode sweep
(down and gate/up projections, split-free and with the K-split workspace
plan), the precision matrix at M = 6 (bits x group size x dtype at N = 1024
and 4096, and the 1%-outlier variant) and the wide LM head (4- and 8-bit).
Per workload and M: graph-replayed us/call, effective weight GB/s, roofline
fraction, the kernel chosen, the streaming-read ceiling at the same byte
count and a short oracle timing on the host.

Counter post-processing (no GPU): ``bench.py --traffic-from FETCH_DIR
WRITE_DIR`` reads two ``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE``
runs of this script, scales the matmul kernel's counters by what the same
counters read for the copy-kernel dispatch of known size that every run
makes, and writes ``profiles/traffic_<workload>.json``.

Trace post-processing (no GPU): ``bench.py --summarize-trace DIR CMD``
reads a ``rocprofv3 --kernel-trace`` run of ``bench.py --timed-only`` (which
launches nothing but the timed graph replays after its warm-up) and writes
``profiles/<kernel>_<workload>_kernel_stats.md``: the per-dispatch durations
of the timed region's matmul kernels, against the bench line of that run.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
COPY_CAL_BYTES = 64 << 20      # copy-kernel dispatch used to scale byte counters


def weight_bytes(N, K, bits, gs):
    return N * K * bits // 8 + 4 * N * (K // gs)


def alg_bytes(M, N, K, bits, gs):
    """Bytes one call must move: packed weights + scale/bias + x + y."""
    return weight_bytes(N, K, bits, gs) + 2 * M * K + 2 * M * N


WORKLOADS = {
    # name: (dtype, bits, gs, M list, N, K)
    "verify": ("f16", 4, 64, (4, 6), 4096, 4096),
    "kv": ("f16", 4, 64, (4, 6), 1024, 4096),
    "tiny": ("f16", 4, 64, (4,), 512, 512),
    "decode_down": ("f16", 4, 64, (8, 16, 32, 36, 48, 64), 4096, 14336),
    "decode_gateup": ("f16", 4, 64, (8, 16, 32, 36, 48, 64), 14336, 4096),
    "lmhead4": ("bf16", 4, 64, (4, 6), 151936, 4096),
    "lmhead8": ("bf16", 8, 64, (4, 6), 151936, 4096),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="verify", choices=sorted(WORKLOADS))
    p.add_argument("--stack-mib", type=int, default=576, help="total weight bytes of the cycled stack")
    p.add_argument("--kernel", type=int, default=None, help="force a kernel variant")
    p.add_argument("--workspace", action="store_true",
                   help="call qmm_small_m_ws (K split where its plan says so) instead of qmm_small_m "
                        "(with --entry nt: qmm_small_m_nt_ws)")
    p.add_argument("--entry", default="small_m", choices=("small_m", "batched", "nt"),
                   help="small_m: y = x W^T per matrix; batched: qmm_small_m_batched over --batch entries, "
                        "each with its own weights and activations; nt: weights stored [K, N] "
                        "(qmm_small_m_nt)")
    p.add_argument("--batch", type=int, default=8, help="entries per batched call (--entry batched)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-extras", action="store_true",
                   help="skip the graph-replay and streaming-read measurements")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="post-process two rocprofv3 --pmc runs of this script (no GPU)")
    p.add_argument("--no-configs", action="store_true", help="skip the per-config sub-record")
    p.add_argument("--config-steps", type=int, default=5, help="timed graph replays per M in the sub-record")
    p.add_argument("--timed-only", action="store_true",
                   help="launch nothing but the warm-up and timed graph replays (and one copy-kernel "
                        "dispatch for the byte counters): for profiler runs")
    p.add_argument("--summarize-trace", nargs="+", metavar="ARG",
                   help="TRACE_DIR COMMAND [REFERENCE_LOG]: post-process a rocprofv3 --kernel-trace run of "
                        "--timed-only, against the bench line of an unprofiled run of the same workload (no GPU)")
    p.add_argument("--summarize-util", nargs="+", metavar="PMC_DIR",
                   help="post-process rocprofv3 --pmc MfmaUtil VALUBusy runs of --timed-only into "
                        "profiles/mfma_valu_utilization.md (no GPU)")
    return p.parse_args()


# Source files each kernel variant is compiled from (its translation unit and
# the headers it includes): the counter summary of a kernel stays valid while
# these are unchanged.
KERNEL_SOURCES = {
    "valu_splitfree": ["qmm_valu.hip"],
    "mfma_splitfree_reg": ["qmm_mfma_reg.hpp", "qmm_mfma_frag.hpp"],
    "mfma_splitfree_pass": ["qmm_mfma_pass.hip", "qmm_mfma_frag.hpp"],
    "mfma_splitfree_tile16": ["qmm_mfma_tile.hpp", "qmm_mfma_frag.hpp"],
    "mfma_splitfree_tile64": ["qmm_mfma_tile.hpp", "qmm_mfma_frag.hpp"],
    "mfma_splitfree_dqlds": ["qmm_mfma_dqlds.hip", "qmm_mfma_frag.hpp"],
    "nt": ["qmm_nt.hip", "qmm_mfma_frag.hpp"],
}
COMMON_SOURCES = ["qmm_device.hpp", "qmm_internal.hpp"]


def kernel_source_digest(kernel_name):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "affine_quantized_gemm_amd", "csrc")
    for f in sorted(set(KERNEL_SOURCES[kernel_name] + COMMON_SOURCES)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, digest):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- counters

def _is_copy_probe(name):
    return name.startswith("(anonymous namespace)::copy_kernel(")


def _is_matmul_kernel(name):
    return name.startswith("void qmm::") and "quantize_kernel" not in name


def _read_counter_dir(d, counter):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per_kernel, copies = {}, []
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                name, v = row["Kernel_Name"], float(row["Counter_Value"])
                if _is_copy_probe(name):
                    copies.append(v)
                elif _is_matmul_kernel(name):
                    per_kernel.setdefault(name, []).append(v)
    if not copies or not per_kernel:
        raise SystemExit(f"{d}: missing copy or matmul dispatches for {counter}")
    name = max(per_kernel, key=lambda k: len(per_kernel[k]))
    vals = per_kernel[name]
    return name, sum(vals) / len(vals), len(vals), sum(copies) / len(copies)


def _labelled_dispatches(d, counter, line):
    """The matmul-kernel dispatches of a --timed-only run under --pmc, in
    launch order, each labelled with its M from the run's launch sequence
    (per M: S*P eager calls then one capture replay; then warm-up and timed
    replays, M after M).  None if the count does not match that sequence."""
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    rows = {}
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and _is_matmul_kernel(r["Kernel_Name"]):
                    rows[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
    c = line["config"]
    Ms, SP = line["us_per_call"].keys(), c["stack"] * c["passes"]
    Ms = [int(k[1:]) for k in Ms]
    seq = []
    for M in Ms:
        seq += [M] * (2 * SP)
    for _ in range(line["warmup"] + line["steps"]):
        for M in Ms:
            seq += [M] * SP
    ids = sorted(rows)
    if len(ids) != len(seq):
        return None
    return [(M, rows[i][0], rows[i][1]) for M, i in zip(seq, ids)]


def _short_kernel(name):
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void qmm::", "")


def _bench_line(d):
    for fn in glob.glob(os.path.join(d, "*.log")) + glob.glob(os.path.join(d, "*.json")):
        with open(fn) as f:
            for line in f:
                if line.startswith("{") and '"metric"' in line:
                    return json.loads(line)
    raise SystemExit(f"no bench JSON line in {d}")


def traffic_from(fetch_dir, write_dir):
    bf, bw = _bench_line(fetch_dir), _bench_line(write_dir)
    if bf["kernel_source_digest"] != bw["kernel_source_digest"] or bf["config"] != bw["config"]:
        raise SystemExit("the two counter runs used different sources or workloads")
    kf, fetch_kib, nf, copy_fetch_kib = _read_counter_dir(fetch_dir, "FETCH_SIZE")
    kw, write_kib, nw, copy_write_kib = _read_counter_dir(write_dir, "WRITE_SIZE")
    if kf != kw:
        raise SystemExit(f"different dominant kernels: {kf} vs {kw}")
    f_scale = COPY_CAL_BYTES / (copy_fetch_kib * 1024.0)
    w_scale = COPY_CAL_BYTES / (copy_write_kib * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    wl = bf["config"]["workload_name"]
    out = {
        "workload": wl,
        "kernel": kf,
        "kernel_source_digest": bf["kernel_source_digest"],
        "dispatches": {"FETCH_SIZE": nf, "WRITE_SIZE": nw},
        "fetch_kib_per_launch_raw": round(fetch_kib, 1),
        "write_kib_per_launch_raw": round(write_kib, 1),
        "copy_calibration": {"bytes": COPY_CAL_BYTES, "fetch_kib": copy_fetch_kib, "write_kib": copy_write_kib,
                             "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
        "fetch_bytes_per_launch": int(fetch_b),
        "write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(fetch_b + write_b),
        "alg_bytes_per_launch": bf["roofline"]["alg_bytes_per_launch"],
        "traffic_over_alg": round((fetch_b + write_b) / bf["roofline"]["alg_bytes_per_launch"], 4),
    }
    # per M (decode sweeps run several kernels): mean bytes per dispatch
    lf = _labelled_dispatches(fetch_dir, "FETCH_SIZE", bf)
    lw = _labelled_dispatches(write_dir, "WRITE_SIZE", bw)
    if lf and lw:
        c = bf["config"]
        per_m = {}
        for M in sorted({m for m, _, _ in lf}):
            fv = [v for m, _, v in lf if m == M]
            wv = [v for m, _, v in lw if m == M]
            names = sorted({_short_kernel(n) for m, n, _ in lf if m == M})
            hbm = (sum(fv) / len(fv)) * 1024.0 * f_scale + (sum(wv) / len(wv)) * 1024.0 * w_scale
            alg = alg_bytes(M, c["N"], c["K"], c["bits"], c["group_size"])
            per_m[f"M{M}"] = {"kernel": names, "hbm_bytes_per_launch": int(hbm), "alg_bytes_per_launch": alg,
                              "traffic_over_alg": round(hbm / alg, 4)}
        out["per_m"] = per_m
    path = os.path.join(ROOT, "profiles", f"traffic_{wl}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


# ---------------------------------------------------------------- oracle leg

def cpu_baseline(dt, bits, gs, Ms, N, K, budget_s, entry="small_m"):
    """The oracle, untuned, on one matrix of the workload (host cores).  For
    the LM head only a slice of the output columns is computed, scaled to a
    per-call figure (columns are independent)."""
    import numpy as np
    import synth
    from oracle import qmm_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    host_cores = len(os.sched_getaffinity(0))
    Ns = min(N, 16384)
    if entry == "nt":  # weights [K, N] quantized along N: the whole matrix
        Ns = N
        w = synth.to_oracle(synth.normal((K, N), 0.02, dt, 9000))
    else:
        w = synth.to_oracle(synth.normal((Ns, K), 0.02, dt, 9000))
    wq, sc, bi = O.quantize(w, dt, bits, gs)
    xs = {M: synth.to_oracle(synth.normal((M, K), 1.0, dt, 9100 + M)) for M in Ms}
    calls = 0
    t0 = time.perf_counter()
    while True:
        for M in Ms:
            if entry == "nt":
                O.qmm_nt(xs[M], wq, sc, bi, dt, bits, gs, N)
            else:  # (a batched call is this per entry)
                O.qmm(xs[M], wq, sc, bi, dt, bits, gs)
            calls += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    per_call = el / calls * (N / Ns)
    sample = (f"{calls} oracle calls (M in {list(Ms)}) on one {Ns}x{K} matrix" + (" stored [K, N]" if entry == "nt" else "")
              + (" (one entry of a batched call; per-entry figures)" if entry == "batched" else "")
              + (f" ({Ns} of the {N} output columns, time scaled by {N / Ns:.2f})" if Ns < N else "")
              + f", {el:.1f} s; {per_call * 1e6:.0f} us per full call")
    return {"value": round(weight_bytes(N, K, bits, gs) / per_call / 1e9, 4), "unit": "GB/s",
            "cores": int(threads), "kind": "oracle", "sample": sample,
            "us_per_call": round(per_call * 1e6, 1), "host_cores": host_cores, "blas_threads": int(threads)}


# ---------------------------------------------------------------- GPU legs

def capture(torch, fn):
    """Capture fn's launches (on torch's current stream inside the capture)
    into one HIP graph; fn runs once eagerly first on the capture stream."""
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
    return g


def stream_us_per_call(torch, fn, n_calls, reps):
    """fn's launches issued one by one from Python on the current stream
    (host launch cost included)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n_calls)


def c_loop_us_per_call(torch, Q, x, stack, bits, gs, y, passes, reps):
    """The stack's qmm_small_m calls issued back to back from the library's C
    loop, stream-launched (no interpreter between launches): the GPU period
    per call (events) and the host time per launch.  The arguments are
    validated once, before the timed calls."""
    args = Q.small_m_loop_args(x, stack, bits, gs, y)
    sh = torch.cuda.current_stream().cuda_stream
    if Q.qmm_probe_small_m_loop(*args, passes, sh) != Q.QMM_OK:
        raise SystemExit("qmm_probe_small_m_loop failed")
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st = 0
    e0.record()
    t0 = time.perf_counter()
    for _ in range(reps):
        st |= Q.qmm_probe_small_m_loop(*args, passes, sh)
    host = time.perf_counter() - t0
    e1.record()
    torch.cuda.synchronize()
    if st != Q.QMM_OK:
        raise SystemExit("qmm_probe_small_m_loop failed")
    n = reps * passes * len(stack)
    return e0.elapsed_time(e1) * 1e3 / n, host * 1e6 / n


def stream_read_ceiling(torch, Q, B, stack_bytes, reps):
    """A plain coalesced read of B bytes per launch, cycling a pool the size
    of the weight stack, replayed from a HIP graph like the timed step: what
    any kernel streaming B bytes per launch can reach here."""
    B16 = B // 16 * 16
    n = max(1, stack_bytes // B16)
    pool = torch.empty(n * B16, dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    views = [pool[i * B16:(i + 1) * B16] for i in range(n)]
    passes = max(1, -(-32 // n))  # at least 32 launches per replayed graph
    best = None
    for shape, grid in ((0, 1024), (0, 2048), (0, 4096), (1, 256), (1, 512), (1, 1024)):
        def reads(grid=grid, shape=shape):
            for _ in range(passes):
                for v in views:
                    Q.probe_stream_read(v, sink, grid, shape)
        g = capture(torch, reads)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * n * passes)
        if best is None or us < best[0]:
            best = (us, grid, shape)
    del pool
    return {"us_per_call": round(best[0], 3), "gbs": round(B16 / (best[0] * 1e-6) / 1e9, 1), "grid": best[1],
            "shape": best[2]}


def copy_calibration(torch, Q):
    """One copy-kernel dispatch of COPY_CAL_BYTES (its byte counters scale
    the matmul kernel's in counter runs); checked for correctness."""
    src = torch.arange(COPY_CAL_BYTES // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    Q.probe_copy(src, dst)
    torch.cuda.synchronize()
    if not torch.equal(src, dst):
        raise RuntimeError("probe copy mismatch")


# ---------------------------------------------------------------- per-config sub-record

KSHORT = {"valu_splitfree": "valu", "mfma_splitfree_reg": "reg", "mfma_splitfree_pass": "pass",
          "mfma_splitfree_tile16": "tile16", "mfma_splitfree_tile64": "tile64"}


def config_cells():
    """(key, dtype, bits, gs, Ms, N, K, entry, wstd, outlier, stack) of every
    workload in the benchmark set; stack None = >= --stack-mib of distinct
    matrices, an int = that many matrices."""
    cells = [("c1_tiny", "f16", 4, 64, (4,), 512, 512, "small_m", 1.0, 0.0, 1),
             ("c2_verify_stack32", "f16", 4, 64, (4, 6), 4096, 4096, "small_m", 0.02, 0.0, 32)]
    dec = (8, 16, 32, 36, 48, 64)
    for name, N, K in (("down", 4096, 14336), ("gateup", 14336, 4096)):
        cells.append((f"c3_{name}", "f16", 4, 64, dec, N, K, "small_m", 0.02, 0.0, None))
        cells.append((f"c3_{name}_ws", "f16", 4, 64, dec, N, K, "ws", 0.02, 0.0, None))
    for dt in ("f16", "bf16"):
        for bits in (4, 6, 8):
            for gs in (32, 64, 128):
                for N in (1024, 4096):
                    cells.append((f"c4_{dt}_{bits}b_gs{gs}_N{N}", dt, bits, gs, (6,), N, 4096, "small_m", 0.02, 0.0,
                                  None))
                cells.append((f"c4_{dt}_{bits}b_gs{gs}_N1024_outlier", dt, bits, gs, (6,), 1024, 4096, "small_m",
                              0.02, 0.01, None))
    cells.append(("c5_lmhead4", "bf16", 4, 64, (4, 6), 151936, 4096, "small_m", 0.02, 0.0, None))
    cells.append(("c5_lmhead8", "bf16", 8, 64, (4, 6), 151936, 4096, "small_m", 0.02, 0.0, None))
    return cells


def oracle_us_per_call(dt, bits, gs, M, N, K, wstd, rows=512, seed=9300):
    """One untuned oracle call (unpack, fp64 dequant, fp64 matmul) on the
    first min(N, rows) output columns, scaled to all N (columns are
    independent); the quantization is not timed."""
    import synth
    from oracle import qmm_oracle as O
    Ns = min(N, rows)
    w = synth.to_oracle(synth.normal((Ns, K), wstd, dt, seed))
    wq, sc, bi = O.quantize(w, dt, bits, gs)
    x = synth.to_oracle(synth.normal((M, K), 1.0, dt, seed + 1))
    best = None
    for _ in range(2):
        t = time.perf_counter()
        O.qmm(x, wq, sc, bi, dt, bits, gs)
        el = time.perf_counter() - t
        best = el if best is None else min(best, el)
    return best * 1e6 * N / Ns


def measure_cell(torch, Q, synth, cell, steps, warmup, stack_mib, ceilings):
    """Graph-replayed timing of one workload of the benchmark set (the same
    protocol as the headline: distinct quantized matrices cycled call by
    call, at least 32 calls per replayed graph, events around each replay)."""
    key, dt, bits, gs, Ms, N, K, entry, wstd, outlier, stack = cell
    tdt = synth.TORCH_DT[dt]
    dev = torch.device("cuda:0")
    B = weight_bytes(N, K, bits, gs)
    S = stack if stack is not None else max(1, -(-(stack_mib << 20) // B))
    mats = []
    for i in range(S):
        w = synth.normal((N, K), wstd, dt, 20000 + 7 * i, device=dev, outlier_frac=outlier)
        mats.append(Q.quantize(w, bits, gs))
        del w
    P = max(1, -(-32 // S))
    xs = {M: synth.normal((M, K), 1.0, dt, 20500 + M, device=dev) for M in Ms}
    ys = {M: torch.empty((M, N), dtype=tdt, device=dev) for M in Ms}
    wss = {M: torch.empty((max(16, Q.workspace_bytes(tdt, bits, gs, M, N, K)),), dtype=torch.uint8, device=dev)
           for M in Ms} if entry == "ws" else {}

    def calls(M):
        for _ in range(P):
            for (wq, sc, bi) in mats:
                if entry == "ws":
                    Q.small_m_ws(xs[M], wq, sc, bi, bits, gs, workspace=wss[M], out=ys[M])
                else:
                    Q.small_m(xs[M], wq, sc, bi, bits, gs, out=ys[M])

    us, kern, cl = [], [], []
    for M in Ms:
        g = capture(torch, lambda M=M: calls(M))
        # at least `warmup` replays and 30 ms of them: a cell follows a run of
        # cells with microsecond kernels, and a first timed block right after
        # a short warm-up read up to 6 % slow on the long LM-head calls
        t_w = time.perf_counter()
        n_w = 0
        while n_w < warmup or time.perf_counter() - t_w < 0.03:
            g.replay()
            torch.cuda.synchronize()
            n_w += 1
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3 / (steps * S * P))
        del g
        if entry != "ws":  # the same calls stream-launched from the library's C loop
            cl.append(c_loop_us_per_call(torch, Q, xs[M], mats, bits, gs, ys[M], P, steps)[0])
        if entry == "ws":
            k, sp = Q.split_plan(tdt, bits, gs, M, N, K)
            kern.append(KSHORT[Q.kernel_name(k)] + (f"/split{sp}" if sp > 1 else ""))
        else:
            kern.append(KSHORT[Q.kernel_name(Q.select_kernel(tdt, bits, gs, M, N, K))])
    del mats, xs, ys, wss
    if B not in ceilings and stack is None:
        ceilings[B] = stream_read_ceiling(torch, Q, B, S * B, max(2, steps))["us_per_call"]
    ceil = ceilings.get(B)
    rec = {"M": list(Ms), "us": [round(u, 3) for u in us],
           "gbs": [round(B / (u * 1e-6) / 1e9, 1) for u in us],
           "frac": [round(alg_bytes(M, N, K, bits, gs) / (u * 1e-6) / 1e9 / HBM_PEAK_GBS, 4) for M, u in zip(Ms, us)],
           "kernel": kern, "stack": S}
    if cl:
        rec["c_loop_us"] = [round(u, 3) for u in cl]
    if ceil is not None:
        rec["ceil_us"] = ceil
        rec["of_ceil"] = [round(ceil / u, 3) for u in us]
    rec["oracle_us"] = round(oracle_us_per_call(dt, bits, gs, Ms[-1], N, K, wstd), 0)
    return rec


def empty_kernel_period(torch, Q, reps=20):
    """Graph-replayed back-to-back period of a near-empty kernel (one
    workgroup reading 16 bytes): the launch floor under any kernel here."""
    src = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")

    def launches():
        for _ in range(64):
            Q.probe_stream_read(src, sink, 1, 0)
    g = capture(torch, launches)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / (reps * 64), 3)


def run_configs(torch, Q, synth, steps, stack_mib):
    t0 = time.perf_counter()
    ceilings = {}
    out = {}
    for cell in config_cells():
        out[cell[0]] = measure_cell(torch, Q, synth, cell, steps, 2, stack_mib, ceilings)
        torch.cuda.empty_cache()
        print(f"config {cell[0]}: {out[cell[0]]['us']} us", file=sys.stderr, flush=True)
    out["wall_s"] = round(time.perf_counter() - t0, 1)
    return out


# ---------------------------------------------------------------- utilisation summary

def summarize_util(dirs):
    """MfmaUtil and VALUBusy (rocprofv3's derived counters) per workload, M
    and kernel, mean over every dispatch of that M in each run."""
    lines = ["# Matrix-core and vector-ALU utilization (rocprofv3 derived counters)", "",
             "Commands (from the repository root), one run per workload:", "",
             "    cd /tmp && export TMPDIR=/tmp && cd -"]
    rows = []
    for d in dirs:
        line = _bench_line(d)
        wl = line["config"]["workload_name"]
        lines.append(f"    rocprofv3 --pmc MfmaUtil VALUBusy -d {d} -o run --output-format csv -- python3 bench.py "
                     f"--workload {wl} --timed-only --steps {line['steps']} --warmup {line['warmup']}")
        mu = _labelled_dispatches(d, "MfmaUtil", line)
        vb = _labelled_dispatches(d, "VALUBusy", line)
        if not mu or not vb:
            raise SystemExit(f"{d}: dispatches do not match the run's launch sequence")
        for M in sorted({m for m, _, _ in mu}):
            a = [v for m, _, v in mu if m == M]
            b = [v for m, _, v in vb if m == M]
            names = ", ".join(sorted({_short_kernel(n) for m, n, _ in mu if m == M}))
            rows.append(f"| {wl} | {M} | `{names}` | {len(a)} | {sum(a) / len(a):.1f} | {sum(b) / len(b):.1f} |")
    lines += ["", "`MfmaUtil` = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) x 100; `VALUBusy` = "
              "SQ_ACTIVE_INST_VALU / CUs / GRBM_GUI_ACTIVE x 100 (rocprofv3's definitions).  Mean over the "
              "dispatches of each M in the run (eager, capture replay, warm-up and timed calls).", "",
              "| workload | M | kernel | dispatches | MfmaUtil % | VALUBusy % |", "|---|---|---|---|---|---|", *rows, ""]
    path = os.path.join(ROOT, "profiles", "mfma_valu_utilization.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {path}")


# ---------------------------------------------------------------- trace summary

def _line_in(path):
    with open(path) as f:
        for ln in f:
            if ln.startswith("{") and '"metric"' in ln:
                return json.loads(ln)
    raise SystemExit(f"no bench JSON line in {path}")


def summarize_trace(trace_dir, command, reference=None):
    """Per-dispatch durations of the timed region of a --timed-only run
    under rocprofv3 --kernel-trace, against the bench line of that run and,
    if given, of an unprofiled run of the same workload."""
    line = _bench_line(trace_dir)
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if _is_matmul_kernel(name):
                    rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), name))
    rows.sort()
    n_timed = line["timed_dispatches"]
    main_rows = [r for r in rows if "reduce_partials" not in r[2]]
    timed = main_rows[-n_timed:]
    t_lo = timed[0][0]
    red = [r for r in rows if "reduce_partials" in r[2] and r[0] >= t_lo]
    per = {}
    for a, b, name in timed + red:
        per.setdefault(name, []).append((b - a) / 1e3)
    short = _short_kernel
    calls_per_step = n_timed / line["steps"]
    wl, kname = line["config"]["workload_name"], line["roofline"]["kernel"]
    main_name = max((n for n in per if "reduce_partials" not in n), key=lambda n: len(per[n]))
    avg_main = sum(sum(v) for n, v in per.items() if "reduce_partials" not in n) / n_timed
    lines = [f"# rocprofv3 kernel trace, timed region only: {wl} workload", "",
             "Command (from the repository root):", "", "    cd /tmp && export TMPDIR=/tmp && cd -",
             f"    {command}", "",
             f"Dispatches of the timed region: the last {n_timed} matmul-kernel dispatches of the run "
             f"({line['steps']} steps x {calls_per_step:.0f} calls; the run launches nothing else after "
             "its warm-up but one copy kernel). Durations from the trace's start and end stamps.", "",
             "| kernel | dispatches | avg us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -len(kv[1])):
        vs = sorted(v)
        lines.append(f"| `{short(name)}` | {len(v)} | {sum(v) / len(v):.3f} | {vs[len(vs) // 2]:.3f} | "
                     f"{vs[0]:.3f} | {vs[-1]:.3f} |")
    alg = line["roofline"]["alg_bytes_per_launch"]
    lines += ["", "Against the bench line of the same run (events around each graph replay, profiler attached):", "",
              f"- ms_per_step {line['ms_per_step']}; us_per_call {json.dumps(line['us_per_call'])}",
              f"- matmul kernels: {avg_main:.3f} us average x {calls_per_step:.0f} calls per step = "
              f"{avg_main * calls_per_step / 1e3:.4f} ms of the {line['ms_per_step']} ms step",
              f"- roofline from the trace: {alg} algorithmic bytes per launch / {avg_main:.3f} us = "
              f"{alg / (avg_main * 1e-6) / 1e9:.1f} GB/s = frac {alg / (avg_main * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f} "
              f"(the line's event-timed frac: {line['roofline']['frac']})",
              f"- kernel_source_digest {line['kernel_source_digest']}", ""]
    if reference:
        ref = _line_in(reference)
        if ref["config"] != line["config"] or ref["kernel_source_digest"] != line["kernel_source_digest"]:
            raise SystemExit("the reference line is of another workload or other kernel sources")
        ref_frac = ref["roofline"]["frac"]
        tr_frac = alg / (avg_main * 1e-6) / 1e9 / HBM_PEAK_GBS
        lines += ["Against the bench line of an unprofiled run of the same workload and sources "
                  f"(`{reference}`):", "",
                  f"- ms_per_step {ref['ms_per_step']}; us_per_call {json.dumps(ref['us_per_call'])}; "
                  f"launch_us {ref['roofline']['launch_us']}",
                  f"- kernels from the trace x calls per step = {avg_main * calls_per_step / 1e3:.4f} ms "
                  f"against its {ref['ms_per_step']} ms step (ratio "
                  f"{avg_main * calls_per_step / 1e3 / ref['ms_per_step']:.3f}: below 1 the gaps between launches, "
                  "and for a split call its reduction pass; above 1 the tracer's lengthening of each dispatch)",
                  f"- roofline frac from the trace {tr_frac:.4f} against the line's {ref_frac} "
                  f"({(tr_frac / ref_frac - 1) * 100:+.1f} %; the line divides by the whole call, the trace by "
                  "the matmul kernel alone)", ""]
    name = kname if kname == "nt" else KSHORT.get(kname, kname)
    path = os.path.join(ROOT, "profiles", f"{kname}_{wl}_kernel_stats.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {path} ({name}: {avg_main:.3f} us avg over {n_timed} timed dispatches)")


def main():
    args = parse()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_util:
        summarize_util(args.summarize_util)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the per-GPU path would be sharded by output columns with no collective).", file=sys.stderr)
        sys.exit(2)
    import torch
    import affine_quantized_gemm_amd as Q
    import synth

    dt, bits, gs, Ms, N, K = WORKLOADS[args.workload]
    tdt = synth.TORCH_DT[dt]
    NB = args.batch if args.entry == "batched" else 1  # entries per call
    if NB < 1:
        raise SystemExit("--batch must be at least 1")
    B = NB * weight_bytes(N, K, bits, gs)  # weight bytes of one call
    S = max(1, -(-(args.stack_mib << 20) // B))
    if args.workload == "tiny":
        S = 1
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    # ---- synthetic weights, quantized on the GPU; raw weights freed right away
    stack = []
    for i in range(S):
        if args.entry == "batched":  # one weight set per entry
            ents = []
            for b in range(NB):
                w = synth.normal((N, K), 0.02, dt, synth.seed_for(2, 0, NB * i + b), device=dev)
                ents.append(Q.quantize(w, bits, gs))
                del w
            stack.append(tuple(torch.stack([e[j] for e in ents]) for j in range(3)))
            del ents
        else:
            shape = (K, N) if args.entry == "nt" else (N, K)  # nt: W stored [K, N]
            w = synth.normal(shape, 0.02, dt, synth.seed_for(2, 0, i), device=dev)
            stack.append(Q.quantize(w, bits, gs))
            del w
    xshape = (lambda M: (NB, M, K)) if args.entry == "batched" else (lambda M: (M, K))
    yshape = (lambda M: (NB, M, N)) if args.entry == "batched" else (lambda M: (M, N))
    xs = {M: synth.normal(xshape(M), 1.0, dt, synth.seed_for(2, 1, M), device=dev) for M in Ms}
    ys = {M: torch.empty(yshape(M), dtype=tdt, device=dev) for M in Ms}
    torch.cuda.synchronize()

    # passes over the stack per step and M: at least 32 calls per replayed
    # graph, so that a graph launch is not charged to a handful of calls
    P = max(1, -(-32 // S))

    # --workspace: the workspace entry point (K split across workgroups where
    # its plan says so), with the workspace allocated here, outside the timing
    wsb = Q.nt_workspace_bytes if args.entry == "nt" else Q.workspace_bytes
    wss = {M: torch.empty((max(16, wsb(tdt, bits, gs, M, N, K)),), dtype=torch.uint8, device=dev)
           for M in Ms} if args.workspace else {}

    def calls(M):
        x, y = xs[M], ys[M]
        for _ in range(P):
            for (wq, sc, bi) in stack:
                if args.entry == "batched":
                    Q.small_m_batched(x, wq, sc, bi, bits, gs, out=y)
                elif args.entry == "nt":
                    Q.small_m_nt(x, wq, sc, bi, bits, gs, out=y, split=args.workspace,
                                 workspace=wss[M] if args.workspace else None)
                elif args.workspace:
                    Q.small_m_ws(x, wq, sc, bi, bits, gs, workspace=wss[M], out=y)
                else:
                    Q.small_m(x, wq, sc, bi, bits, gs, out=y, kernel=args.kernel)

    # The step's launches are captured once per M into a HIP graph and the
    # graphs are replayed: the calls are launch-bound from Python (a few us
    # of host time each, comparable to one verify-shape kernel).
    graphs = {M: capture(torch, lambda M=M: calls(M)) for M in Ms}
    for _ in range(args.warmup):
        for M in Ms:
            graphs[M].replay()
    torch.cuda.synchronize()

    # ---- timed steps; events around each M block give per-launch durations
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in Ms]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_start.record(stream)
    for s in range(args.steps):
        for j, M in enumerate(Ms):
            ev[s][j][0].record(stream)
            graphs[M].replay()
            ev[s][j][1].record(stream)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e_start.elapsed_time(e_end)
    per_m = {M: sum(ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(args.steps)) * 1e3
             / (args.steps * S * P) for j, M in enumerate(Ms)}
    ncalls = args.steps * S * P * len(Ms)
    gbs = B * ncalls / (ms * 1e-3) / 1e9

    # ---- roofline of the matmul kernel: algorithmic bytes / mean launch duration
    alg = {M: NB * alg_bytes(M, N, K, bits, gs) for M in Ms}
    alg_mean = sum(alg.values()) / len(Ms)
    launch_us = sum(per_m.values()) / len(Ms)
    achieved = alg_mean / (launch_us * 1e-6) / 1e9
    def chosen(M):
        if args.entry == "nt":
            sp = Q.nt_workspace_bytes(tdt, bits, gs, M, N, K) // max(1, 4 * M * N) if args.workspace else 0
            return "nt" + (f" (K split {sp})" if sp > 1 else "")
        if args.workspace:
            k, sp = Q.split_plan(tdt, bits, gs, M, N, K)
            return Q.kernel_name(k) + (f" (K split {sp})" if sp > 1 else "")
        return Q.kernel_name(args.kernel if args.kernel is not None else Q.select_kernel(tdt, bits, gs, M, N, K))

    kid = args.kernel if args.kernel is not None else (
        Q.split_plan(tdt, bits, gs, Ms[-1], N, K)[0] if args.workspace else Q.select_kernel(tdt, bits, gs, Ms[-1], N, K))
    kname = "nt" if args.entry == "nt" else Q.kernel_name(kid)
    digest = kernel_source_digest(kname)
    kernels = {f"M{M}": chosen(M) for M in Ms}

    # matmul-kernel dispatches of the timed region (a batched call that the
    # register kernel does not take is one launch per entry)
    per_call = 1
    if args.entry == "batched" and any(Q.select_kernel(tdt, bits, gs, M, N, K) != Q.KERNEL_MFMA_REG for M in Ms):
        per_call = NB
    timed_dispatches = args.steps * S * P * len(Ms) * per_call

    extras = {}
    if not args.no_extras and not args.timed_only:
        extras["empty_kernel_period_us"] = empty_kernel_period(torch, Q)
        extras["stream_launched_us_per_call"] = {
            f"M{M}": round(stream_us_per_call(torch, lambda M=M: calls(M), S * P, max(2, args.steps // 4)), 3)
            for M in Ms}
        if args.entry == "small_m" and not args.workspace and args.kernel is None:
            loop = {M: c_loop_us_per_call(torch, Q, xs[M], stack, bits, gs, ys[M], P, max(2, args.steps // 4))
                    for M in Ms}
            extras["c_loop_launched_us_per_call"] = {f"M{M}": round(loop[M][0], 3) for M in Ms}
            extras["c_loop_host_us_per_launch"] = {f"M{M}": round(loop[M][1], 3) for M in Ms}
        extras["stream_read_ceiling"] = stream_read_ceiling(torch, Q, B, S * B, max(2, args.steps // 2))
    copy_calibration(torch, Q)

    out = {
        "metric": "effective weight GB/s of the affine-quantized small-M QMM "
                  "((packed weight + scale/bias bytes) / time per call)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: M in {list(Ms)}, K={K}, N={N}, {bits}-bit, group {gs}, {dt}; "
                               + (f"{NB} entries per batched call; " if NB > 1 else "")
                               + (f"weights stored [K, N]; " if args.entry == "nt" else "")
                               + f"{S} distinct {'weight sets' if NB > 1 else 'matrices'} ({S * B / 2**20:.0f} MiB) cycled per call, "
                               f"{P} pass(es) over them per M per step",
                   "workload_name": args.workload,
                   "entry": {"batched": "qmm_small_m_batched",
                             "nt": "qmm_small_m_nt_ws" if args.workspace else "qmm_small_m_nt"}.get(
                       args.entry, "qmm_small_m_ws" if args.workspace else "qmm_small_m"),
                   **({"batch": NB} if args.entry == "batched" else {}),
                   **({"weights": "[K, N], quantized along N"} if args.entry == "nt" else {}),
                   "M": list(Ms), "N": N, "K": K, "bits": bits, "group_size": gs, "stack": S, "passes": P,
                   "kernel": kernels},
        "us_per_call": {f"M{M}": round(per_m[M], 3) for M in Ms},
        "weight_gbs_per_m": {f"M{M}": round(B / (per_m[M] * 1e-6) / 1e9, 1) for M in Ms},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(args.workload, digest) if args.entry == "small_m" else None,
                     "alg_bytes_per_launch": int(alg_mean), "launch_us": round(launch_us, 3),
                     "kernel": kname},
        **extras,
        "kernel_source_digest": digest,
        "library_build_digest": Q.BUILD_DIGEST,
        "timed_dispatches": timed_dispatches,
        "wall_s": round(wall, 3),
    }
    default_run = (args.workload == "verify" and args.entry == "small_m" and args.kernel is None
                   and not args.workspace)
    if default_run and not args.no_configs and not args.timed_only:
        out["configs"] = run_configs(torch, Q, synth, args.config_steps, args.stack_mib)
    if not args.no_cpu_baseline and not args.timed_only:
        out["cpu_baseline"] = cpu_baseline(dt, bits, gs, Ms, N, K, args.cpu_seconds, args.entry)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

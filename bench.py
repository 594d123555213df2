"""Benchmark: effective weight GB/s and us/call of the verify-shape QMM.

Workload (default): the verify shapes M = 4 and M = 6 with K = N = 4096
(a q/o-projection shape), 4-bit codes, group size 64, fp16 activations
~N(0, 1), weights ~N(0, 0.02).  A stack of distinct quantized matrices,
more than twice the 256 MiB Infinity Cache, is cycled call by call so the
weights stream from HBM.  One step = one call per matrix of the stack at
M = 4, then one per matrix at M = 6.

Metric: effective weight GB/s = (packed weight bytes + 4 bytes of scale/bias
per group) / time per call, GB = 1e9 bytes -- the byte count of the MLX
issue #4720 reproducer ("To Reproduce").  Printed as one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
INFINITY_CACHE = 256 << 20


def weight_bytes(N, K, bits, gs):
    return N * K * bits // 8 + 4 * N * (K // gs)


WORKLOADS = {
    # name: (dtype, bits, gs, M list, N, K)
    "verify": ("f16", 4, 64, (4, 6), 4096, 4096),
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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    return p.parse_args()


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "affine_quantized_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, digest):
    """HBM traffic per launch from committed rocprofv3 counter summaries, if
    they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != digest:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(dt, bits, gs, Ms, N, K, budget_s):
    """The oracle, untuned, on one matrix of the workload (host cores)."""
    import numpy as np
    import synth
    from oracle import qmm_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    w = synth.to_oracle(synth.normal((N, K), 0.02, dt, 9000))
    wq, sc, bi = O.quantize(w, dt, bits, gs)
    xs = {M: synth.to_oracle(synth.normal((M, K), 1.0, dt, 9100 + M)) for M in Ms}
    calls = 0
    t0 = time.perf_counter()
    while True:
        for M in Ms:
            O.qmm(xs[M], wq, sc, bi, dt, bits, gs)
            calls += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    per_call = el / calls
    return {"value": weight_bytes(N, K, bits, gs) / per_call / 1e9, "unit": "GB/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"{calls} oracle calls (M in {list(Ms)}) on one {N}x{K} matrix, {el:.1f} s; "
                      f"{per_call * 1e6:.0f} us/call"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              f"(the per-GPU path would be sharded by output columns with no collective).", file=sys.stderr)
        sys.exit(2)
    import torch
    import affine_quantized_gemm_amd as Q
    import synth

    dt, bits, gs, Ms, N, K = WORKLOADS[args.workload]
    tdt = synth.TORCH_DT[dt]
    B = weight_bytes(N, K, bits, gs)
    S = max(1, -(-(args.stack_mib << 20) // B))
    if args.workload == "tiny":
        S = 1
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    # ---- synthetic weights, quantized on the GPU; raw weights freed right away
    stack = []
    for i in range(S):
        w = synth.normal((N, K), 0.02, dt, synth.seed_for(2, 0, i), device=dev)
        stack.append(Q.quantize(w, bits, gs))
        del w
    xs = {M: synth.normal((M, K), 1.0, dt, synth.seed_for(2, 1, M), device=dev) for M in Ms}
    ys = {M: torch.empty((M, N), dtype=tdt, device=dev) for M in Ms}
    torch.cuda.synchronize()

    def step():
        for M in Ms:
            x, y = xs[M], ys[M]
            for (wq, sc, bi) in stack:
                Q.small_m(x, wq, sc, bi, bits, gs, out=y, kernel=args.kernel)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-M timing (us/call), events on the stream the kernels run on
    per_m = {}
    for M in Ms:
        x, y = xs[M], ys[M]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(1, 2 * args.steps)
        e0.record(stream)
        for _ in range(reps):
            for (wq, sc, bi) in stack:
                Q.small_m(x, wq, sc, bi, bits, gs, out=y, kernel=args.kernel)
        e1.record(stream)
        torch.cuda.synchronize()
        per_m[M] = e0.elapsed_time(e1) * 1e3 / (reps * S)

    # ---- timed steps
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1)
    calls = args.steps * S * len(Ms)
    us_call = ms * 1e3 / calls
    gbs = B * calls / (ms * 1e-3) / 1e9

    # roofline of the dominant kernel: algorithmic bytes (weights + x + y) per launch
    alg = {M: B + 2 * M * K + 2 * M * N for M in Ms}
    alg_mean = sum(alg.values()) / len(Ms)
    achieved = sum(alg[M] / (per_m[M] * 1e-6) for M in Ms) / len(Ms) / 1e9
    digest = kernel_source_digest()
    kid = args.kernel if args.kernel is not None else Q.select_kernel(tdt, bits, gs, Ms[-1], N, K)
    out = {
        "metric": "effective weight GB/s of the verify-shape affine-quantized QMM (M=4 and M=6)",
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
                               f"{S} distinct matrices ({S * B / 2**20:.0f} MiB) cycled per call",
                   "M": list(Ms), "N": N, "K": K, "bits": bits, "group_size": gs, "stack": S,
                   "kernel": Q.kernel_name(kid)},
        "us_per_call": {f"M{M}": round(per_m[M], 3) for M in Ms},
        "weight_gbs_per_m": {f"M{M}": round(B / (per_m[M] * 1e-6) / 1e9, 1) for M in Ms},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(args.workload, digest),
                     "alg_bytes_per_launch": int(alg_mean), "kernel": Q.kernel_name(kid)},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(dt, bits, gs, Ms, N, K, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

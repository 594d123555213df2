"""Parity at the full workload sizes, in the launch configuration bench.py
times (kernel chosen by qmm_small_m), on sampled output columns.

Workloads: tiny verify (M=4, 512x512), verify (M=4/6, 4096x4096), batched
decode (M=8..64, down 14336->4096 and gate/up 4096->14336), the precision
matrix at M=6 (bits x group x dtype, N=1024/4096, with an outlier variant) and
the wide LM head (M=4/6, N=151936, bf16, 4- and 8-bit).  Weights are drawn on
the GPU with a seeded generator; the oracle quantizes the sampled rows from a
host copy of the same weights and must agree bit for bit with the GPU
quantizer, then checks the sampled outputs."""

import numpy as np
import pytest
import torch

import synth
from oracle import qmm_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import affine_quantized_gemm_amd as Q
    return Q


def check(Q, dt, bits, gs, Ms, N, K, seed, wstd=0.02, outlier=0.0, ncols=192, kernels=(None,)):
    dev = torch.device("cuda")
    w = synth.normal((N, K), wstd, dt, seed, device=dev, outlier_frac=outlier)
    wq, sc, bi = Q.quantize(w, bits, gs)
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([rng.choice(N, size=min(ncols, N), replace=False),
                                     np.arange(max(0, N - 17), N), np.arange(min(16, N))]))
    idx = torch.from_numpy(cols).to(dev)
    w_rows = synth.to_oracle(w.index_select(0, idx))
    owq, osc, obi = O.quantize(w_rows, dt, bits, gs)
    assert np.array_equal(synth.to_oracle(wq.index_select(0, idx)), owq)
    assert np.array_equal(synth.to_oracle(sc.index_select(0, idx)), osc)
    assert np.array_equal(synth.to_oracle(bi.index_select(0, idx)), obi)
    del w
    for M in Ms:
        x = synth.normal((M, K), 1.0, dt, seed + 1000 + M, device=dev)
        yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
        for kernel in kernels:
            if kernel is not None and not Q.kernel_supported(synth.TORCH_DT[dt], bits, gs, M, N, K, kernel):
                continue
            print(f"config {dt} b{bits} gs{gs} M={M} N={N} K={K} kernel={kernel}", flush=True)
            y = Q.small_m(x, wq, sc, bi, bits, gs, kernel=kernel)
            yg = O.to_f64(synth.to_oracle(y.index_select(1, idx)), dt)
            ok, worst = O.within_tolerance(yg, yo, T)
            assert ok, (M, kernel, worst)
            assert torch.isfinite(y.float()).all()


def test_tiny_verify_full_output(Q):
    """Tiny verify case, every output checked: M=4, K=N=512, W ~ N(0,1), seed 0."""
    dt, bits, gs, M, N, K = "f16", 4, 64, 4, 512, 512
    w = synth.normal((N, K), 1.0, dt, 0)
    x = synth.normal((M, K), 1.0, dt, 1)
    wq, sc, bi = Q.quantize(w.cuda(), bits, gs)
    owq, osc, obi = O.quantize(synth.to_oracle(w), dt, bits, gs)
    assert np.array_equal(synth.to_oracle(wq), owq)
    yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
    for kernel in (None, 0, 1, 2):
        if kernel is not None and not Q.kernel_supported(torch.float16, bits, gs, M, N, K, kernel):
            continue
        y = Q.small_m(x.cuda(), wq, sc, bi, bits, gs, kernel=kernel)
        ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
        assert ok, (kernel, worst)


def test_verify_shapes(Q):
    check(Q, "f16", 4, 64, (4, 6), 4096, 4096, seed=2000, kernels=(None, 0, 1, 2))


@pytest.mark.parametrize("N,K", [(4096, 14336), (14336, 4096)])
def test_batched_decode(Q, N, K):
    check(Q, "f16", 4, 64, (8, 16, 32, 36, 48, 64), N, K, seed=3000 + N)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [4, 6, 8])
@pytest.mark.parametrize("gs", [32, 64, 128])
def test_precision_matrix(Q, dt, bits, gs):
    for N in (1024, 4096):
        check(Q, dt, bits, gs, (6,), N, 4096, seed=4000 + bits * 10 + gs + N, ncols=96)
    check(Q, dt, bits, gs, (6,), 1024, 4096, seed=4500 + bits * 10 + gs, outlier=0.01, ncols=96)


@pytest.mark.parametrize("bits", [4, 8])
def test_lm_head(Q, bits):
    check(Q, "bf16", bits, 64, (4, 6), 151936, 4096, seed=5000 + bits, ncols=256)

"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

quantize / dequantize must match bit for bit; the matmul must satisfy
|y - y_oracle| <= 4e-3 * sum_k |x_k| |w_hat_k| + 1e-3 elementwise.
Every call goes through the C ABI (via the thin binding)."""

import numpy as np
import pytest
import torch

import synth
from oracle import qmm_oracle as O

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}
COMBOS = [(dt, bits, gs) for dt in ("f16", "bf16") for bits in (4, 6, 8) for gs in (32, 64, 128)]


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import affine_quantized_gemm_amd as Q
    return Q


def weight_sets(dt, N, K, gs, seed):
    return {
        "normal": synth.normal((N, K), 0.02, dt, seed),
        "outlier": synth.normal((N, K), 0.02, dt, seed + 1, outlier_frac=0.01),
        "mixed": synth.special_groups("mixed", N, K, gs, dt, seed + 2),
        "tiny": synth.special_groups("tiny", N, K, gs, dt, seed + 3),
        "constant": synth.special_groups("constant", N, K, gs, dt, seed + 4),
    }


def oracle_quant(w_cpu, dt, bits, gs):
    return O.quantize(synth.to_oracle(w_cpu), dt, bits, gs)


@pytest.mark.parametrize("dt,bits,gs", COMBOS)
def test_quantize_dequantize_bit_exact(Q, dt, bits, gs):
    N, K = 40, 512
    for kind, w in weight_sets(dt, N, K, gs, 100 + bits + gs).items():
        print(f"quantize {dt} bits={bits} gs={gs} kind={kind}", flush=True)
        wq, sc, bi = Q.quantize(w.cuda(), bits, gs)
        torch.cuda.synchronize()
        owq, osc, obi = oracle_quant(w, dt, bits, gs)
        assert np.array_equal(synth.to_oracle(wq), owq), kind
        assert np.array_equal(synth.to_oracle(sc).view(np.uint16), osc.view(np.uint16)), kind
        assert np.array_equal(synth.to_oracle(bi).view(np.uint16), obi.view(np.uint16)), kind
        # dequantize from the oracle's own packed weights
        d = Q.dequantize(synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(),
                         synth.from_oracle(obi, dt).cuda(), bits, gs)
        torch.cuda.synchronize()
        od = O.dequantize(owq, osc, obi, dt, bits, gs, K)
        assert np.array_equal(synth.to_oracle(d).view(np.uint16), od.view(np.uint16)), kind


def run_case(Q, dt, bits, gs, M, N, K, seed, kernel=None, outlier=0.0, wstd=0.02):
    w = synth.normal((N, K), wstd, dt, seed, outlier_frac=outlier)
    x = synth.normal((M, K), 1.0, dt, seed + 1)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    y = Q.small_m(x.cuda(), synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(),
                  synth.from_oracle(obi, dt).cuda(), bits, gs, kernel=kernel)
    torch.cuda.synchronize()
    yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
    yg = O.to_f64(synth.to_oracle(y), dt)
    return O.within_tolerance(yg, yo, T)


def supported(Q, kernel, M, bits=4, gs=64, N=64, K=512, dt=torch.float16):
    return kernel is None or Q.kernel_supported(dt, bits, gs, M, N, K, kernel)


KERNELS = [None, 0, 1, 2, 3, 4, 5]


@pytest.mark.parametrize("dt,bits,gs", COMBOS)
@pytest.mark.parametrize("M", [1, 4, 6, 8])
def test_small_m_formats(Q, dt, bits, gs, M):
    N, K = 80, 512
    for kernel in KERNELS:
        if not supported(Q, kernel, M, bits, gs, N, K, DT[dt]):
            continue
        print(f"small_m {dt} b{bits} gs{gs} M={M} kernel={kernel}", flush=True)
        ok, worst = run_case(Q, dt, bits, gs, M, N, K, seed=7 * M + bits, kernel=kernel)
        assert ok, (kernel, worst)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("M", [2, 3, 5, 7, 12, 16, 24, 32, 36, 48, 64])
def test_small_m_all_m(Q, dt, M):
    N, K = 144, 1024
    for kernel in KERNELS:
        if not supported(Q, kernel, M, 4, 64, N, K, DT[dt]):
            continue
        print(f"small_m {dt} M={M} kernel={kernel}", flush=True)
        ok, worst = run_case(Q, dt, 4, 64, M, N, K, seed=300 + M, kernel=kernel, outlier=0.01)
        assert ok, (kernel, worst)


@pytest.mark.parametrize("dt,bits,gs", COMBOS)
def test_dequant_to_lds_kernel(Q, dt, bits, gs):
    """The weights-dequantized-into-LDS variant (forced): every format, 1..4
    row blocks with ragged M, two K chunks (the prefetch past the end reads
    the last chunk again), against the oracle."""
    N, K = 192, 512
    for M in (1, 6, 17, 40, 64):
        assert Q.kernel_supported(DT[dt], bits, gs, M, N, K, Q.KERNEL_MFMA_DQLDS)
        print(f"dqlds {dt} b{bits} gs{gs} M={M} N={N} K={K}", flush=True)
        ok, worst = run_case(Q, dt, bits, gs, M, N, K, seed=11 * M + bits + gs, kernel=Q.KERNEL_MFMA_DQLDS,
                             outlier=0.01)
        assert ok, (M, worst)


def test_dequant_to_lds_kernel_large(Q):
    """The same variant at the verify shape's width and depth (64 column
    tiles, 16 chunks of K) and at 4 row blocks."""
    for dt, bits, gs, M in (("f16", 4, 64, 16), ("bf16", 8, 32, 64)):
        print(f"dqlds {dt} b{bits} gs{gs} M={M} N=4096 K=4096", flush=True)
        ok, worst = run_case(Q, dt, bits, gs, M, 4096, 4096, seed=77 + M, kernel=Q.KERNEL_MFMA_DQLDS)
        assert ok, (dt, bits, worst)
    assert not Q.kernel_supported(torch.float16, 4, 64, 6, 4096 + 16, 4096, Q.KERNEL_MFMA_DQLDS)  # N % 64
    assert not Q.kernel_supported(torch.float16, 8, 64, 6, 4096, 4096 + 128, Q.KERNEL_MFMA_DQLDS)  # K % 256
    assert Q.kernel_supported(torch.float16, 6, 64, 6, 4096, 4096 + 256, Q.KERNEL_MFMA_DQLDS)


def kernel_built(Q, kernel, M=6, K=512):
    return Q.kernel_supported(torch.float16, 4, 64, M, 64, K, kernel)


@pytest.mark.parametrize("M,N,K,gs", [(1, 1, 64, 64), (3, 17, 128, 32), (8, 1000, 128, 128), (64, 33, 192, 64),
                                      (16, 15, 64, 32), (6, 4099, 256, 128)])
def test_edge_shapes(Q, M, N, K, gs):
    for dt in ("f16", "bf16"):
        for bits in (4, 6, 8):
            for kernel in KERNELS:
                if not supported(Q, kernel, M, bits, gs, N, K, DT[dt]):
                    continue
                print(f"edge {dt} b{bits} M={M} N={N} K={K} gs={gs} kernel={kernel}", flush=True)
                ok, worst = run_case(Q, dt, bits, gs, M, N, K, seed=M + N + K, kernel=kernel)
                assert ok, (dt, bits, kernel, worst)


def test_empty_problems(Q):
    x = torch.zeros((0, 256), dtype=torch.float16, device="cuda")
    w = synth.normal((16, 256), 0.02, "f16", 1).cuda()
    wq, sc, bi = Q.quantize(w, 4, 64)
    y = Q.small_m(x, wq, sc, bi, 4, 64)
    assert y.shape == (0, 16)
    w0 = torch.zeros((0, 256), dtype=torch.float16, device="cuda")
    wq0, sc0, bi0 = Q.quantize(w0, 4, 64)
    y0 = Q.small_m(torch.ones((4, 256), dtype=torch.float16, device="cuda"), wq0, sc0, bi0, 4, 64)
    assert y0.shape == (4, 0)


def test_one_hot_rows_equal_dequantized_weights_valu(Q):
    """With one-hot x the group-factored VALU kernel forms fl32(s*q + b) and
    rounds it once, which is exactly the dequantize output."""
    for dt, bits, gs in (("f16", 4, 64), ("bf16", 8, 32), ("f16", 6, 128)):
        K, N = 256, 48
        w = synth.normal((N, K), 0.02, dt, 5).cuda()
        wq, sc, bi = Q.quantize(w, bits, gs)
        d = Q.dequantize(wq, sc, bi, bits, gs)
        for k0 in range(0, K, 8):
            x = torch.zeros((8, K), dtype=DT[dt], device="cuda")
            x[torch.arange(8), torch.arange(k0, k0 + 8)] = 1
            y = Q.small_m(x, wq, sc, bi, bits, gs, kernel=Q.KERNEL_VALU)
            assert torch.equal(y.view(torch.int16), d[:, k0:k0 + 8].t().contiguous().view(torch.int16))


def test_padded_zero_rows_are_inert(Q):
    """Zero rows appended to x give zero outputs and leave the other rows
    bit-for-bit unchanged (rows are independent in every variant)."""
    for kernel in KERNELS[1:]:
        if not kernel_built(Q, kernel):
            continue
        K, N = 512, 64
        w = synth.normal((N, K), 0.02, "f16", 9).cuda()
        wq, sc, bi = Q.quantize(w, 4, 64)
        x = synth.normal((5, K), 1.0, "f16", 10).cuda()
        xp = torch.cat([x, torch.zeros((3, K), dtype=x.dtype, device="cuda")])
        y = Q.small_m(x, wq, sc, bi, 4, 64, kernel=kernel)
        yp = Q.small_m(xp, wq, sc, bi, 4, 64, kernel=kernel)
        assert torch.all(yp[5:] == 0)
        assert torch.equal(yp[:5].view(torch.int16), y.view(torch.int16)), kernel


def test_deterministic(Q):
    for kernel in KERNELS:
        if kernel is not None and not kernel_built(Q, kernel):
            continue
        K, N, M = 4096, 4096, 6
        if kernel is not None and not kernel_built(Q, kernel, M, K):
            continue
        w = synth.normal((N, K), 0.02, "f16", 11).cuda()
        wq, sc, bi = Q.quantize(w, 4, 64)
        x = synth.normal((M, K), 1.0, "f16", 12).cuda()
        y0 = Q.small_m(x, wq, sc, bi, 4, 64, kernel=kernel)
        for _ in range(20):
            y = Q.small_m(x, wq, sc, bi, 4, 64, kernel=kernel)
            assert torch.equal(y.view(torch.int16), y0.view(torch.int16))


def test_errors_raise(Q):
    w = synth.normal((16, 256), 0.02, "f16", 1).cuda()
    wq, sc, bi = Q.quantize(w, 4, 64)
    x = torch.ones((4, 264), dtype=torch.float16, device="cuda")[:, 8:]
    with pytest.raises(ValueError):
        Q.small_m(x, wq, sc, bi, 4, 64)            # non-contiguous view
    xm = torch.ones((4 * 256 + 4,), dtype=torch.float16, device="cuda")[4:].view(4, 256)
    with pytest.raises(Q.QmmError) as e:
        Q.small_m(xm, wq, sc, bi, 4, 64)            # 8-byte offset: misaligned
    assert e.value.status == Q.QMM_ERR_MISALIGNED
    with pytest.raises(Q.QmmError) as e:
        Q.small_m(torch.ones((65, 256), dtype=torch.float16, device="cuda"), wq, sc, bi, 4, 64)
    assert e.value.status == Q.QMM_ERR_UNSUPPORTED


@pytest.mark.parametrize("K", [2112, 4160, 8256])
@pytest.mark.parametrize("dt,bits,gs", [("f16", 4, 64), ("bf16", 4, 32), ("f16", 6, 128), ("bf16", 8, 64),
                                        ("f16", 8, 32), ("bf16", 6, 64)])
def test_pass_kernel_multipass(Q, K, dt, bits, gs):
    """K walked in several passes with a partial last pass (and, at 4 bits,
    a k-block cut by K); M across 16-row blocks; ragged N.  (Group 128: K
    rounded up to a whole number of groups, 2176 / 4224 / 8320.)"""
    K += (-K) % gs
    for M, N in ((1, 17), (16, 300), (17, 33), (40, 129)):
        print(f"pass {dt} b{bits} gs{gs} M={M} N={N} K={K}", flush=True)
        ok, worst = run_case(Q, dt, bits, gs, M, N, K, seed=K + M + bits, kernel=Q.KERNEL_MFMA_PASS)
        assert ok, (M, N, worst)


@pytest.mark.parametrize("dt,bits,gs", COMBOS)
def test_multi_tile_ragged(Q, dt, bits, gs):
    """More column tiles than resident workgroups (258 tiles of 16 over 256
    workgroups) with a ragged last tile: the persistent multi-tile kernel,
    its prefetch past a workgroup's last tile, and (vector form) the
    cooperative scale/bias blocks, for every format."""
    M, N, K = 6, 16 * 257 + 5, 4096
    print(f"multi {dt} b{bits} gs{gs} M={M} N={N} K={K}", flush=True)
    ok, worst = run_case(Q, dt, bits, gs, M, N, K, seed=bits * 100 + gs, kernel=Q.KERNEL_MFMA_REG, outlier=0.01)
    assert ok, worst
    ok, worst = run_case(Q, dt, bits, gs, 16, N, K, seed=bits * 100 + gs + 1, kernel=Q.KERNEL_MFMA_REG)
    assert ok, worst


@pytest.mark.parametrize("dt,bits,gs,K", [("f16", 4, 64, 4096), ("bf16", 4, 32, 2048), ("bf16", 4, 128, 4096),
                                          ("f16", 8, 64, 4096), ("bf16", 8, 128, 4096), ("bf16", 8, 32, 4096)])
def test_multi_tile_ring(Q, dt, bits, gs, K):
    """Multi-tile kernel over 4-5 tiles per workgroup (1027 tiles of 16,
    ragged last one), every output checked at M = 1, 4, 6, 8, 16: the weight
    and scale/bias ring wraps around more than once per workgroup (4-bit;
    8-bit at M <= 8 where its ring fits in LDS, the register form above)."""
    N = 16 * 1027 + 5
    w = synth.normal((N, K), 0.02, dt, 7000 + gs + bits)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    for M in (1, 4, 6, 8, 16):
        print(f"ring {dt} b{bits} gs{gs} M={M} N={N} K={K}", flush=True)
        x = synth.normal((M, K), 1.0, dt, 7100 + M)
        y = Q.small_m(x.cuda(), wq, sc, bi, bits, gs, kernel=Q.KERNEL_MFMA_REG)
        torch.cuda.synchronize()
        yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
        ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
        assert ok, (M, worst)


@pytest.mark.parametrize("kernel", [3, 4])
@pytest.mark.parametrize("dt,bits,gs", [("f16", 4, 64), ("bf16", 4, 32), ("f16", 4, 128), ("bf16", 6, 64),
                                        ("f16", 6, 32), ("bf16", 8, 128), ("f16", 8, 64)])
def test_tile_kernels(Q, kernel, dt, bits, gs):
    """The shared-activation tile kernels: more column tiles than resident
    workgroups (persistent walk over tiles, weight prefetch across a tile
    boundary), a last pass with fewer k-blocks than k-groups, M across one to
    four 16-row blocks with ragged ends, and a ragged last column tile."""
    bn = {Q.KERNEL_MFMA_TILE16: 16, Q.KERNEL_MFMA_TILE64: 64}[kernel]
    N = bn * 257 + 5
    kblk = 128 if bits == 4 else 64
    K = 16 * kblk + max(kblk, gs)   # passes of 4 (or 2) k-blocks and a short last pass
    seed = kernel * 1000 + bits * 10 + gs
    w = synth.normal((N, K), 0.02, dt, seed, outlier_frac=0.01)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    wq, sc, bi = (synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(),
                  synth.from_oracle(obi, dt).cuda())
    for M in (1, 17, 40, 64):
        print(f"tile kernel={kernel} {dt} b{bits} gs{gs} M={M} N={N} K={K}", flush=True)
        x = synth.normal((M, K), 1.0, dt, seed + M)
        y = Q.small_m(x.cuda(), wq, sc, bi, bits, gs, kernel=kernel)
        torch.cuda.synchronize()
        yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
        ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
        assert ok, (M, worst)


@pytest.mark.parametrize("kernel", [3, 4])
@pytest.mark.parametrize("dt,bits,gs", [("f16", 4, 64), ("bf16", 4, 32), ("bf16", 6, 128), ("f16", 8, 64)])
def test_split_k(Q, kernel, dt, bits, gs):
    """K split across workgroups (workspace path): splits that divide the
    passes evenly and unevenly (the last split shorter), a split larger than
    the passes (reduced), a short last pass, M across row blocks, ragged N;
    deterministic across repeats."""
    kblk = 128 if bits == 4 else 64
    kw = {Q.KERNEL_MFMA_TILE16: 4, Q.KERNEL_MFMA_TILE64: 2}[kernel]
    K = (9 * kw) * kblk + max(kblk, gs)      # 9 full passes + a short one
    N = 64 * 5 + 7
    seed = 5000 + kernel * 100 + bits * 10 + gs
    w = synth.normal((N, K), 0.02, dt, seed, outlier_frac=0.01)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    wq, sc, bi = (synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(),
                  synth.from_oracle(obi, dt).cuda())
    for M in (1, 17, 64):
        x = synth.normal((M, K), 1.0, dt, seed + M)
        yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
        xc = x.cuda()
        for split in (2, 3, 4, 64):
            print(f"split kernel={kernel} {dt} b{bits} gs{gs} M={M} N={N} K={K} split={split}", flush=True)
            ws = torch.empty((split * M * N * 4 + 16,), dtype=torch.uint8, device="cuda")
            y = Q.small_m_ws(xc, wq, sc, bi, bits, gs, workspace=ws, kernel=kernel, split=split)
            torch.cuda.synchronize()
            ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
            assert ok, (M, split, worst)
            y2 = Q.small_m_ws(xc, wq, sc, bi, bits, gs, workspace=ws, kernel=kernel, split=split)
            assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), (M, split)


@pytest.mark.parametrize("dt,gs,K", [("f16", 64, 4096), ("bf16", 32, 2048), ("bf16", 128, 4096)])
def test_reg_row_blocks(Q, dt, gs, K):
    """The register kernel above 16 rows: one 16-row block per workgroup
    layer (the last one partial), every column tile of the slot, over a
    ragged N (1027 tiles of 16); every output checked."""
    N = 16 * 1027 + 5
    w = synth.normal((N, K), 0.02, dt, 8500 + gs)
    owq, osc, obi = oracle_quant(w, dt, 4, gs)
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    for M in (17, 24, 32, 40, 48, 64):
        print(f"reg rows {dt} gs{gs} M={M} N={N} K={K}", flush=True)
        x = synth.normal((M, K), 1.0, dt, 8600 + M)
        y = Q.small_m(x.cuda(), wq, sc, bi, 4, gs, kernel=Q.KERNEL_MFMA_REG)
        torch.cuda.synchronize()
        yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, 4, gs)
        ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
        assert ok, (M, worst)


@pytest.mark.parametrize("dt,bits,gs,K,N", [("f16", 4, 64, 4096, 1024), ("bf16", 8, 64, 4096, 16 * 255 + 7),
                                            ("f16", 6, 128, 4096, 4096), ("bf16", 6, 32, 2048, 1000),
                                            ("f16", 8, 32, 4096, 515), ("bf16", 4, 64, 2048, 9)])
def test_reg_row_blocks_single_tile(Q, dt, bits, gs, K, N):
    """The register kernel above 16 rows where 16 rows take one tile per
    workgroup: a grid of tiles x 16-row blocks (the last block partial),
    ragged and narrow N; every output checked, and each row block
    bit-identical to the same rows computed alone."""
    w = synth.normal((N, K), 0.02, dt, 8700 + bits * 10 + gs)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    for M in (17, 24, 33, 48, 64):
        print(f"reg rows single-tile {dt} {bits}-bit gs{gs} M={M} N={N} K={K}", flush=True)
        x = synth.normal((M, K), 1.0, dt, 8800 + M)
        xc = x.cuda()
        y = Q.small_m(xc, wq, sc, bi, bits, gs, kernel=Q.KERNEL_MFMA_REG)
        torch.cuda.synchronize()
        yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
        ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
        assert ok, (M, worst)
        for r0 in range(0, M, 16):
            yb = Q.small_m(xc[r0:r0 + 16].contiguous(), wq, sc, bi, bits, gs, kernel=Q.KERNEL_MFMA_REG)
            assert torch.equal(y[r0:r0 + 16].view(torch.int16), yb.view(torch.int16)), (M, r0)


@pytest.mark.parametrize("dt,bits,gs,B,M,N,K", [
    ("f16", 4, 64, 4, 6, 1024, 4096),          # register kernel, one tile per workgroup, one launch
    ("bf16", 4, 64, 3, 24, 1000, 2048),        # ... on 16-row blocks, ragged N
    ("bf16", 4, 64, 2, 8, 16 * 300 + 5, 4096),  # LDS ring, entries sharing the resident workgroups
    ("f16", 8, 64, 3, 12, 16 * 270, 4096),     # 8-bit register prefetch, several tiles per workgroup
    ("f16", 4, 64, 3, 36, 16 * 300, 4096),     # LDS ring on row blocks
    ("f16", 4, 64, 3, 8, 256, 14336),          # pass kernel: a launch per entry
    ("bf16", 6, 128, 2, 40, 8192, 4096),       # 64-column tile kernel: a launch per entry
    ("f16", 4, 64, 100, 4, 40, 4096),          # many small entries: LDS ring over 3 ragged tiles each
    ("bf16", 8, 64, 6, 6, 1024, 4096),         # 8-bit, entries' tiles beyond the resident workgroups
    ("f16", 4, 64, 300, 4, 8, 2048),           # entries narrower than a tile: one tile each
])
def test_batched(Q, dt, bits, gs, B, M, N, K):
    """qmm_small_m_batched: every entry against the oracle's batched product
    and bit-identical to qmm_small_m on that entry alone."""
    print(f"batched {dt} {bits}-bit gs{gs} B={B} M={M} N={N} K={K} "
          f"kernel={Q.kernel_name(Q.select_kernel(DT[dt], bits, gs, M, N, K))}", flush=True)
    xs, qs = [], []
    for b in range(B):
        w = synth.normal((N, K), 0.02, dt, 9000 + 10 * b + bits)
        qs.append(oracle_quant(w, dt, bits, gs))
        xs.append(synth.to_oracle(synth.normal((M, K), 1.0, dt, 9100 + 10 * b + M)))
    owq, osc, obi = (np.stack([q[i] for q in qs]) for i in range(3))
    ox = np.stack(xs)
    x = synth.from_oracle(ox, dt).cuda()
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    y = Q.small_m_batched(x, wq, sc, bi, bits, gs)
    torch.cuda.synchronize()
    assert y.shape == (B, M, N)
    yo, T = O.qmm_batched(ox, owq, osc, obi, dt, bits, gs)
    ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
    assert ok, worst
    for b in range(B):
        yb = Q.small_m(x[b], wq[b], sc[b], bi[b], bits, gs)
        assert torch.equal(y[b].view(torch.int16), yb.view(torch.int16)), b


@pytest.mark.parametrize("dt,bits,gs,K", [("f16", 4, 64, 512), ("bf16", 4, 32, 2048), ("f16", 4, 128, 4096),
                                          ("bf16", 8, 64, 1024), ("f16", 8, 128, 4096), ("bf16", 8, 32, 512)])
def test_whole_line_weight_loads(Q, dt, bits, gs, K):
    """The register kernel's whole-line instantiation (4/8-bit, one block of
    at most 8 rows) and the fragment-load one just above it (9, 12 rows), on
    narrow N (rows clamped to N - 1), one exact tile, a ragged last tile and
    several tiles; every output against the oracle, and a batched call
    bit-identical to the standalone one."""
    for N in (5, 16, 37, 1027):
        w = synth.normal((N, K), 0.02, dt, 19000 + N + bits + gs)
        owq, osc, obi = oracle_quant(w, dt, bits, gs)
        wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
        for M in (1, 5, 8, 9, 12):
            print(f"whole-line {dt} b{bits} gs{gs} M={M} N={N} K={K}", flush=True)
            x = synth.normal((M, K), 1.0, dt, 19100 + M)
            y = Q.small_m(x.cuda(), wq, sc, bi, bits, gs)
            torch.cuda.synchronize()
            yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
            ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
            assert ok, (N, M, worst)
    B, M, N = 3, 6, 40  # (a ragged last tile; entry sizes multiples of 16 bytes, as batching requires)
    xs = synth.normal((B, M, K), 1.0, dt, 19200).cuda()
    ents = [Q.quantize(synth.normal((N, K), 0.02, dt, 19300 + b).cuda(), bits, gs) for b in range(B)]
    wq, sc, bi = (torch.stack([e[i] for e in ents]) for i in range(3))
    yb = Q.small_m_batched(xs, wq, sc, bi, bits, gs)
    for b in range(B):
        y1 = Q.small_m(xs[b], wq[b], sc[b], bi[b], bits, gs)
        torch.cuda.synchronize()
        assert torch.equal(yb[b].view(torch.int16), y1.view(torch.int16)), b


def nt_case(Q, dt, bits, gs, M, N, K, seed, outlier=0.0):
    """qmm_small_m_nt on W [K, N] quantized along N, against the oracle."""
    w = synth.normal((K, N), 0.02, dt, seed, outlier_frac=outlier)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    x = synth.normal((M, K), 1.0, dt, seed + 1)
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    y = Q.small_m_nt(x.cuda(), wq, sc, bi, bits, gs)
    torch.cuda.synchronize()
    assert y.shape == (M, N)
    yo, T = O.qmm_nt(synth.to_oracle(x), owq, osc, obi, dt, bits, gs, N)
    return O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T), (x.cuda(), wq, sc, bi, y)


@pytest.mark.parametrize("dt,bits,gs", COMBOS)
def test_nt_formats(Q, dt, bits, gs):
    """Non-transposed weights, every format: 16-row blocks 1..4, every output."""
    for M in (1, 6, 17, 64):
        print(f"nt {dt} {bits}-bit gs{gs} M={M} N=256 K=96", flush=True)
        (ok, worst), _ = nt_case(Q, dt, bits, gs, M, 256, 96, 9500 + 10 * bits + M)
        assert ok, (M, worst)


@pytest.mark.parametrize("dt,bits,gs,M,N,K", [
    ("f16", 4, 64, 4, 4096, 4096),     # verify shape, weights [K, N]
    ("bf16", 4, 64, 6, 1024, 4160),    # K past one staged chunk of scales
    ("f16", 8, 32, 16, 64, 8192),      # one line of columns (4 blocks, not a multiple of 8)
    ("bf16", 6, 128, 36, 384, 640),    # 24 blocks
    ("f16", 4, 32, 64, 1024, 2048),
])
def test_nt_shapes(Q, dt, bits, gs, M, N, K):
    print(f"nt {dt} {bits}-bit gs{gs} M={M} N={N} K={K}", flush=True)
    (ok, worst), (x, wq, sc, bi, y) = nt_case(Q, dt, bits, gs, M, N, K, 9700 + M, outlier=0.01)
    assert ok, worst
    y2 = Q.small_m_nt(x, wq, sc, bi, bits, gs)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))  # deterministic


@pytest.mark.parametrize("dt,bits,gs,M,N,K", [
    ("f16", 4, 64, 6, 4096, 4096),      # transpose reads: 16 blocks of 256 columns x 16 slices
    ("bf16", 6, 128, 36, 384, 640),     # 3 workgroups x 10 slices of 64 rows
    ("f16", 8, 32, 16, 64, 8192),       # one workgroup holding 64 columns, 16 slices
    ("bf16", 4, 32, 64, 1024, 4160),    # 15 slices, the last one shorter
    ("f16", 4, 64, 4, 16448, 256),      # 129 workgroups: unsplit, the last one 64 columns wide
])
def test_nt_split(Q, dt, bits, gs, M, N, K):
    """Non-transposed weights with K split across 128-column workgroups (and
    the unsplit 128-column form for wide N): every output against the
    oracle, two calls bit-identical."""
    print(f"nt split {dt} {bits}-bit gs{gs} M={M} N={N} K={K} "
          f"workspace={Q.nt_workspace_bytes(DT[dt], bits, gs, M, N, K)}", flush=True)
    w = synth.normal((K, N), 0.02, dt, 9900 + M, outlier_frac=0.01)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    x = synth.normal((M, K), 1.0, dt, 9901 + M)
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    xc = x.cuda()
    y = Q.small_m_nt(xc, wq, sc, bi, bits, gs, split=True)
    torch.cuda.synchronize()
    yo, T = O.qmm_nt(synth.to_oracle(x), owq, osc, obi, dt, bits, gs, N)
    ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
    assert ok, worst
    y2 = Q.small_m_nt(xc, wq, sc, bi, bits, gs, split=True)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    y3 = Q.small_m_nt(xc, wq, sc, bi, bits, gs)
    ok3, worst3 = O.within_tolerance(O.to_f64(synth.to_oracle(y3), dt), yo, T)
    assert ok3, worst3


@pytest.mark.parametrize("dt,bits,gs,M,N,K", [
    ("bf16", 8, 32, 3, 4096, 4160),     # 8 groups per block; no divisor fits: 17 slices, the last 64 rows
    ("f16", 8, 128, 16, 4096, 4096),    # 2 groups per block, one full row block
    ("f16", 4, 64, 1, 4160, 2048),      # 17 blocks, the last 64 columns wide (scales one by one)
    ("bf16", 4, 64, 40, 4096, 4096),    # 3 row blocks
    ("f16", 4, 32, 64, 4352, 1024),     # 4 row blocks, 17 blocks
])
def test_nt_transpose_read_split(Q, dt, bits, gs, M, N, K):
    """The transpose-read K split (4/8-bit codes, N >= 4096): scale runs of
    8, 2 and 1 values, a 64-column last block, a short last slice, 1..4 row
    blocks.  Every output against the oracle; a second call on the same
    workspace bit-identical."""
    need = Q.nt_workspace_bytes(DT[dt], bits, gs, M, N, K)
    print(f"nt transpose-read split {dt} {bits}-bit gs{gs} M={M} N={N} K={K} workspace={need}", flush=True)
    assert need > 0  # a split
    w = synth.normal((K, N), 0.02, dt, 9950 + M, outlier_frac=0.01)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    x = synth.normal((M, K), 1.0, dt, 9951 + M)
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    xc = x.cuda()
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    y = Q.small_m_nt(xc, wq, sc, bi, bits, gs, split=True, workspace=ws)
    torch.cuda.synchronize()
    yo, T = O.qmm_nt(synth.to_oracle(x), owq, osc, obi, dt, bits, gs, N)
    ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
    assert ok, worst
    y2 = Q.small_m_nt(xc, wq, sc, bi, bits, gs, split=True, workspace=ws)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_nt_split_workspace_reuse(Q):
    """One workspace serves a sequence of K-split calls of different shapes
    and forms (transpose reads on 1..2 row blocks, the 16-wavefront form):
    every result bit-identical to a call on a fresh workspace."""
    cases = [("f16", 4, 64, 6, 4096, 4096), ("f16", 4, 64, 16, 14336, 4096), ("bf16", 8, 64, 24, 4096, 2048),
             ("f16", 6, 64, 6, 1024, 4096), ("bf16", 4, 32, 2, 8192, 1024)]
    need = max(Q.nt_workspace_bytes(DT[c[0]], *c[1:]) for c in cases)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    prepared = []
    for i, (dt, bits, gs, M, N, K) in enumerate(cases):
        w = synth.normal((K, N), 0.02, dt, 9980 + i, device="cuda")
        wq, sc, bi = Q.quantize(w, bits, gs)
        prepared.append((synth.normal((M, K), 1.0, dt, 9990 + i, device="cuda"), wq, sc, bi, bits, gs))
    for rep in range(2):
        for (dt, bits, gs, M, N, K), (x, wq, sc, bi, b, g) in zip(cases, prepared):
            print(f"nt workspace reuse pass {rep}: {dt} {bits}-bit gs{gs} M={M} N={N} K={K}", flush=True)
            y_fresh = Q.small_m_nt(x, wq, sc, bi, b, g, split=True)
            y = Q.small_m_nt(x, wq, sc, bi, b, g, split=True, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), y_fresh.view(torch.int16)), (dt, bits, gs, M, N, K)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [4, 6, 8])
def test_nt_smallest_shapes(Q, dt, bits):
    """The smallest non-transposed problems: K = 32 (one step), N = 64 (one
    workgroup of the split form holding half its columns), M = 1 and 17;
    split-free and with the K split, every output."""
    gs = 32
    for M, N, K in ((1, 64, 32), (17, 64, 32), (1, 64, 128), (17, 192, 64)):
        print(f"nt smallest {dt} {bits}-bit M={M} N={N} K={K}", flush=True)
        w = synth.normal((K, N), 0.02, dt, 9950 + bits + K)
        owq, osc, obi = oracle_quant(w, dt, bits, gs)
        x = synth.normal((M, K), 1.0, dt, 9951 + M)
        wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
        yo, T = O.qmm_nt(synth.to_oracle(x), owq, osc, obi, dt, bits, gs, N)
        for split in (False, True):
            y = Q.small_m_nt(x.cuda(), wq, sc, bi, bits, gs, split=split)
            torch.cuda.synchronize()
            ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
            assert ok, (M, N, K, split, worst)


def test_batched_and_nt_empty_problems(Q):
    """Empty batched and non-transposed problems launch nothing and return
    empty outputs of the right shapes."""
    x = torch.zeros((0, 4, 256), dtype=torch.float16, device="cuda")
    wq = torch.zeros((0, 64, 32), dtype=torch.int32, device="cuda")
    sb = torch.zeros((0, 64, 4), dtype=torch.float16, device="cuda")
    assert Q.small_m_batched(x, wq, sb, sb, 4, 64).shape == (0, 4, 64)
    w = synth.normal((3, 64, 256), 0.02, "f16", 1).cuda()
    qs = [Q.quantize(w[b], 4, 64) for b in range(3)]
    wq3, sc3, bi3 = (torch.stack([q[i] for q in qs]) for i in range(3))
    x0 = torch.zeros((3, 0, 256), dtype=torch.float16, device="cuda")
    assert Q.small_m_batched(x0, wq3, sc3, bi3, 4, 64).shape == (3, 0, 64)
    wkn = synth.normal((256, 128), 0.02, "f16", 2).cuda()
    wqn, scn, bin_ = Q.quantize(wkn, 4, 64)
    xn = torch.zeros((0, 256), dtype=torch.float16, device="cuda")
    assert Q.small_m_nt(xn, wqn, scn, bin_, 4, 64).shape == (0, 128)
    assert Q.small_m_nt(xn, wqn, scn, bin_, 4, 64, split=True).shape == (0, 128)


@pytest.mark.parametrize("dt,gs,K,splits", [("f16", 64, 14336, (7,)), ("bf16", 32, 8192, (2, 4)),
                                             ("f16", 128, 8192, (2,))])
def test_reg_split_k(Q, dt, gs, K, splits):
    """The register kernel's K split (slices it covers, fp32 partials in the
    workspace, fixed-order reduction; above 16 rows also on 16-row blocks)
    over a ragged N (258 tiles of 16), every output checked; two runs
    bit-identical."""
    N = 16 * 257 + 5
    w = synth.normal((N, K), 0.02, dt, 8000 + gs)
    owq, osc, obi = oracle_quant(w, dt, 4, gs)
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    for M in (1, 8, 16, 24, 48, 64):
        x = synth.normal((M, K), 1.0, dt, 8100 + M)
        yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, 4, gs)
        for split in splits:
            print(f"reg split {dt} gs{gs} M={M} N={N} K={K} split={split}", flush=True)
            y0 = Q.small_m_ws(x.cuda(), wq, sc, bi, 4, gs, kernel=Q.KERNEL_MFMA_REG, split=split)
            y1 = Q.small_m_ws(x.cuda(), wq, sc, bi, 4, gs, kernel=Q.KERNEL_MFMA_REG, split=split)
            torch.cuda.synchronize()
            assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
            ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y0), dt), yo, T)
            assert ok, (M, split, worst)


@pytest.mark.parametrize("M", [8, 16, 24, 36, 64])
def test_small_m_ws_planned(Q, M):
    """qmm_small_m_ws with its own plan on the down projection (4096 x 14336:
    the register kernel on 7 K slices at M <= 16, the 64-column tile kernel
    split 4 ways above) against the oracle; a plan without a split takes no
    workspace."""
    dt, bits, gs, N, K = "f16", 4, 64, 4096, 14336
    assert Q.split_plan(torch.float16, bits, gs, M, N, K)[1] > 1
    w = synth.normal((N, K), 0.02, dt, 900 + M)
    owq, osc, obi = oracle_quant(w, dt, bits, gs)
    wq, sc, bi = (synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(),
                  synth.from_oracle(obi, dt).cuda())
    x = synth.normal((M, K), 1.0, dt, 901 + M)
    need = Q.workspace_bytes(torch.float16, bits, gs, M, N, K)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    print(f"ws planned M={M} need={need}", flush=True)
    y = Q.small_m_ws(x.cuda(), wq, sc, bi, bits, gs, workspace=ws)
    torch.cuda.synchronize()
    yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
    ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
    assert ok, worst
    # no split planned (verify rows): no workspace needed, same path as qmm_small_m
    assert Q.workspace_bytes(torch.float16, bits, gs, 6, 4096, 4096) == 0


def test_small_m_ws_errors(Q):
    w = synth.normal((4096, 14336), 0.02, "f16", 1).cuda()
    wq, sc, bi = Q.quantize(w, 4, 64)
    x = torch.ones((32, 14336), dtype=torch.float16, device="cuda")
    need = Q.workspace_bytes(torch.float16, 4, 64, 32, 4096, 14336)
    small = torch.empty((need - 64,), dtype=torch.uint8, device="cuda")
    with pytest.raises(Q.QmmError) as e:
        Q.small_m_ws(x, wq, sc, bi, 4, 64, workspace=small)
    assert e.value.status == Q.QMM_ERR_INVALID_ARG

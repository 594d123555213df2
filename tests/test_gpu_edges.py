"""GPU parity on the method's edge cases, through every matmul path.

The weights and activations here are the ones that stress the arithmetic
rather than the layout:
  * constant groups (scale 0), groups spanning a few ulps, and a random mix of
    those with normal and outlier groups (the quantizer's degenerate cases);
  * all-positive activations and weights (no cancellation: the tightest case
    for the accepted error, dominated by bf16 output rounding);
  * fp16 activations far from N(0, 1): whole quantization groups of values
    +-100..1000 and single spikes, whose unit sums exceed fp16's range;
  * the narrowest ring form (8-bit, group 32, K = 256, a single activation
    row of 512 bytes);
  * 6/8-bit codes at wide N above 16 rows, where fp16 runs the kernel that
    dequantizes the weights into LDS.
Every path a caller can reach is run on them: each kernel variant that
supports the shape (including the register kernel's single-tile, LDS-ring and
row-block forms), the K split with a workspace, the batched entry point and
the non-transposed entry point.  Every output is checked against the oracle
(|y - y_o| <= 4e-3 sum_k |x_k| |w_hat_k| + 1e-3)."""

import numpy as np
import pytest
import torch

import synth
from oracle import qmm_oracle as O

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import affine_quantized_gemm_amd as Q
    return Q


def _dev(a, dt=None):
    return synth.from_oracle(a, dt).cuda()


class Prepared:
    """A weight matrix quantized by the oracle, with its device copies."""

    def __init__(self, dt, bits, gs, w):
        self.dt, self.bits, self.gs = dt, bits, gs
        self.N, self.K = w.shape
        self.owq, self.osc, self.obi = O.quantize(synth.to_oracle(w), dt, bits, gs)
        self.wq, self.sc, self.bi = _dev(self.owq), _dev(self.osc, dt), _dev(self.obi, dt)


def check_all_paths(Q, P, xs, label, splits=True, batched=True, worst_out=None):
    """Every path for each activation block in ``xs`` (host tensors [M, K]);
    one oracle product over all of them stacked (rows are independent)."""
    dt, bits, gs, N, K = P.dt, P.bits, P.gs, P.N, P.K
    tdt = DT[dt]
    yo_all, T_all = O.qmm(np.concatenate([synth.to_oracle(x) for x in xs]), P.owq, P.osc, P.obi, dt, bits, gs)
    ran = []
    r0 = 0
    for x in xs:
        M = x.shape[0]
        yo, T = yo_all[r0:r0 + M], T_all[r0:r0 + M]
        r0 += M
        xc = x.cuda()

        def verify(y, what):
            torch.cuda.synchronize()
            ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
            if worst_out is not None:
                worst_out.append(worst)
            assert ok, (label, M, what, worst)

        for kernel in (None, Q.KERNEL_VALU, Q.KERNEL_MFMA_REG, Q.KERNEL_MFMA_PASS, Q.KERNEL_MFMA_TILE16,
                       Q.KERNEL_MFMA_TILE64, Q.KERNEL_MFMA_DQLDS):
            if kernel is not None and not Q.kernel_supported(tdt, bits, gs, M, N, K, kernel):
                continue
            what = "dispatch" if kernel is None else Q.kernel_name(kernel)
            print(f"{label}: {dt} {bits}-bit gs{gs} M={M} N={N} K={K} {what}", flush=True)
            verify(Q.small_m(xc, P.wq, P.sc, P.bi, bits, gs, kernel=kernel), what)
            ran.append(what)
        if splits:
            # the planned workspace path, then forced splits where they run
            # (a variant that cannot take the split returns UNSUPPORTED
            # before launching anything)
            print(f"{label}: M={M} small_m_ws planned", flush=True)
            verify(Q.small_m_ws(xc, P.wq, P.sc, P.bi, bits, gs), "ws planned")
            for kernel, split in ((Q.KERNEL_MFMA_REG, 2), (Q.KERNEL_MFMA_TILE16, 3), (Q.KERNEL_MFMA_TILE64, 2)):
                what = f"split {Q.kernel_name(kernel)} x{split}"
                try:
                    y = Q.small_m_ws(xc, P.wq, P.sc, P.bi, bits, gs, kernel=kernel, split=split)
                except Q.QmmError as e:
                    if e.status != Q.QMM_ERR_UNSUPPORTED:
                        raise
                    continue
                print(f"{label}: M={M} {what}", flush=True)
                verify(y, what)
                ran.append(what)
        if batched:
            print(f"{label}: M={M} batched x2", flush=True)
            args = (torch.stack([xc, xc]), torch.stack([P.wq, P.wq]), torch.stack([P.sc, P.sc]),
                    torch.stack([P.bi, P.bi]), bits, gs)
            entry_bytes = (M * K * 2, N * K * bits // 8, N * (K // gs) * 2, M * N * 2)
            if any(b % 16 for b in entry_bytes):
                # the second entry's arrays would start misaligned: refused
                with pytest.raises(Q.QmmError) as e:
                    Q.small_m_batched(*args)
                assert e.value.status == Q.QMM_ERR_MISALIGNED
            else:
                yb = Q.small_m_batched(*args)
                verify(yb[0], "batched entry 0")
                verify(yb[1], "batched entry 1")
    return ran


def check_nt(Q, dt, bits, gs, w_kn, x, label):
    """Non-transposed entry point (split-free and K split) on W [K, N]."""
    K, N = w_kn.shape
    owq, osc, obi = O.quantize(synth.to_oracle(w_kn), dt, bits, gs)
    yo, T = O.qmm_nt(synth.to_oracle(x), owq, osc, obi, dt, bits, gs, N)
    wq, sc, bi = _dev(owq), _dev(osc, dt), _dev(obi, dt)
    for split in (False, True):
        print(f"{label}: nt {dt} {bits}-bit gs{gs} M={x.shape[0]} N={N} K={K} split={split}", flush=True)
        y = Q.small_m_nt(x.cuda(), wq, sc, bi, bits, gs, split=split)
        torch.cuda.synchronize()
        ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo, T)
        assert ok, (label, split, worst)


FORMATS = [("f16", 4, 64), ("bf16", 4, 32), ("f16", 4, 128), ("bf16", 6, 64), ("f16", 6, 128),
           ("bf16", 8, 64), ("f16", 8, 32)]
# (N, K): the register kernel single-tile (1000 columns, K = 4096: 16
# wavefronts, 2 or 4 k-blocks each) and multi-tile (more 16-column tiles than
# resident workgroups, ragged last tile; the LDS-ring form at 4 and 8 bits)
SHAPES = [(1000, 4096), (16 * 300 + 5, 2048)]


@pytest.mark.parametrize("kind", ["constant", "tiny", "mixed"])
@pytest.mark.parametrize("dt,bits,gs", FORMATS)
def test_special_groups_every_path(Q, kind, dt, bits, gs):
    """Constant, tiny-range and mixed groups through every matmul path."""
    for si, (N, K) in enumerate(SHAPES):
        P = Prepared(dt, bits, gs, synth.special_groups(kind, N, K, gs, dt, 11000 + 10 * bits + gs + si))
        xs = [synth.normal((M, K), 1.0, dt, 11100 + M + si) for M in (6, 40)]
        check_all_paths(Q, P, xs, f"{kind} N={N}", batched=(si == 0))
    wk = synth.special_groups(kind, 256, 1024, gs, dt, 11200 + bits + gs)  # W [K, N], groups along N
    check_nt(Q, dt, bits, gs, wk, synth.normal((6, 256), 1.0, dt, 11201), kind)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("bits,gs", [(4, 64), (4, 128), (6, 32), (8, 64)])
def test_all_positive_inputs(Q, dt, bits, gs):
    """x >= 0 and W >= 0: no cancellation anywhere, so y is as large as T
    allows and the output rounding uses most of the accepted error in bf16."""
    worst = []
    for si, (N, K) in enumerate(SHAPES):
        P = Prepared(dt, bits, gs, synth.normal((N, K), 0.02, dt, 12000 + bits + gs + si).abs())
        xs = [synth.normal((M, K), 1.0, dt, 12100 + M + si).abs() for M in (4, 6, 24)]
        check_all_paths(Q, P, xs, f"positive N={N}", batched=(si == 0), worst_out=worst)
    wk = synth.normal((512, 1024), 0.02, dt, 12200 + bits).abs()
    check_nt(Q, dt, bits, gs, wk, synth.normal((6, 512), 1.0, dt, 12201).abs(), "positive")
    print(f"all-positive {dt} {bits}-bit gs{gs}: worst err/bound {max(worst):.3f}", flush=True)


def large_activations(M, K, dt, seed):
    """N(0, 1) rows in which some whole 128-wide (hence group-covering)
    blocks hold one value of +-100..1000 and a few single elements spikes of
    +-2000..30000 (y stays well inside fp16's range)."""
    rng = np.random.default_rng(seed)
    x = synth.normal((M, K), 1.0, "f16", seed).float().numpy()
    nblk = K // 128
    for m in range(M):
        for blk in rng.choice(nblk, size=max(1, nblk // 8), replace=False):
            x[m, blk * 128:(blk + 1) * 128] = rng.choice([-1.0, 1.0]) * rng.uniform(100.0, 1000.0)
        spikes = rng.choice(K, size=4, replace=False)
        x[m, spikes] = rng.choice([-1.0, 1.0], size=4) * rng.uniform(2000.0, 30000.0, size=4)
    return torch.from_numpy(x).to(DT[dt])


@pytest.mark.parametrize("dt,bits,gs", [("f16", 4, 64), ("f16", 4, 128), ("f16", 4, 32), ("f16", 6, 64),
                                        ("f16", 8, 128), ("f16", 8, 32), ("bf16", 4, 64)])
def test_large_activations_every_path(Q, dt, bits, gs):
    """Whole groups of activations at +-100..1000 and single spikes: the
    register kernel's unit sums (sum x * code offset) pass fp16's largest
    value; every form and path must still be within tolerance."""
    for si, (N, K) in enumerate(SHAPES):
        P = Prepared(dt, bits, gs, synth.normal((N, K), 0.02, dt, 13000 + bits + gs + si, outlier_frac=0.01))
        xs = [large_activations(M, K, dt, 13100 + M + si) for M in (1, 6, 16, 40)]
        check_all_paths(Q, P, xs, f"large-x N={N}", batched=(si == 0))
    # K deeper than the register kernel takes whole: its K split and the pass kernel
    P = Prepared(dt, bits, gs, synth.normal((16 * 300 + 5, 8192), 0.02, dt, 13200 + bits + gs))
    check_all_paths(Q, P, [large_activations(8, 8192, dt, 13201)], "large-x K=8192", batched=False)
    wk = synth.normal((512, 1024), 0.02, dt, 13300 + bits + gs)
    check_nt(Q, dt, bits, gs, wk, large_activations(6, 512, dt, 13301), "large-x")


@pytest.mark.parametrize("kind", ["constant", "tiny", "mixed", "positive", "large-x"])
@pytest.mark.parametrize("dt,bits,gs", [("f16", 6, 32), ("f16", 8, 128), ("bf16", 8, 64)])
def test_wide_n_dequant_to_lds_path(Q, kind, dt, bits, gs):
    """6/8-bit codes at N >= 8192 above 16 rows, where the dispatch takes the
    kernel that dequantizes the weights into LDS (fp16; bf16 takes the
    64-column tile kernel): the edge cases above through it and every other
    path that runs the shape."""
    N, K = 8192, 512
    seed = 14000 + 10 * bits + gs
    if kind in ("constant", "tiny", "mixed"):
        w = synth.special_groups(kind, N, K, gs, dt, seed)
    else:
        w = synth.normal((N, K), 0.02, dt, seed, outlier_frac=0.01)
        if kind == "positive":
            w = w.abs()
    if kind == "large-x" and dt == "f16":
        xs = [large_activations(M, K, dt, seed + M) for M in (24, 40)]
    else:
        xs = [synth.normal((M, K), 1.0, dt, seed + M) for M in (24, 40)]
        if kind == "positive":
            xs = [x.abs() for x in xs]
    P = Prepared(dt, bits, gs, w)
    want = "mfma_splitfree_dqlds" if dt == "f16" else "mfma_splitfree_tile64"
    assert Q.kernel_name(Q.select_kernel(DT[dt], bits, gs, 24, N, K)) == want
    ran = check_all_paths(Q, P, xs, f"{kind} N={N}", batched=False)
    assert "mfma_splitfree_dqlds" in ran


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_narrowest_ring_form(Q, dt):
    """8-bit, group 32, K = 256 at M <= 8 over more 16-column tiles than the
    1024 resident 4-wavefront workgroups: the 2-slot weight ring, whose loads
    past a workgroup's last tile must stay inside the arrays (one activation
    row is only 512 bytes here).  Every output checked."""
    bits, gs, K, N = 8, 32, 256, 16 * 1027 + 5
    assert Q.select_kernel(DT[dt], bits, gs, 1, N, K) == Q.KERNEL_MFMA_REG
    P = Prepared(dt, bits, gs, synth.normal((N, K), 0.02, dt, 14000))
    xs = [synth.normal((M, K), 1.0, dt, 14001 + M) for M in (1, 3, 8)]
    check_all_paths(Q, P, xs, "ring K=256", splits=False)


def test_verify_shape_every_output(Q):
    """The verify workload (M = 4 and 6, K = N = 4096, 4-bit, group 64, fp16)
    in the launch configuration the benchmark times, every output checked."""
    dt, bits, gs, N, K = "f16", 4, 64, 4096, 4096
    P = Prepared(dt, bits, gs, synth.normal((N, K), 0.02, dt, 15000))
    xs = [synth.normal((M, K), 1.0, dt, 15001 + M) for M in (4, 6)]
    check_all_paths(Q, P, xs, "verify", splits=False, batched=False)


@pytest.mark.parametrize("bits", [4, 8])
def test_lm_head_ragged_tail(Q, bits):
    """A wide LM-head-like product whose N is not a multiple of the 16-column
    tile (N = 151936 + 5): the shifted last tile of the multi-tile forms.
    Quantized on the GPU; the first 64 and last 400 columns and a random
    sample are checked (the quantizer bit-exact on those rows)."""
    dt, gs, K, N = "bf16", 64, 4096, 151936 + 5
    dev = torch.device("cuda")
    w = synth.normal((N, K), 0.02, dt, 16000 + bits, device=dev)
    wq, sc, bi = Q.quantize(w, bits, gs)
    rng = np.random.default_rng(16000 + bits)
    cols = np.unique(np.concatenate([np.arange(64), np.arange(N - 400, N), rng.choice(N, 512, replace=False)]))
    idx = torch.from_numpy(cols).to(dev)
    owq, osc, obi = O.quantize(synth.to_oracle(w.index_select(0, idx)), dt, bits, gs)
    assert np.array_equal(synth.to_oracle(wq.index_select(0, idx)), owq)
    del w
    for M in (4, 6):
        x = synth.normal((M, K), 1.0, dt, 16100 + M, device=dev)
        yo, T = O.qmm(synth.to_oracle(x), owq, osc, obi, dt, bits, gs)
        print(f"lm head ragged {bits}-bit M={M} N={N}", flush=True)
        y = Q.small_m(x, wq, sc, bi, bits, gs)
        ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y.index_select(1, idx)), dt), yo, T)
        assert ok, (M, worst)

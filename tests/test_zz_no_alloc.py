"""qmm_small_m_noalloc (the entry point for callers that cannot allocate):
through the C ABI, against qmm_small_m_ws on the same inputs -- bit for bit,
since it runs the same plan and kernels -- and against the oracle, on two
calls in a row, the second smaller (the scratch keeps the first call's
partial sums, which must not leak into the second)."""

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


def noalloc_abi(Q, x, wq, sc, bi, bits, gs, y):
    M, K = x.shape
    N = wq.shape[0]
    return Q.qmm_small_m_noalloc(Q.QMM_F16 if x.dtype == torch.float16 else Q.QMM_BF16, bits, gs, M, N, K,
                                 x.data_ptr(), wq.data_ptr(), sc.data_ptr(), bi.data_ptr(), y.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("dt,bits,gs,N,K,Ms", [
    ("f16", 4, 64, 4096, 14336, (64, 8)),    # 64-column tiles split 4 ways, then the register kernel on 7 slices
    ("bf16", 4, 32, 4096, 8192, (36, 16)),   # split plans at both sizes, the second smaller
    ("f16", 8, 64, 4096, 4096, (36, 6)),     # a split, then a call with no split planned
])
def test_noalloc_matches_workspace_entry_point(Q, dt, bits, gs, N, K, Ms):
    w = synth.normal((N, K), 0.02, dt, 17000 + bits + gs)
    owq, osc, obi = O.quantize(synth.to_oracle(w), dt, bits, gs)
    wq, sc, bi = synth.from_oracle(owq).cuda(), synth.from_oracle(osc, dt).cuda(), synth.from_oracle(obi, dt).cuda()
    tdt = synth.TORCH_DT[dt]
    xs = [synth.normal((M, K), 1.0, dt, 17100 + M) for M in Ms]
    yo_all, T_all = O.qmm(np.concatenate([synth.to_oracle(x) for x in xs]), owq, osc, obi, dt, bits, gs)
    r0 = 0
    for x in xs:
        M = x.shape[0]
        need = Q.workspace_bytes(tdt, bits, gs, M, N, K)
        print(f"noalloc {dt} {bits}-bit gs{gs} M={M} N={N} K={K} plan={Q.split_plan(tdt, bits, gs, M, N, K)} "
              f"workspace={need}", flush=True)
        assert need <= Q.NOALLOC_SCRATCH_BYTES
        xc = x.cuda()
        y = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        assert noalloc_abi(Q, xc, wq, sc, bi, bits, gs, y) == Q.QMM_OK
        y_ws = Q.small_m_ws(xc, wq, sc, bi, bits, gs)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ws.view(torch.int16)), M
        ok, worst = O.within_tolerance(O.to_f64(synth.to_oracle(y), dt), yo_all[r0:r0 + M], T_all[r0:r0 + M])
        assert ok, (M, worst)
        r0 += M


def test_noalloc_tensor_helper_and_oversized_problem(Q):
    """The tensor helper gives the same result; a problem whose planned
    workspace exceeds the scratch is refused before anything runs."""
    dt, bits, gs, N, K, M = "f16", 4, 64, 4096, 14336, 24
    w = synth.normal((N, K), 0.02, dt, 17500).cuda()
    wq, sc, bi = Q.quantize(w, bits, gs)
    x = synth.normal((M, K), 1.0, dt, 17501).cuda()
    y = Q.small_m_noalloc(x, wq, sc, bi, bits, gs)
    assert torch.equal(y.view(torch.int16), Q.small_m_ws(x, wq, sc, bi, bits, gs).view(torch.int16))
    big_n = 32768
    assert Q.workspace_bytes(torch.float16, bits, gs, 16, big_n, K) > Q.NOALLOC_SCRATCH_BYTES
    with pytest.raises(Q.QmmError) as e:
        Q.small_m_noalloc(torch.zeros((16, K), dtype=torch.float16, device="cuda"),
                          torch.zeros((big_n, K // 8), dtype=torch.int32, device="cuda"),
                          torch.zeros((big_n, K // gs), dtype=torch.float16, device="cuda"),
                          torch.zeros((big_n, K // gs), dtype=torch.float16, device="cuda"), bits, gs)
    assert e.value.status == Q.QMM_ERR_UNSUPPORTED

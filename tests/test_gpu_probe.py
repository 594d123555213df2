"""The measurement helpers do what qmm.h says: the copy moves every byte,
the streaming read runs to completion on sizes with and without a ragged
tail of 16-byte units, and the C launch loop makes the calls it names."""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def Q():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import affine_quantized_gemm_amd as Q
    return Q


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (8 << 20) + 16 * 7])
def test_copy_exact(Q, nbytes):
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    Q.probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("nbytes,grid", [(16, 0), (4096 + 48, 0), ((8 << 20) + 16 * 7, 1024), (64 << 20, 4096)])
def test_stream_read_runs(Q, nbytes, grid, shape):
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    Q.probe_stream_read(src, sink, grid, shape)
    torch.cuda.synchronize()
    # all-ones data XOR-reduces to a value that is never the kernel's trigger
    assert int(sink.abs().sum()) == 0


def test_small_m_loop_matches_calls(Q):
    """The C launch loop makes the same calls as qmm_small_m one by one:
    after it, y holds the product with the last weight set, bit for bit."""
    import synth
    M, N, K, bits, gs = 6, 1024, 2048, 4, 64
    stack = []
    for i in range(3):
        w = synth.normal((N, K), 0.02, "f16", 18000 + i).cuda()
        stack.append(Q.quantize(w, bits, gs))
    x = synth.normal((M, K), 1.0, "f16", 18100).cuda()
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    Q.probe_small_m_loop(x, stack, bits, gs, y, passes=2)
    ref = Q.small_m(x, *stack[-1], bits, gs)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))

"""The tensor-level helpers check every operand's shape, dtype and device
against the problem size before any pointer reaches the library.

These run on the CPU: with host tensors, a call whose operands are
consistent gets as far as the device check ("must be a GPU tensor"), and a
call with any inconsistent operand is rejected before it."""

import pytest
import torch

import affine_quantized_gemm_amd as Q

F16, BF16 = torch.float16, torch.bfloat16


def operands(M=4, N=48, K=256, bits=4, gs=64, dt=F16, batch=None):
    lead = () if batch is None else (batch,)
    x = torch.zeros((*lead, M, K), dtype=dt)
    wq = torch.zeros((*lead, N, K * bits // 32), dtype=torch.int32)
    sc = torch.zeros((*lead, N, K // gs), dtype=dt)
    bi = torch.zeros((*lead, N, K // gs), dtype=dt)
    return x, wq, sc, bi


def consistent(call):
    """A consistent call on host tensors fails only at the device check."""
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call()


def rejected(call, match):
    with pytest.raises((ValueError, Q.QmmError), match=match):
        call()


def test_small_m_consistent_operands_reach_the_device_check():
    x, wq, sc, bi = operands()
    consistent(lambda: Q.small_m(x, wq, sc, bi, 4, 64))
    consistent(lambda: Q.small_m(x, wq, sc, bi, 4, 64, out=torch.zeros((4, 48), dtype=F16)))
    x6, wq6, sc6, bi6 = operands(bits=6, gs=128, dt=BF16)
    consistent(lambda: Q.small_m(x6, wq6, sc6, bi6, 6, 128))
    consistent(lambda: Q.small_m_ws(x6, wq6, sc6, bi6, 6, 128))


@pytest.mark.parametrize("case,match", [
    ("bits", "wq has shape"),            # packed for 4 bits, called with 8
    ("gs", "scales has shape"),          # scales for gs 64, called with 32
    ("wq_rows", "scales has shape"),     # wq and scales disagree on N
    ("wq_dtype", "wq has dtype"),
    ("sc_dtype", "scales has dtype"),    # bf16 scales with fp16 x
    ("bi_shape", "biases has shape"),
    ("out_shape", "out has shape"),      # too small an output
    ("out_dtype", "out has dtype"),
    ("x_dims", "x must be 2-D"),
    ("x_dtype", "dtype"),
    ("bad_bits", "bits=5"),
    ("bad_gs", "group_size=48"),
])
def test_small_m_rejects_inconsistent_operands(case, match):
    x, wq, sc, bi = operands()
    bits, gs, out = 4, 64, None
    if case == "bits":
        bits = 8
    elif case == "gs":
        gs = 32
    elif case == "wq_rows":
        wq = torch.zeros((47, 32), dtype=torch.int32)
    elif case == "wq_dtype":
        wq = torch.zeros((48, 32), dtype=torch.int64)
    elif case == "sc_dtype":
        sc = sc.to(BF16)
    elif case == "bi_shape":
        bi = torch.zeros((48, 3), dtype=F16)
    elif case == "out_shape":
        out = torch.zeros((4, 40), dtype=F16)
    elif case == "out_dtype":
        out = torch.zeros((4, 48), dtype=torch.float32)
    elif case == "x_dims":
        x = x.reshape(1, 4, 256)
    elif case == "x_dtype":
        x = x.to(torch.float32)
    elif case == "bad_bits":
        bits = 5
    elif case == "bad_gs":
        gs = 48
    rejected(lambda: Q.small_m(x, wq, sc, bi, bits, gs, out=out), match)
    rejected(lambda: Q.small_m_ws(x, wq, sc, bi, bits, gs, out=out), match)


def test_batched_checks_every_entry_shape():
    x, wq, sc, bi = operands(batch=3)
    consistent(lambda: Q.small_m_batched(x, wq, sc, bi, 4, 64))
    rejected(lambda: Q.small_m_batched(x, wq[:2], sc, bi, 4, 64), "wq has shape")
    rejected(lambda: Q.small_m_batched(x, wq, sc[:, :40], bi, 4, 64), "scales has shape")
    rejected(lambda: Q.small_m_batched(x, wq, sc, bi, 6, 64), "wq has shape")
    rejected(lambda: Q.small_m_batched(x, wq, sc, bi, 4, 64, out=torch.zeros((3, 4, 47), dtype=F16)),
             "out has shape")
    rejected(lambda: Q.small_m_batched(x[0], wq, sc, bi, 4, 64), "x must be 3-D")


def test_nt_checks_the_k_by_n_layout():
    M, K, N, bits, gs = 4, 96, 256, 4, 64
    x = torch.zeros((M, K), dtype=BF16)
    wq = torch.zeros((K, N * bits // 32), dtype=torch.int32)
    sc = torch.zeros((K, N // gs), dtype=BF16)
    consistent(lambda: Q.small_m_nt(x, wq, sc, sc.clone(), bits, gs))
    rejected(lambda: Q.small_m_nt(x, wq[:95], sc, sc.clone(), bits, gs), "wq has shape")
    rejected(lambda: Q.small_m_nt(x, wq, sc[:, :2], sc.clone(), bits, gs), "scales has shape")
    rejected(lambda: Q.small_m_nt(x, wq, sc, sc.clone(), bits, 32), "scales has shape")
    rejected(lambda: Q.small_m_nt(x, wq, sc, sc.clone(), bits, gs, out=torch.zeros((M, N), dtype=F16)),
             "out has dtype")


def test_quantize_and_dequantize_check_shapes():
    consistent(lambda: Q.quantize(torch.zeros((16, 256), dtype=F16), 4, 64))
    rejected(lambda: Q.quantize(torch.zeros((16, 256), dtype=F16), 4, 48), "group_size=48")
    rejected(lambda: Q.quantize(torch.zeros((16, 96), dtype=F16), 4, 64), "group_size=64")
    rejected(lambda: Q.quantize(torch.zeros((256,), dtype=F16), 4, 64), "2-D")
    _, wq, sc, bi = operands(N=16, K=256)
    consistent(lambda: Q.dequantize(wq, sc, bi, 4, 64))
    rejected(lambda: Q.dequantize(wq, sc, bi, 6, 64), "wq has shape")
    rejected(lambda: Q.dequantize(wq, sc, bi[:8], 4, 64), "biases has shape")


def test_small_m_loop_args_checks_every_weight_set():
    """The C launch loop's argument builder validates the weight sets of the
    stack against x and out (on host tensors a consistent set stops at the
    device check), and refuses an empty stack."""
    x, wq, sc, bi = operands()
    out = torch.zeros((4, 48), dtype=F16)
    with pytest.raises(ValueError, match="empty stack"):
        Q.small_m_loop_args(x, [], 4, 64, out)
    consistent(lambda: Q.small_m_loop_args(x, [(wq, sc, bi), (wq, sc, bi)], 4, 64, out))
    _, wq_b, sc_b, bi_b = operands(N=64)  # a second weight set of another width
    rejected(lambda: Q.small_m_loop_args(x, [(wq_b, sc_b, bi_b), (wq, sc, bi)], 4, 64, out), "out has shape")
    rejected(lambda: Q.small_m_loop_args(x, [(wq, sc_b, bi)], 4, 64, out), "scales has shape")

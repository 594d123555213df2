"""The C-ABI library loads without a GPU, exports every symbol qmm.h
declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

import affine_quantized_gemm_amd as Q

A = 0x10000          # a 16-byte-aligned fake address (never dereferenced)
MIS = 0x10008        # misaligned fake address


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qmm.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"qmm_quantize", "qmm_dequantize", "qmm_small_m"} <= set(names)
    lib = ctypes.CDLL(Q.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(Q.EXPORTS)


def mm(dt=0, bits=4, gs=64, M=4, N=64, K=256, x=A, wq=A, s=A, b=A, y=A):
    return Q.qmm_small_m(dt, bits, gs, M, N, K, x, wq, s, b, y, None)


@pytest.mark.parametrize("kw,status", [
    (dict(bits=5), Q.QMM_ERR_UNSUPPORTED),
    (dict(bits=2), Q.QMM_ERR_UNSUPPORTED),
    (dict(gs=48), Q.QMM_ERR_UNSUPPORTED),
    (dict(gs=16), Q.QMM_ERR_UNSUPPORTED),
    (dict(gs=128, K=192), Q.QMM_ERR_UNSUPPORTED),
    (dict(K=96, gs=32), Q.QMM_ERR_UNSUPPORTED),
    (dict(K=32, gs=32), Q.QMM_ERR_UNSUPPORTED),
    (dict(K=0), Q.QMM_ERR_UNSUPPORTED),
    (dict(M=65), Q.QMM_ERR_UNSUPPORTED),
    (dict(dt=2), Q.QMM_ERR_UNSUPPORTED),
    (dict(dt=-1), Q.QMM_ERR_UNSUPPORTED),
    (dict(M=-1), Q.QMM_ERR_INVALID_ARG),
    (dict(N=-3), Q.QMM_ERR_INVALID_ARG),
    (dict(K=-64), Q.QMM_ERR_INVALID_ARG),
    (dict(x=None), Q.QMM_ERR_INVALID_ARG),
    (dict(wq=None), Q.QMM_ERR_INVALID_ARG),
    (dict(s=None), Q.QMM_ERR_INVALID_ARG),
    (dict(b=None), Q.QMM_ERR_INVALID_ARG),
    (dict(y=None), Q.QMM_ERR_INVALID_ARG),
    (dict(x=MIS), Q.QMM_ERR_MISALIGNED),
    (dict(wq=MIS), Q.QMM_ERR_MISALIGNED),
    (dict(y=MIS), Q.QMM_ERR_MISALIGNED),
    (dict(M=0, x=None, y=None), Q.QMM_OK),     # empty problem: nothing launched
    (dict(N=0, wq=None, s=None, b=None, y=None), Q.QMM_OK),
])
def test_small_m_validation(kw, status):
    assert mm(**kw) == status


def test_forced_validation():
    args = (0, 4, 64, 4, 64, 256, A, A, A, A, A, None)
    assert Q.qmm_small_m_forced(*args, 99) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_small_m_forced(*args, -1) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_small_m_forced(0, 5, 64, 4, 64, 256, A, A, A, A, A, None, 0) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_small_m_forced(0, 4, 64, 0, 64, 256, None, A, A, A, None, None, 0) == Q.QMM_OK


def test_quantize_dequantize_validation():
    qz = Q.qmm_quantize
    assert qz(0, 7, 64, 8, 256, A, A, A, A, None) == Q.QMM_ERR_UNSUPPORTED
    assert qz(0, 4, 64, 8, 100, A, A, A, A, None) == Q.QMM_ERR_UNSUPPORTED
    assert qz(0, 4, 64, -8, 256, A, A, A, A, None) == Q.QMM_ERR_INVALID_ARG
    assert qz(0, 4, 64, 8, 256, None, A, A, A, None) == Q.QMM_ERR_INVALID_ARG
    assert qz(0, 4, 64, 8, 256, A, MIS, A, A, None) == Q.QMM_ERR_MISALIGNED
    assert qz(1, 6, 32, 0, 256, None, None, None, None, None) == Q.QMM_OK
    dq = Q.qmm_dequantize
    assert dq(3, 4, 64, 8, 256, A, A, A, A, None) == Q.QMM_ERR_UNSUPPORTED
    assert dq(0, 4, 64, 8, 256, A, A, None, A, None) == Q.QMM_ERR_INVALID_ARG
    assert dq(0, 4, 64, 8, 256, A, A, A, MIS, None) == Q.QMM_ERR_MISALIGNED
    assert dq(0, 8, 128, 0, 256, None, None, None, None, None) == Q.QMM_OK


def test_helpers():
    assert Q.packed_words(4, 4096) == 512
    assert Q.packed_words(6, 4096) == 768
    assert Q.packed_words(8, 64) == 16
    assert Q.packed_words(5, 64) == -1
    assert Q.packed_words(6, 48) == 9
    assert Q.packed_words(6, 4) == -1
    assert Q.strerror(Q.QMM_ERR_MISALIGNED).startswith("array base pointer")
    assert Q.strerror(12345) == "unknown status"
    names = {Q.kernel_name(k) for k in Q.KERNEL_IDS}
    assert len(names) == len(Q.KERNEL_IDS) and "?" not in names
    assert Q.kernel_name(17) == "?"


def test_kernel_supported():
    import torch
    f16 = torch.float16
    assert Q.kernel_supported(f16, 4, 64, 64, 4096, 4096, Q.KERNEL_VALU)
    # above 16 rows the register kernel runs on 16-row blocks: 4-bit with more tiles than
    # row-block slots, or any width with at most one tile per resident workgroup; K it covers
    # with 16 wavefronts
    assert Q.kernel_supported(f16, 4, 64, 17, 4096, 4096, Q.KERNEL_MFMA_REG)
    assert Q.kernel_supported(f16, 4, 64, 64, 14336, 4096, Q.KERNEL_MFMA_REG)
    assert Q.kernel_supported(f16, 4, 64, 17, 1024, 4096, Q.KERNEL_MFMA_REG)
    assert Q.kernel_supported(f16, 8, 64, 64, 4096, 4096, Q.KERNEL_MFMA_REG)
    assert Q.kernel_supported(f16, 6, 128, 40, 4096, 4096, Q.KERNEL_MFMA_REG)
    assert not Q.kernel_supported(f16, 8, 64, 17, 14336, 4096, Q.KERNEL_MFMA_REG)  # 8-bit, 896 tiles
    assert not Q.kernel_supported(f16, 4, 64, 17, 4096, 1024, Q.KERNEL_MFMA_REG)  # 8 wavefronts
    assert Q.kernel_supported(f16, 4, 64, 16, 4096, 1024, Q.KERNEL_MFMA_REG)
    assert not Q.kernel_supported(f16, 4, 64, 17, 4096, 14336, Q.KERNEL_MFMA_REG)
    assert not Q.kernel_supported(f16, 4, 64, 65, 4096, 4096, Q.KERNEL_MFMA_REG)
    assert not Q.kernel_supported(f16, 4, 64, 4, 4096, 4096, 42)
    assert Q.qmm_kernel_supported(0, 5, 64, 4, 64, 256, 0) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_kernel_supported(0, 4, 64, -1, 64, 256, 0) == Q.QMM_ERR_INVALID_ARG
    # whatever select_kernel picks must itself be supported
    for M in (1, 4, 6, 8, 16, 17, 32, 64):
        for K in (512, 4096, 14336):
            k = Q.select_kernel(f16, 4, 64, M, 4096, K)
            assert Q.kernel_supported(f16, 4, 64, M, 4096, K, k)


def test_select_kernel_is_total_over_supported_shapes():
    import torch
    for dt in (torch.float16, torch.bfloat16):
        for bits in (4, 6, 8):
            for gs in (32, 64, 128):
                for M in (1, 2, 4, 6, 8, 9, 16, 17, 32, 36, 48, 64):
                    for N, K in ((1, 64 * 2), (1024, 4096), (4096, 14336), (151936, 4096)):
                        if K % gs:
                            continue
                        k = Q.select_kernel(dt, bits, gs, M, N, K)
                        assert k in Q.KERNEL_IDS, (dt, bits, gs, M, N, K, k)
    assert Q.select_kernel(torch.float16, 4, 64, 65, 64, 256) == Q.QMM_ERR_UNSUPPORTED
    assert Q.select_kernel(torch.float16, 4, 64, -1, 64, 256) == Q.QMM_ERR_INVALID_ARG


def test_probe_validation():
    assert Q.qmm_probe_stream_read(A, -16, A, 0, 1, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_probe_stream_read(A, 24, A, 0, 1, None) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_probe_stream_read(None, 64, A, 0, 1, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_probe_stream_read(A, 64, None, 0, 1, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_probe_stream_read(MIS, 64, A, 0, 1, None) == Q.QMM_ERR_MISALIGNED
    assert Q.qmm_probe_stream_read(A, 64, A, -1, 1, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_probe_stream_read(None, 0, None, 0, 1, None) == Q.QMM_OK
    assert Q.qmm_probe_stream_read(A, 64, A, 0, 2, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_probe_stream_read(A, 64, A, 0, -1, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_probe_copy(A, A, 8, None) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_probe_copy(A, MIS, 64, None) == Q.QMM_ERR_MISALIGNED
    assert Q.qmm_probe_copy(A, None, 64, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_probe_copy(None, None, 0, None) == Q.QMM_OK


def test_probe_small_m_loop_validation():
    """The C launch loop checks its own arguments, then stops at the first
    call that qmm_small_m rejects (all before any HIP call)."""
    arr = ctypes.c_void_p * 2
    ptrs = arr(A, A)
    loop = Q.qmm_probe_small_m_loop
    assert loop(0, 4, 64, 4, 64, 256, A, ptrs, ptrs, ptrs, A, -1, 1, None) == Q.QMM_ERR_INVALID_ARG
    assert loop(0, 4, 64, 4, 64, 256, A, ptrs, ptrs, ptrs, A, 2, -1, None) == Q.QMM_ERR_INVALID_ARG
    assert loop(0, 4, 64, 4, 64, 256, A, None, ptrs, ptrs, A, 2, 1, None) == Q.QMM_ERR_INVALID_ARG
    assert loop(0, 4, 64, 4, 64, 256, A, ptrs, ptrs, None, A, 2, 1, None) == Q.QMM_ERR_INVALID_ARG
    assert loop(0, 4, 64, 4, 64, 256, A, None, None, None, A, 0, 1, None) == Q.QMM_OK
    assert loop(0, 4, 64, 4, 64, 256, A, ptrs, ptrs, ptrs, A, 2, 0, None) == Q.QMM_OK
    # each call's own validation: a bad format, a misaligned first weight set
    assert loop(0, 5, 64, 4, 64, 256, A, ptrs, ptrs, ptrs, A, 2, 1, None) == Q.QMM_ERR_UNSUPPORTED
    assert loop(0, 4, 64, 4, 64, 256, A, arr(MIS, A), ptrs, ptrs, A, 2, 1, None) == Q.QMM_ERR_MISALIGNED


def test_dispatch_follows_measured_crossovers():
    """qmm_select_kernel encodes the crossovers measured on MI355X
    (affine_quantized_gemm_amd/sweep.py): the register-resident MFMA kernel
    wherever it runs (M <= 16 with K <= 4096; above 16 rows on 16-row blocks:
    4-bit when N has more tiles than their slots, any width when 16 rows take
    one tile per workgroup); otherwise M <= 16 -> the
    pass kernel; M > 16 -> for wide N the weights dequantized into LDS
    (fp16, 6/8-bit) or the 64-column tile kernel, the 16-column
    tile kernel for M > 32 when N gives every CU a tile, the pass kernel
    otherwise (and wherever the tile kernels cannot run)."""
    import torch
    f16, bf16 = torch.float16, torch.bfloat16
    sel = lambda dt, b, gs, M, N, K: Q.kernel_name(Q.select_kernel(dt, b, gs, M, N, K))
    for M in (1, 2, 3, 4, 6, 8, 16):
        assert sel(f16, 4, 64, M, 4096, 4096) == "mfma_splitfree_reg"
        assert sel(f16, 8, 64, M, 4096, 4096) == "mfma_splitfree_reg"
        assert sel(bf16, 4, 64, M, 151936, 4096) == "mfma_splitfree_reg"
        assert sel(f16, 4, 64, M, 4096, 14336) == "mfma_splitfree_pass"
    for M in (17, 24, 32, 36, 48, 64):
        assert sel(f16, 4, 64, M, 14336, 4096) == "mfma_splitfree_reg"
        assert sel(f16, 4, 64, M, 4096, 4096) == "mfma_splitfree_reg"
        assert sel(bf16, 4, 64, M, 151936, 4096) == "mfma_splitfree_reg"
        assert sel(bf16, 8, 64, M, 151936, 4096) == "mfma_splitfree_tile64"
        # 16 rows take one tile per workgroup: the register kernel on tiles x row blocks
        assert sel(f16, 8, 64, M, 4096, 4096) == "mfma_splitfree_reg"
        assert sel(bf16, 6, 128, M, 4096, 4096) == "mfma_splitfree_reg"
        assert sel(f16, 4, 64, M, 1024, 4096) == "mfma_splitfree_reg"
        assert sel(f16, 4, 64, M, 4096, 14336) == ("mfma_splitfree_tile16" if M > 32 else "mfma_splitfree_pass")
        # fp16 6/8-bit at wide N: the weights dequantized into LDS (bf16: 64-column tiles)
        assert sel(f16, 8, 64, M, 14336, 4096) == "mfma_splitfree_dqlds"
        assert sel(f16, 6, 32, M, 14336, 4096) == "mfma_splitfree_dqlds"
        assert sel(bf16, 6, 32, M, 14336, 4096) == "mfma_splitfree_tile64"
        assert sel(f16, 8, 64, M, 14336, 4160) == "mfma_splitfree_tile64"  # K not a multiple of 256
        # 6/8-bit with more tiles than resident workgroups, N >= 4096 but < 8192
        assert sel(f16, 8, 64, M, 6144, 4096) == ("mfma_splitfree_tile16" if M > 32 else "mfma_splitfree_pass")
        # fewer 16-column tiles than CUs, K the register kernel does not take: the pass kernel
        assert sel(f16, 4, 64, M, 1024, 4160) == "mfma_splitfree_pass"
        # K that is not a whole number of 4-bit k-blocks: the pass kernel
        assert sel(f16, 4, 64, M, 14336, 4160) == "mfma_splitfree_pass"
    assert sel(f16, 6, 64, 40, 4096, 4160) == "mfma_splitfree_tile16"   # 6-bit k-blocks are 64 codes
    # 6/8-bit at group size 32 above 48 rows: the 16-column tile kernel (sweep.py --formats)
    for dt in (f16, bf16):
        for b in (6, 8):
            assert sel(dt, b, 32, 64, 4096, 4096) == "mfma_splitfree_tile16"
            assert sel(dt, b, 32, 48, 4096, 4096) == "mfma_splitfree_reg"
            assert sel(dt, b, 64, 64, 4096, 4096) == "mfma_splitfree_reg"


def test_dispatch_matches_the_format_sweep():
    """Every (format, shape, M) row measured by sweep.py --formats (committed
    in profiles/dispatch_formats.md): the variant qmm_select_kernel returns
    now is within 5 % of the fastest measured one."""
    import torch
    rows = []
    with open(os.path.join(ROOT, "profiles", "dispatch_formats.md")) as f:
        lines = [l for l in f if l.startswith("| ") and not l.startswith("| shape") and "---" not in l]
    header = None
    with open(os.path.join(ROOT, "profiles", "dispatch_formats.md")) as f:
        for l in f:
            if l.startswith("| shape"):
                header = [c.strip() for c in l.strip().strip("|").split("|")]
    assert header and len(lines) == 324
    names = {"reg": 1, "pass": 2, "tile16": 3, "tile64": 4, "dqlds": 5}
    dts = {"f16": torch.float16, "bf16": torch.bfloat16}
    worst = 0.0
    for l in lines:
        c = dict(zip(header, [v.strip() for v in l.strip().strip("|").split("|")]))
        dt, bits, gs, _ = c["shape"].split("-")
        N, K = (int(v) for v in c["N x K"].split(" x "))
        M = int(c["M"])
        times = {k: float(c[k]) for k in names if c.get(k, "-") != "-"}
        sel = Q.kernel_name(Q.select_kernel(dts[dt], int(bits[:-1]), int(gs[2:]), M, N, K)).replace(
            "mfma_splitfree_", "")
        worst = max(worst, times[sel] / min(times.values()))
        assert times[sel] <= 1.05 * min(times.values()), (c["shape"], M, sel, times)
    assert worst <= 1.05


def test_split_plan_and_workspace_bytes():
    """The K-split plan of qmm_small_m_ws (crossovers measured with sweep.py
    --splits): the register kernel on the fewest K slices it covers where it
    cannot take K whole (4-bit); else the 64-column tile kernel split
    min(4, 256 / tiles) ways when N gives 32..64 such tiles and M >= 24;
    otherwise no split and no workspace (exactly qmm_small_m)."""
    import torch
    f16, bf16 = torch.float16, torch.bfloat16
    # down projection 4096 x 14336, 4-bit: the register kernel on 7 K slices (row blocks above 16 rows)
    for M in (24, 32, 36, 48, 64):
        assert Q.split_plan(f16, 4, 64, M, 4096, 14336) == (Q.KERNEL_MFMA_REG, 7)
        assert Q.workspace_bytes(f16, 4, 64, M, 4096, 14336) == 7 * M * 4096 * 4
    # 8-bit (no register split): 64 tiles of 64 columns -> 4 splits of 56 passes, from M = 24
    for M in (24, 32, 36, 48, 64):
        assert Q.split_plan(f16, 8, 64, M, 4096, 14336) == (Q.KERNEL_MFMA_TILE64, 4)
        assert Q.workspace_bytes(f16, 8, 64, M, 4096, 14336) == 4 * M * 4096 * 4
    # K = N = 4096: the register kernel on row blocks is faster than any split (no workspace),
    # except its single-tile row blocks above 48 rows (6/8-bit): the 64-column tile kernel
    # split 4 ways
    assert Q.split_plan(f16, 4, 64, 48, 4096, 4096) == (Q.KERNEL_MFMA_REG, 1)
    assert Q.split_plan(f16, 4, 64, 64, 4096, 4096) == (Q.KERNEL_MFMA_REG, 1)
    for M in (24, 36, 48):
        assert Q.split_plan(f16, 8, 64, M, 4096, 4096) == (Q.KERNEL_MFMA_REG, 1)
        assert Q.split_plan(bf16, 6, 128, M, 4096, 4096) == (Q.KERNEL_MFMA_REG, 1)
    for M in (49, 64):
        assert Q.split_plan(f16, 8, 64, M, 4096, 4096) == (Q.KERNEL_MFMA_TILE64, 4)
        assert Q.split_plan(bf16, 6, 128, M, 4096, 4096) == (Q.KERNEL_MFMA_TILE64, 4)
    # N = 2048: 32 tiles -> 4 splits (capped); 4-bit takes the register split
    assert Q.split_plan(f16, 8, 64, 64, 2048, 14336) == (Q.KERNEL_MFMA_TILE64, 4)
    assert Q.split_plan(f16, 4, 64, 64, 2048, 14336) == (Q.KERNEL_MFMA_REG, 7)
    # M <= 16 on K the register kernel takes only split: 7 slices of 2048 (down), 2 of 4096 (K = 8192)
    for M in (1, 8, 16):
        assert Q.split_plan(f16, 4, 64, M, 4096, 14336) == (Q.KERNEL_MFMA_REG, 7)
        assert Q.workspace_bytes(f16, 4, 64, M, 4096, 14336) == 7 * M * 4096 * 4
    assert Q.split_plan(bf16, 4, 32, 8, 4096, 8192) == (Q.KERNEL_MFMA_REG, 2)
    # no split: small M, few tiles (k/v), many tiles (gate/up, LM head), K the tile kernels do not take
    for args in ((f16, 8, 64, 16, 4096, 14336), (f16, 4, 64, 36, 4096, 4096), (f16, 4, 64, 64, 1024, 4096),
                 (f16, 4, 64, 64, 14336, 4096), (bf16, 4, 64, 64, 151936, 4096), (f16, 4, 64, 64, 4096, 14400),
                 (f16, 4, 64, 6, 4096, 4096)):
        k, s = Q.split_plan(*args)
        assert s == 1 and k == Q.select_kernel(*args) and Q.workspace_bytes(*args) == 0, args
    assert Q.qmm_small_m_workspace_bytes(0, 4, 64, 65, 4096, 4096) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_small_m_workspace_bytes(0, 4, 64, -1, 4096, 4096) == Q.QMM_ERR_INVALID_ARG


def test_split_entry_validation():
    """Errors of the workspace entry points are returned before any HIP call
    (fake addresses, no GPU)."""
    f16 = Q.QMM_F16
    base = (f16, 4, 64, 32, 4096, 14336, A, A, A, A, A)
    need = 7 * 32 * 4096 * 4  # the plan: the register kernel on 7 K slices
    assert Q.qmm_small_m_workspace_bytes(f16, 4, 64, 32, 4096, 14336) == need
    # workspace too small, missing, or misaligned
    assert Q.qmm_small_m_ws(*base, A, need - 4, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_small_m_ws(*base, None, need, None) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_small_m_ws(*base, MIS, need, None) == Q.QMM_ERR_MISALIGNED
    assert Q.qmm_small_m_ws(*base, A, -1, None) == Q.QMM_ERR_INVALID_ARG
    # forced: split < 1, a split on a kernel that cannot split, a kernel that cannot run the shape
    assert Q.qmm_small_m_split_forced(*base, A, need, None, Q.KERNEL_MFMA_TILE64, 0) == Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_small_m_split_forced(*base, A, need, None, Q.KERNEL_MFMA_PASS, 2) == Q.QMM_ERR_UNSUPPORTED
    assert Q.qmm_small_m_split_forced(*base, A, need, None, Q.KERNEL_MFMA_REG, 1) == Q.QMM_ERR_UNSUPPORTED
    # the register kernel splits K exactly: 14336 = 7 slices of 2048 (not 2 of 7168), M <= 16 only
    small = (f16, 4, 64, 8, 4096, 14336, A, A, A, A, A)
    assert Q.qmm_small_m_split_forced(*small, A, 7 * 8 * 4096 * 4, None, Q.KERNEL_MFMA_REG, 2) == \
        Q.QMM_ERR_UNSUPPORTED
    # (above 16 rows on row blocks too: 7 slices need 7 partial outputs, more than 4 hold)
    assert Q.qmm_small_m_split_forced(*base, A, 4 * 32 * 4096 * 4, None, Q.KERNEL_MFMA_REG, 7) == \
        Q.QMM_ERR_INVALID_ARG
    assert Q.qmm_small_m_split_forced(*small, A, 7 * 8 * 4096 * 4 - 4, None, Q.KERNEL_MFMA_REG, 7) == \
        Q.QMM_ERR_INVALID_ARG
    # the workspace a forced split needs is the reduced split's: 28 passes, split 5 -> 6 passes each -> 5 splits
    assert Q.qmm_small_m_split_forced(*base, A, 5 * 32 * 4096 * 4 - 4, None, Q.KERNEL_MFMA_TILE16, 5) == \
        Q.QMM_ERR_INVALID_ARG
    # empty problems: OK, nothing launched
    assert Q.qmm_small_m_ws(f16, 4, 64, 0, 4096, 14336, None, None, None, None, None, None, 0, None) == Q.QMM_OK


def test_batched_validation():
    """qmm_small_m_batched: errors before any HIP call (fake addresses, no GPU)."""
    bm = Q.qmm_small_m_batched
    ok = (0, 4, 64, 3, 4, 64, 256)  # dt, bits, gs, batch, M, N, K
    ptrs = (A, A, A, A, A, None)
    assert bm(0, 4, 64, -1, 4, 64, 256, *ptrs) == Q.QMM_ERR_INVALID_ARG
    assert bm(0, 4, 64, 2, -1, 64, 256, *ptrs) == Q.QMM_ERR_INVALID_ARG
    assert bm(0, 5, 64, 2, 4, 64, 256, *ptrs) == Q.QMM_ERR_UNSUPPORTED
    assert bm(0, 4, 64, 2, 65, 64, 256, *ptrs) == Q.QMM_ERR_UNSUPPORTED
    assert bm(*ok, None, A, A, A, A, None) == Q.QMM_ERR_INVALID_ARG
    assert bm(*ok, A, A, A, A, MIS, None) == Q.QMM_ERR_MISALIGNED
    # entries that would not start 16-byte aligned: y of one entry is 3 x 17 x 2 bytes
    assert bm(0, 4, 64, 2, 3, 17, 256, *ptrs) == Q.QMM_ERR_MISALIGNED
    # scale rows of one entry: 17 rows x 3 groups x 2 bytes
    assert bm(0, 4, 64, 2, 8, 17, 192, *ptrs) == Q.QMM_ERR_MISALIGNED
    # ... which a single entry does not need
    assert bm(0, 4, 64, 1, 3, 17, 256, None, A, A, A, A, None) == Q.QMM_ERR_INVALID_ARG
    # empty problems: OK with nothing launched, NULL allowed
    assert bm(0, 4, 64, 0, 4, 64, 256, None, None, None, None, None, None) == Q.QMM_OK
    assert bm(0, 4, 64, 3, 0, 64, 256, None, None, None, None, None, None) == Q.QMM_OK
    assert bm(1, 8, 32, 3, 4, 0, 256, None, None, None, None, None, None) == Q.QMM_OK
    # byte offsets that overflow int64
    assert bm(0, 8, 32, 2 ** 62, 64, 4096, 4096, *ptrs) == Q.QMM_ERR_INVALID_ARG


def test_nt_validation():
    """qmm_small_m_nt: N follows the rules of the quantized axis, K a positive
    multiple of 32; errors before any HIP call."""
    nt = Q.qmm_small_m_nt
    ptrs = (A, A, A, A, A, None)
    assert nt(0, 4, 64, -1, 256, 64, *ptrs) == Q.QMM_ERR_INVALID_ARG
    assert nt(0, 4, 64, 4, 256, -32, *ptrs) == Q.QMM_ERR_INVALID_ARG
    assert nt(0, 4, 64, 4, 96, 64, *ptrs) == Q.QMM_ERR_UNSUPPORTED      # N % 64
    assert nt(0, 4, 128, 4, 192, 64, *ptrs) == Q.QMM_ERR_UNSUPPORTED    # N % gs
    assert nt(0, 4, 64, 4, 256, 48, *ptrs) == Q.QMM_ERR_UNSUPPORTED     # K % 32
    assert nt(0, 4, 64, 4, 256, 0, *ptrs) == Q.QMM_ERR_UNSUPPORTED
    assert nt(0, 4, 64, 65, 256, 64, *ptrs) == Q.QMM_ERR_UNSUPPORTED
    assert nt(0, 5, 64, 4, 256, 64, *ptrs) == Q.QMM_ERR_UNSUPPORTED
    assert nt(0, 4, 64, 4, 256, 64, A, None, A, A, A, None) == Q.QMM_ERR_INVALID_ARG
    assert nt(0, 4, 64, 4, 256, 64, A, A, A, MIS, A, None) == Q.QMM_ERR_MISALIGNED
    assert nt(1, 6, 32, 0, 256, 64, None, None, None, None, None, None) == Q.QMM_OK


def test_nt_split_plan_and_validation():
    """qmm_small_m_nt_ws: column blocks with K slices.  4/8-bit with N >=
    4096 (the transpose-read form, 256-column blocks): the fewest slices of
    whole 16 KiB chunks (128 rows at 4 bits, 64 at 8) dividing K for
    224..512 workgroups, else whole chunks for at least 224, unsplit from 256
    blocks; otherwise
    (6-bit, or N below 4096) the 16-wavefront form with 128-column blocks:
    about 256 workgroups, at most 16 slices, unsplit from 128 blocks;
    unsplit when K is short; errors before any HIP call."""
    f16, bf16 = Q.QMM_F16, Q.QMM_BF16
    wb = Q.qmm_small_m_nt_workspace_bytes
    assert wb(f16, 4, 64, 6, 4096, 4096) == 16 * 6 * 4096 * 4      # 16 blocks x 16 slices of 256 rows (transpose reads)
    assert wb(bf16, 8, 32, 6, 4096, 4096) == 16 * 6 * 4096 * 4
    assert wb(f16, 6, 64, 6, 4096, 4096) == 8 * 6 * 4096 * 4       # 6-bit: 32 x 8 slices
    assert wb(f16, 4, 64, 6, 1024, 4096) == 16 * 6 * 1024 * 4      # 8 blocks: the 16-wavefront form, 16 slices
    assert wb(f16, 4, 64, 4, 4096, 14336) == 14 * 4 * 4096 * 4     # 16 x 14 slices of 1024 rows (8 chunks)
    assert wb(f16, 4, 64, 6, 14336, 4096) == 4 * 6 * 14336 * 4     # 56 blocks x 4 slices of 1024 rows
    assert wb(bf16, 8, 64, 6, 4096, 4160) == 17 * 6 * 4096 * 4     # no divisor fits: 16 x 17 slices of 256 rows (the last 64)
    assert wb(f16, 4, 64, 6, 32768, 4096) == 2 * 6 * 32768 * 4     # 128 blocks x 2 slices
    assert wb(f16, 4, 64, 64, 1024, 4160) == 15 * 64 * 1024 * 4    # slices of 288 rows, the last shorter
    assert wb(f16, 6, 64, 6, 16384, 4096) == 0                     # 6-bit, 128 blocks: unsplit
    assert wb(f16, 4, 64, 6, 65536, 4096) == 0                     # 256 blocks: unsplit
    assert wb(f16, 4, 64, 6, 256, 96) == 0                         # one slice of K
    assert wb(f16, 4, 64, -1, 256, 96) == Q.QMM_ERR_INVALID_ARG
    assert wb(f16, 4, 64, 6, 96, 96) == Q.QMM_ERR_UNSUPPORTED
    ws = Q.qmm_small_m_nt_ws
    base = (f16, 4, 64, 6, 4096, 4096, A, A, A, A, A)
    need = 16 * 6 * 4096 * 4
    assert ws(*base, A, need - 4, None) == Q.QMM_ERR_INVALID_ARG
    assert ws(*base, None, need, None) == Q.QMM_ERR_INVALID_ARG
    assert ws(*base, MIS, need, None) == Q.QMM_ERR_MISALIGNED
    assert ws(*base, A, -1, None) == Q.QMM_ERR_INVALID_ARG
    assert ws(f16, 4, 64, 6, 4096, 4096, None, A, A, A, A, A, need, None) == Q.QMM_ERR_INVALID_ARG
    assert ws(f16, 4, 64, 0, 4096, 4096, None, None, None, None, None, None, 0, None) == Q.QMM_OK


def test_header_is_c99_and_links(tmp_path):
    """include/qmm.h is plain C (no torch, no C++): a C99 program compiles
    against it with warnings as errors, links libqmm.so and gets the same
    answers from the host-only entry points as the binding."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_qmm.c"
    src.write_text(r'''
#include "qmm.h"
#include <stdio.h>
int main(void) {
    int k = -1, s = -1;
    if (qmm_packed_words(4, 4096) != 512 || qmm_packed_words(6, 4096) != 768) return 1;
    if (qmm_select_kernel(QMM_F16, 4, 64, 6, 4096, 4096) != QMM_KERNEL_MFMA_REG) return 2;
    if (qmm_small_m(QMM_F16, 5, 64, 4, 64, 256, 0, 0, 0, 0, 0, 0) != QMM_ERR_UNSUPPORTED) return 3;
    if (qmm_split_plan(QMM_F16, 4, 64, 8, 4096, 14336, &k, &s) != QMM_OK || k != QMM_KERNEL_MFMA_REG || s != 7) return 4;
    if (qmm_small_m_nt_workspace_bytes(QMM_F16, 4, 64, 6, 4096, 4096) != 16LL * 6 * 4096 * 4) return 5;
    if (qmm_small_m_batched(QMM_F16, 4, 64, 0, 4, 64, 256, 0, 0, 0, 0, 0, 0) != QMM_OK) return 6;
    printf("%s\n", qmm_kernel_name(QMM_KERNEL_MFMA_REG));
    return 0;
}
''')
    exe = tmp_path / "use_qmm"
    libdir = os.path.dirname(Q.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    str(src), "-L", libdir, "-lqmm", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stderr)
    assert r.stdout.strip() == Q.kernel_name(Q.KERNEL_MFMA_REG)


def test_noalloc_validation():
    """qmm_small_m_noalloc rejects bad arguments and problems whose planned
    workspace exceeds its static scratch before any HIP call."""
    K = 14336

    def na(dt=0, bits=4, gs=64, M=16, N=4096, x=A, wq=A, s=A, b=A, y=A):
        return Q.qmm_small_m_noalloc(dt, bits, gs, M, N, K, x, wq, s, b, y, None)

    assert Q.NOALLOC_SCRATCH_BYTES == 8 * 1024 * 1024
    assert na(M=-1) == Q.QMM_ERR_INVALID_ARG
    assert na(bits=5) == Q.QMM_ERR_UNSUPPORTED
    assert na(M=65) == Q.QMM_ERR_UNSUPPORTED
    assert na(M=0, x=None, y=None) == Q.QMM_OK
    assert na(N=0, x=None, y=None) == Q.QMM_OK
    # planned workspace above the scratch: refused
    big = Q.qmm_small_m_workspace_bytes(0, 4, 64, 16, 32768, K)
    assert big > Q.NOALLOC_SCRATCH_BYTES
    assert na(N=32768) == Q.QMM_ERR_UNSUPPORTED
    # within it, but bad pointers
    assert 0 < Q.qmm_small_m_workspace_bytes(0, 4, 64, 16, 4096, K) <= Q.NOALLOC_SCRATCH_BYTES
    assert na(x=None) == Q.QMM_ERR_INVALID_ARG
    assert na(y=MIS) == Q.QMM_ERR_MISALIGNED


def test_empty_problem_plans():
    """Workspace size and split plan of an empty problem (M = 0 or N = 0):
    no split, no workspace (the plan's per-row-block arithmetic is never
    reached with zero rows)."""
    for M, N in ((0, 4096), (4, 0), (0, 0)):
        assert Q.qmm_small_m_workspace_bytes(0, 4, 64, M, N, 14336) == 0
        kid, split = ctypes.c_int(-1), ctypes.c_int(-1)
        assert Q._lib.qmm_split_plan(0, 4, 64, M, N, 14336, ctypes.byref(kid), ctypes.byref(split)) == Q.QMM_OK
        assert split.value == 1

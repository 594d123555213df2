"""Python binding of libqmm (affine group-quantized small-M matmul, MI355X).

Argument marshalling only: every step runs in the HIP kernels of
``libqmm.so``; PyTorch supplies device memory and the current stream.  The
C entry points are exposed under their C names (``qmm_quantize``,
``qmm_dequantize``, ``qmm_small_m``, ...) taking integer addresses, and
tensor-level helpers (:func:`quantize`, :func:`dequantize`, :func:`small_m`)
mirror the MLX-style API the pages use: ``quantize(w, group_size, bits) ->
(wq, scales, biases)`` and ``quantized_matmul(x, wq, scales, biases,
transpose=True, ...)`` (MLX issue #4720, "To Reproduce").
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqmm.so")

QMM_F16, QMM_BF16 = 0, 1
QMM_OK, QMM_ERR_INVALID_ARG, QMM_ERR_UNSUPPORTED, QMM_ERR_MISALIGNED, QMM_ERR_HIP = 0, -1, -2, -3, -4
KERNEL_VALU, KERNEL_MFMA_REG, KERNEL_MFMA_PASS, KERNEL_MFMA_TILE16, KERNEL_MFMA_TILE64 = 0, 1, 2, 3, 4
KERNEL_MFMA_DQLDS = 5
KERNEL_IDS = (KERNEL_VALU, KERNEL_MFMA_REG, KERNEL_MFMA_PASS, KERNEL_MFMA_TILE16, KERNEL_MFMA_TILE64,
              KERNEL_MFMA_DQLDS)

_DT = {torch.float16: QMM_F16, torch.bfloat16: QMM_BF16}

EXPORTS = (
    "qmm_quantize", "qmm_dequantize", "qmm_small_m", "qmm_small_m_forced",
    "qmm_select_kernel", "qmm_kernel_supported", "qmm_packed_words", "qmm_strerror", "qmm_kernel_name",
    "qmm_probe_stream_read", "qmm_probe_copy",
    "qmm_small_m_ws", "qmm_small_m_workspace_bytes", "qmm_small_m_split_forced", "qmm_split_plan",
    "qmm_small_m_batched", "qmm_small_m_nt", "qmm_small_m_nt_ws", "qmm_small_m_nt_workspace_bytes",
    "qmm_build_digest", "qmm_small_m_noalloc", "qmm_probe_small_m_loop",
)
NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024  # QMM_NOALLOC_SCRATCH_BYTES


class QmmError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} (status {status})")
        self.status = status


class StaleLibraryError(ImportError):
    """libqmm.so was built from other sources than the ones beside it."""


def _load():
    from . import build as _b
    if not os.path.exists(LIB_PATH):
        _b.build(verbose=False)
    lib = ctypes.CDLL(LIB_PATH)
    lib.qmm_build_digest.restype = ctypes.c_char_p
    lib.qmm_build_digest.argtypes = []
    built, current = lib.qmm_build_digest().decode(), _b.source_digest()
    if built != current:
        raise StaleLibraryError(
            f"{LIB_PATH} was built from sources with digest {built}, but the sources beside it have digest "
            f"{current}: rebuild it (python affine_quantized_gemm_amd/build.py)")
    i32, i64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p
    sig = {
        "qmm_quantize": (i32, [i32, i32, i32, i64, i64, vp, vp, vp, vp, vp]),
        "qmm_dequantize": (i32, [i32, i32, i32, i64, i64, vp, vp, vp, vp, vp]),
        "qmm_small_m": (i32, [i32, i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp]),
        "qmm_small_m_forced": (i32, [i32, i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, i32]),
        "qmm_select_kernel": (i32, [i32, i32, i32, i64, i64, i64]),
        "qmm_kernel_supported": (i32, [i32, i32, i32, i64, i64, i64, i32]),
        "qmm_packed_words": (i64, [i32, i64]),
        "qmm_strerror": (ctypes.c_char_p, [i32]),
        "qmm_kernel_name": (ctypes.c_char_p, [i32]),
        "qmm_probe_stream_read": (i32, [vp, i64, vp, i32, i32, vp]),
        "qmm_probe_copy": (i32, [vp, vp, i64, vp]),
        "qmm_small_m_ws": (i32, [i32, i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, i64, vp]),
        "qmm_small_m_workspace_bytes": (i64, [i32, i32, i32, i64, i64, i64]),
        "qmm_small_m_split_forced": (i32, [i32, i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, i64, vp,
                                           i32, i32]),
        "qmm_split_plan": (i32, [i32, i32, i32, i64, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
        "qmm_small_m_batched": (i32, [i32, i32, i32, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]),
        "qmm_small_m_nt": (i32, [i32, i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp]),
        "qmm_small_m_nt_ws": (i32, [i32, i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp, i64, vp]),
        "qmm_small_m_nt_workspace_bytes": (i64, [i32, i32, i32, i64, i64, i64]),
        "qmm_build_digest": (ctypes.c_char_p, []),
        "qmm_small_m_noalloc": (i32, [i32, i32, i32, i64, i64, i64, vp, vp, vp, vp, vp, vp]),
        "qmm_probe_small_m_loop": (i32, [i32, i32, i32, i64, i64, i64, vp, ctypes.POINTER(vp), ctypes.POINTER(vp),
                                         ctypes.POINTER(vp), vp, i32, i32, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
BUILD_DIGEST = _lib.qmm_build_digest().decode()

# ---- C entry points under their C names (integer addresses, status codes) ----
qmm_quantize = _lib.qmm_quantize
qmm_dequantize = _lib.qmm_dequantize
qmm_small_m = _lib.qmm_small_m
qmm_small_m_forced = _lib.qmm_small_m_forced
qmm_select_kernel = _lib.qmm_select_kernel
qmm_packed_words = _lib.qmm_packed_words
qmm_kernel_supported = _lib.qmm_kernel_supported
qmm_probe_stream_read = _lib.qmm_probe_stream_read
qmm_probe_copy = _lib.qmm_probe_copy
qmm_small_m_ws = _lib.qmm_small_m_ws
qmm_small_m_workspace_bytes = _lib.qmm_small_m_workspace_bytes
qmm_small_m_split_forced = _lib.qmm_small_m_split_forced
qmm_split_plan = _lib.qmm_split_plan
qmm_small_m_batched = _lib.qmm_small_m_batched
qmm_small_m_nt = _lib.qmm_small_m_nt
qmm_small_m_nt_ws = _lib.qmm_small_m_nt_ws
qmm_small_m_nt_workspace_bytes = _lib.qmm_small_m_nt_workspace_bytes
qmm_small_m_noalloc = _lib.qmm_small_m_noalloc
qmm_probe_small_m_loop = _lib.qmm_probe_small_m_loop


def strerror(status: int) -> str:
    return _lib.qmm_strerror(int(status)).decode()


def kernel_name(kernel_id: int) -> str:
    return _lib.qmm_kernel_name(int(kernel_id)).decode()


def packed_words(bits: int, K: int) -> int:
    return int(_lib.qmm_packed_words(int(bits), int(K)))


def select_kernel(dtype, bits: int, group_size: int, M: int, N: int, K: int) -> int:
    return int(_lib.qmm_select_kernel(_dt(dtype), bits, group_size, M, N, K))


def kernel_supported(dtype, bits: int, group_size: int, M: int, N: int, K: int, kernel: int) -> bool:
    return int(_lib.qmm_kernel_supported(_dt(dtype), bits, group_size, M, N, K, int(kernel))) == 1


# ---- tensor helpers ----

def _dt(dtype) -> int:
    if dtype not in _DT:
        raise QmmError(QMM_ERR_UNSUPPORTED, f"dtype {dtype}")
    return _DT[dtype]


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(status: int, what: str):
    if status != QMM_OK:
        raise QmmError(status, what)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_WORD_DTYPES = tuple(d for d in (torch.int32, getattr(torch, "uint32", None)) if d is not None)


def _expect(t: torch.Tensor, name: str, shape: tuple, dtypes) -> None:
    """Shape and dtype of an operand against the problem size (checked before
    any pointer reaches the library: a wrong bits, group size or buffer would
    otherwise make the kernels read or write past the tensors)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(v) for v in shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")


def _words(bits: int, n: int) -> int:
    """uint32 words per packed row of n codes (QmmError if unsupported)."""
    w = packed_words(bits, n)
    if w < 0:
        raise QmmError(QMM_ERR_UNSUPPORTED, f"bits={bits} with {n} codes per row")
    return w


def _groups(group_size: int, n: int) -> int:
    if group_size not in (32, 64, 128) or n % group_size:
        raise QmmError(QMM_ERR_UNSUPPORTED, f"group_size={group_size} with {n} codes per row")
    return n // group_size


def _same_device(ref: torch.Tensor, *named):
    for t, n in named:
        if t.device != ref.device:
            raise ValueError(f"{n} is on {t.device}, expected {ref.device}")


def _check_quantized(x_dtype, wq, scales, biases, rows: int, n: int, bits: int, group_size: int,
                     lead: tuple = ()):
    """wq [*lead, rows, words(n)], scales / biases [*lead, rows, n/gs] in x's dtype."""
    _expect(wq, "wq", (*lead, rows, _words(bits, n)), _WORD_DTYPES)
    g = _groups(group_size, n)
    _expect(scales, "scales", (*lead, rows, g), (x_dtype,))
    _expect(biases, "biases", (*lead, rows, g), (x_dtype,))


def quantize(w: torch.Tensor, bits: int, group_size: int, stream=None):
    """W [N, K] (fp16/bf16, GPU) -> (wq [N, K*bits/32] int32 words, scales, biases)."""
    if w.dim() != 2:
        raise ValueError(f"w must be 2-D [N, K], got shape {tuple(w.shape)}")
    _dt(w.dtype)
    N, K = w.shape
    nw = _words(bits, K)
    _groups(group_size, K)
    _dev(w, "w")
    wq = torch.empty((N, nw), dtype=torch.int32, device=w.device)
    sc = torch.empty((N, K // group_size), dtype=w.dtype, device=w.device)
    bi = torch.empty_like(sc)
    _check(qmm_quantize(_dt(w.dtype), bits, group_size, N, K, w.data_ptr(), wq.data_ptr(),
                        sc.data_ptr(), bi.data_ptr(), _stream(stream)), "qmm_quantize")
    return wq, sc, bi


def dequantize(wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int, group_size: int,
               stream=None) -> torch.Tensor:
    """(wq, scales, biases) -> W_hat [N, K] in the scales' dtype."""
    if scales.dim() != 2:
        raise ValueError(f"scales must be 2-D [N, K/gs], got shape {tuple(scales.shape)}")
    _dt(scales.dtype)
    N = scales.shape[0]
    K = scales.shape[1] * group_size
    _check_quantized(scales.dtype, wq, scales, biases, N, K, bits, group_size)
    for t, n in ((wq, "wq"), (scales, "scales"), (biases, "biases")):
        _dev(t, n)
    _same_device(wq, (scales, "scales"), (biases, "biases"))
    out = torch.empty((N, K), dtype=scales.dtype, device=wq.device)
    _check(qmm_dequantize(_dt(scales.dtype), bits, group_size, N, K, wq.data_ptr(), scales.data_ptr(),
                          biases.data_ptr(), out.data_ptr(), _stream(stream)), "qmm_dequantize")
    return out


def probe_stream_read(src: torch.Tensor, sink: torch.Tensor, grid: int = 0, shape: int = 1, stream=None):
    """Stream ``src`` (whole tensor) through a read-only kernel (measurement
    helper); shape 0: grid-stride loop, 1: 8 KiB chunks per wavefront."""
    _dev(src, "src")
    _dev(sink, "sink")
    if sink.numel() * sink.element_size() < 1024:
        raise ValueError("sink must hold 256 uint32")
    _check(qmm_probe_stream_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), grid, shape,
                                 _stream(stream)), "qmm_probe_stream_read")


def probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """dst <- src byte for byte (measurement helper; equal byte sizes)."""
    _dev(src, "src")
    _dev(dst, "dst")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst differ in size")
    _check(qmm_probe_copy(src.data_ptr(), dst.data_ptr(), nb, _stream(stream)), "qmm_probe_copy")


def small_m_loop_args(x: torch.Tensor, stack, bits: int, group_size: int, out: torch.Tensor) -> tuple:
    """Validated leading arguments of qmm_probe_small_m_loop for ``stack`` (a
    non-empty list of (wq, scales, biases)) with x and ``out``: the C call
    then takes ``(*args, passes, stream)``.  The tensors must stay alive
    while the tuple is used."""
    if not stack:
        raise ValueError("empty stack")
    for (wq, scales, biases) in stack:
        _check_small_m(x, wq, scales, biases, bits, group_size, out)
    n = len(stack)
    arr = ctypes.c_void_p * n
    wqs = arr(*[t[0].data_ptr() for t in stack])
    scs = arr(*[t[1].data_ptr() for t in stack])
    bis = arr(*[t[2].data_ptr() for t in stack])
    M, K = x.shape
    N = stack[0][0].shape[0]
    return (_dt(x.dtype), bits, group_size, M, N, K, x.data_ptr(), wqs, scs, bis, out.data_ptr(), n)


def probe_small_m_loop(x: torch.Tensor, stack, bits: int, group_size: int, out: torch.Tensor, passes: int = 1,
                       stream=None):
    """``passes`` times over ``stack`` (a list of (wq, scales, biases)), one
    qmm_small_m call per weight set into ``out``, issued from a C loop
    (measurement helper: the stream-launched rate without Python between
    the calls; ``small_m_loop_args`` validates once for repeated calls)."""
    if not stack:
        return
    _check(qmm_probe_small_m_loop(*small_m_loop_args(x, stack, bits, group_size, out), passes, _stream(stream)),
           "qmm_probe_small_m_loop")


def _check_small_m(x, wq, scales, biases, bits, group_size, out):
    """Shapes, dtypes and devices of a transposed product; returns (M, K, N)."""
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [M, K], got shape {tuple(x.shape)}")
    _dt(x.dtype)
    if wq.dim() != 2:
        raise ValueError(f"wq must be 2-D [N, K*bits/32], got shape {tuple(wq.shape)}")
    M, K = x.shape
    N = wq.shape[0]
    _check_quantized(x.dtype, wq, scales, biases, N, K, bits, group_size)
    if out is not None:
        _expect(out, "out", (M, N), (x.dtype,))
    for t, n in ((x, "x"), (wq, "wq"), (scales, "scales"), (biases, "biases")):
        _dev(t, n)
    _same_device(x, (wq, "wq"), (scales, "scales"), (biases, "biases"))
    if out is not None:
        _dev(out, "out")
        _same_device(x, (out, "out"))
    return M, K, N


def small_m(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int,
            group_size: int, out: torch.Tensor | None = None, kernel: int | None = None,
            stream=None) -> torch.Tensor:
    """y [M, N] = x [M, K] . dequant(wq, scales, biases)^T (``kernel`` forces a variant)."""
    M, K, N = _check_small_m(x, wq, scales, biases, bits, group_size, out)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    args = (_dt(x.dtype), bits, group_size, M, N, K, x.data_ptr(), wq.data_ptr(), scales.data_ptr(),
            biases.data_ptr(), out.data_ptr(), _stream(stream))
    if kernel is None:
        _check(qmm_small_m(*args), "qmm_small_m")
    else:
        _check(qmm_small_m_forced(*args, int(kernel)), "qmm_small_m_forced")
    return out


def small_m_batched(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int,
                    group_size: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y [B, M, N]: y[b] = x[b] . dequant(wq[b], scales[b], biases[b])^T, one weight set per entry
    (x [B, M, K], wq [B, N, words], scales / biases [B, N, K/gs])."""
    if x.dim() != 3:
        raise ValueError(f"x must be 3-D [B, M, K], got shape {tuple(x.shape)}")
    _dt(x.dtype)
    if wq.dim() != 3:
        raise ValueError(f"wq must be 3-D [B, N, K*bits/32], got shape {tuple(wq.shape)}")
    B, M, K = x.shape
    N = wq.shape[1]
    _check_quantized(x.dtype, wq, scales, biases, N, K, bits, group_size, lead=(B,))
    if out is not None:
        _expect(out, "out", (B, M, N), (x.dtype,))
    for t, n in ((x, "x"), (wq, "wq"), (scales, "scales"), (biases, "biases")):
        _dev(t, n)
    _same_device(x, (wq, "wq"), (scales, "scales"), (biases, "biases"))
    if out is None:
        out = torch.empty((B, M, N), dtype=x.dtype, device=x.device)
    else:
        _dev(out, "out")
        _same_device(x, (out, "out"))
    _check(qmm_small_m_batched(_dt(x.dtype), bits, group_size, B, M, N, K, x.data_ptr(), wq.data_ptr(),
                               scales.data_ptr(), biases.data_ptr(), out.data_ptr(), _stream(stream)),
           "qmm_small_m_batched")
    return out


def nt_workspace_bytes(dtype, bits: int, group_size: int, M: int, N: int, K: int) -> int:
    """Bytes of workspace :func:`small_m_nt` with ``split=True`` needs (0: it runs unsplit)."""
    r = int(_lib.qmm_small_m_nt_workspace_bytes(_dt(dtype), bits, group_size, M, N, K))
    if r < 0:
        raise QmmError(r, "qmm_small_m_nt_workspace_bytes")
    return r


def small_m_nt(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int,
               group_size: int, out: torch.Tensor | None = None, stream=None, split: bool = False,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y [M, N] = x [M, K] . dequant(W) for W stored [K, N] and quantized along N
    (wq [K, N*bits/32], scales / biases [K, N/gs]: :func:`quantize` of a [K, N] matrix)."""
    if x.dim() != 2:
        raise ValueError(f"x must be 2-D [M, K], got shape {tuple(x.shape)}")
    _dt(x.dtype)
    if wq.dim() != 2:
        raise ValueError(f"wq must be 2-D [K, N*bits/32], got shape {tuple(wq.shape)}")
    if bits not in (4, 6, 8):
        raise QmmError(QMM_ERR_UNSUPPORTED, f"bits={bits}")
    M, K = x.shape
    N = wq.shape[1] * 32 // bits
    _check_quantized(x.dtype, wq, scales, biases, K, N, bits, group_size)
    if out is not None:
        _expect(out, "out", (M, N), (x.dtype,))
    for t, n in ((x, "x"), (wq, "wq"), (scales, "scales"), (biases, "biases")):
        _dev(t, n)
    _same_device(x, (wq, "wq"), (scales, "scales"), (biases, "biases"))
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    else:
        _dev(out, "out")
        _same_device(x, (out, "out"))
    args = (_dt(x.dtype), bits, group_size, M, N, K, x.data_ptr(), wq.data_ptr(), scales.data_ptr(),
            biases.data_ptr(), out.data_ptr())
    if not split:
        _check(qmm_small_m_nt(*args, _stream(stream)), "qmm_small_m_nt")
        return out
    # K split (workspace entry point): a workspace of the planned size unless given
    need = nt_workspace_bytes(x.dtype, bits, group_size, M, N, K)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(qmm_small_m_nt_ws(*args, ws_ptr, ws_bytes, _stream(stream)), "qmm_small_m_nt_ws")
    return out


def workspace_bytes(dtype, bits: int, group_size: int, M: int, N: int, K: int) -> int:
    """Bytes of workspace :func:`small_m_ws` needs (0: it runs split-free)."""
    r = int(_lib.qmm_small_m_workspace_bytes(_dt(dtype), bits, group_size, M, N, K))
    if r < 0:
        raise QmmError(r, "qmm_small_m_workspace_bytes")
    return r


def split_plan(dtype, bits: int, group_size: int, M: int, N: int, K: int) -> tuple[int, int]:
    """(kernel id, K split) that :func:`small_m_ws` uses."""
    k, s = ctypes.c_int(0), ctypes.c_int(0)
    _check(_lib.qmm_split_plan(_dt(dtype), bits, group_size, M, N, K, ctypes.byref(k), ctypes.byref(s)),
           "qmm_split_plan")
    return k.value, s.value


def small_m_ws(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int,
               group_size: int, workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
               kernel: int | None = None, split: int | None = None, stream=None) -> torch.Tensor:
    """As :func:`small_m`, K possibly split across workgroups with fp32 partial
    outputs in ``workspace`` (a device tensor the caller keeps; allocated here
    when not given).  ``kernel`` and ``split`` force the variant and split."""
    M, K, N = _check_small_m(x, wq, scales, biases, bits, group_size, out)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    if workspace is None:
        need = workspace_bytes(x.dtype, bits, group_size, M, N, K) if kernel is None else \
            max(1, int(split or 1)) * M * N * 4
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace")
    _same_device(x, (workspace, "workspace"))
    nb = workspace.numel() * workspace.element_size()
    args = (_dt(x.dtype), bits, group_size, M, N, K, x.data_ptr(), wq.data_ptr(), scales.data_ptr(),
            biases.data_ptr(), out.data_ptr(), workspace.data_ptr(), nb, _stream(stream))
    if kernel is None and split is None:
        _check(qmm_small_m_ws(*args), "qmm_small_m_ws")
    else:
        kid = kernel if kernel is not None else split_plan(x.dtype, bits, group_size, M, N, K)[0]
        _check(qmm_small_m_split_forced(*args, int(kid), int(split or 1)), "qmm_small_m_split_forced")
    return out


def small_m_noalloc(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int,
                    group_size: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """As :func:`small_m_ws` with its own plan, the K-split partials in the
    library's static per-GPU scratch instead of a workspace (the call itself
    allocates nothing when ``out`` is given).  Calls that overlap on one GPU
    race on that scratch."""
    M, K, N = _check_small_m(x, wq, scales, biases, bits, group_size, out)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check(qmm_small_m_noalloc(_dt(x.dtype), bits, group_size, M, N, K, x.data_ptr(), wq.data_ptr(),
                               scales.data_ptr(), biases.data_ptr(), out.data_ptr(), _stream(stream)),
           "qmm_small_m_noalloc")
    return out

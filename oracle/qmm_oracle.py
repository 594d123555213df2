"""Plain CPU oracle for affine group-quantized small-M matmul.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module: only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from the package.

What it computes (sources are the web pages this project is built from):

* Affine quantization of weights at 4, 6 or 8 bits with one fp16/bf16 scale
  and one bias per group of 32, 64 or 128 consecutive K elements, fp16/bf16
  activations -- "What Are NAX Verify Kernels and When Is the Turbo Profile
  Activated in MTPLX?", section "Supported Data Formats and Quantization
  Schemes".
* Separate ``scales`` and ``biases`` operands next to the packed ``w_q``
  words -- "How the NAX Verify Kernel Path Improves Decode Performance in
  MTPLX", section "Implementation and Configuration" (the usage example).
* The transposed product y = x . dequant(W)^T with W stored [N, K] -- MLX
  issue #4720, "To Reproduce" (``quantized_matmul(..., transpose=True)``).
* The batched form, one weight matrix per batch entry (the adjacent API
  case to the transposed, non-batched call of MLX issue #4720, "Describe the
  bug").
* The non-transposed product y = x . dequant(W) with W stored [K, N] and
  quantized along N (the other orientation of the same call).
* Weight bytes per call = packed words + 4 bytes of scale/bias per group --
  MLX issue #4720, "To Reproduce" (the ``wbytes`` expression).

The quantizer formula itself is not printed on the pages.  The reading used
here is min/max affine: scale = (max - min) / (2^bits - 1), bias = min,
q = round((w - bias) / scale) clamped to [0, 2^bits - 1].  Where the pages
are silent the choices are:

* the scale is computed in IEEE fp32 and stored in the activation dtype
  rounded toward +infinity, so that every element dequantizes to within
  half a step of its original value;
* q is fitted against the *stored* scale, with round-half-to-even;
* a constant group (max == min) stores scale 0 and q = 0, which dequantizes
  exactly to the bias;
* a group whose minimum is a zero stores the bias +0 (signed zeros compare
  equal, so the minimum's sign would otherwise depend on element order);
* packing is a little-endian bitstream per row: value k occupies bits
  [bits*k, bits*k + bits), stored as little-endian uint32 words (4-bit:
  8 values per word, low nibble first; 8-bit: 4 per word; 6-bit: 4 values
  per 24 bits, so 16 values per 3 words).

Dtype convention: fp16 arrays are ``np.float16``; bf16 arrays are
``np.uint16`` holding the bf16 bit patterns (numpy has no bf16 type).

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(closed-form words, hand-worked quantization examples, brute-force nearest
grid points, exact-rational matmuls, one-hot/ones/zero inputs).
"""

from __future__ import annotations

import numpy as np

F16 = "f16"
BF16 = "bf16"
DTYPES = (F16, BF16)
SUPPORTED_BITS = (4, 6, 8)
SUPPORTED_GROUP_SIZES = (32, 64, 128)


# ---------------------------------------------------------------------------
# dtype helpers (fp16 via numpy, bf16 via explicit bit manipulation)
# ---------------------------------------------------------------------------

def to_f32(a: np.ndarray, dt: str) -> np.ndarray:
    """Exact widening of fp16 values / bf16 bit patterns to fp32."""
    if dt == F16:
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    if dt == BF16:
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32)
    raise ValueError(dt)


def to_f64(a: np.ndarray, dt: str) -> np.ndarray:
    return to_f32(a, dt).astype(np.float64)


def f32_to_dt_rne(f: np.ndarray, dt: str) -> np.ndarray:
    """Round fp32 values to the dtype, nearest-even (finite inputs)."""
    f = np.asarray(f, dtype=np.float32)
    if dt == F16:
        return f.astype(np.float16)
    if dt == BF16:
        u = f.view(np.uint32).astype(np.uint64)
        lsb = (u >> np.uint64(16)) & np.uint64(1)
        return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    raise ValueError(dt)


def f32_to_dt_ru(f: np.ndarray, dt: str) -> np.ndarray:
    """Round non-negative fp32 values to the dtype, toward +infinity.

    Nearest-even first; where that landed below the input, step up one unit
    in the last place.
    """
    f = np.asarray(f, dtype=np.float32)
    assert np.all(f >= 0), "scale must be non-negative"
    r = f32_to_dt_rne(f, dt)
    below = to_f32(r, dt) < f
    if dt == F16:
        r = r.copy()
        r[below] = np.nextafter(r[below], np.float16(np.inf))
        return r
    r = r.copy()
    r[below] = r[below] + np.uint16(1)  # positive bf16: next bit pattern is next value up
    return r


# ---------------------------------------------------------------------------
# sizes
# ---------------------------------------------------------------------------

def packed_words(bits: int, K: int) -> int:
    """uint32 words holding one row of K values at ``bits`` bits."""
    assert (K * bits) % 32 == 0
    return K * bits // 32


def weight_bytes(N: int, K: int, bits: int, group_size: int) -> int:
    """Packed weight bytes plus 2+2 bytes of scale/bias per group.

    The MLX issue #4720 reproducer ("To Reproduce") counts exactly these
    bytes for its GB/s figure: N*K*bits/8 + N*K/gs*4 (activations and
    outputs excluded).
    """
    return N * K * bits // 8 + 4 * N * (K // group_size)


# ---------------------------------------------------------------------------
# packing: a little-endian bitstream per row
# ---------------------------------------------------------------------------

def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """[N, K] integer codes -> [N, K*bits/32] little-endian uint32 words."""
    q = np.asarray(q)
    N, K = q.shape
    assert bits in SUPPORTED_BITS and (K * bits) % 32 == 0
    assert q.min(initial=0) >= 0 and q.max(initial=0) < (1 << bits)
    out = np.empty((N, packed_words(bits, K)), dtype=np.uint32)
    shifts = np.arange(bits, dtype=np.uint32)
    for r0 in range(0, N, 512):
        qq = q[r0:r0 + 512].astype(np.uint32)
        # bit i of value k lands at stream position bits*k + i
        stream = ((qq[..., None] >> shifts) & np.uint32(1)).astype(np.uint8)
        stream = stream.reshape(qq.shape[0], K * bits)
        as_bytes = np.packbits(stream, axis=-1, bitorder="little")
        out[r0:r0 + 512] = as_bytes.view("<u4")
    return out


def unpack(words: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Inverse of :func:`pack`: [N, K*bits/32] words -> [N, K] codes (int32)."""
    words = np.ascontiguousarray(words, dtype="<u4")
    N = words.shape[0]
    assert words.shape[1] == packed_words(bits, K)
    out = np.empty((N, K), dtype=np.int32)
    place = (1 << np.arange(bits)).astype(np.int32)
    for r0 in range(0, N, 512):
        ww = words[r0:r0 + 512]
        stream = np.unpackbits(ww.view(np.uint8), axis=-1, bitorder="little")
        stream = stream.reshape(ww.shape[0], K, bits).astype(np.int32)
        out[r0:r0 + 512] = stream @ place
    return out


# ---------------------------------------------------------------------------
# quantize / dequantize
# ---------------------------------------------------------------------------

def quantize(w: np.ndarray, dt: str, bits: int, group_size: int):
    """Affine min/max group quantization of W [N, K] (dtype ``dt``).

    Returns (wq [N, K*bits/32] uint32, scales [N, K/gs] dt, biases [N, K/gs] dt).
    Steps per group, in fp32 with IEEE rounding:
      lo = min w, hi = max w                        (exact dtype values)
      s  = RU_dt( fl32( fl32(hi - lo) / (2^bits - 1) ) ),  b = lo
      q  = 0 if s == 0 else clamp(rint_half_even(fl32(fl32(w - b) / s)), 0, 2^bits - 1)
    """
    assert dt in DTYPES and bits in SUPPORTED_BITS and group_size in SUPPORTED_GROUP_SIZES
    N, K = w.shape
    assert K % group_size == 0
    G = K // group_size
    Q = np.float32((1 << bits) - 1)
    wf = to_f32(w, dt).reshape(N, G, group_size)
    assert np.all(np.isfinite(wf)), "inputs must be finite"
    # A zero minimum is taken as +0 so that the bias does not depend on the
    # order in which -0 and +0 are met (adding +0 maps -0 to +0 exactly).
    lo = (wf.min(axis=-1) + np.float32(0.0)).astype(np.float32)
    hi = wf.max(axis=-1)
    span = (hi - lo).astype(np.float32)                      # fl32(hi - lo)
    assert np.all(np.isfinite(span)), "group range must be finite in fp32"
    s32 = (span / Q).astype(np.float32)                     # fl32(span / Q)
    s_dt = f32_to_dt_ru(s32, dt)
    s = to_f32(s_dt, dt)
    b_dt = f32_to_dt_rne(lo, dt)                            # exact: lo is a dtype value
    b = to_f32(b_dt, dt)
    assert np.array_equal(b, lo) and not np.any(np.signbit(b) & (b == 0))
    diff = (wf - b[..., None]).astype(np.float32)            # fl32(w - b)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (diff / s[..., None]).astype(np.float32)         # fl32(diff / s)
    q = np.clip(np.rint(t), 0, Q)
    q = np.where(s[..., None] == 0, 0, q).astype(np.int32).reshape(N, K)
    return pack(q, bits), s_dt, b_dt


def dequantize(wq, scales, biases, dt: str, bits: int, group_size: int, K: int) -> np.ndarray:
    """Dequantized weights in the dtype: RNE_dt( fl32(s*q + b) ).

    s*q is exact in fp32 (at most 8+11 significant bits), so this is a single
    fp32 rounding followed by the rounding to the dtype.
    """
    q = unpack(wq, bits, K).astype(np.float32)
    N = q.shape[0]
    s = np.repeat(to_f32(scales, dt), group_size, axis=1).reshape(N, K)
    b = np.repeat(to_f32(biases, dt), group_size, axis=1).reshape(N, K)
    return f32_to_dt_rne((s * q + b).astype(np.float32), dt)


def dequantize_exact(wq, scales, biases, dt: str, bits: int, group_size: int, K: int) -> np.ndarray:
    """Dequantized weights without any rounding: f64(s)*q + f64(b).

    Exact in fp64 for every finite fp16 input and for bf16 groups whose
    range is not vanishingly small against their minimum.
    """
    q = unpack(wq, bits, K).astype(np.float64)
    N = q.shape[0]
    s = np.repeat(to_f64(scales, dt), group_size, axis=1).reshape(N, K)
    b = np.repeat(to_f64(biases, dt), group_size, axis=1).reshape(N, K)
    return s * q + b


# ---------------------------------------------------------------------------
# matmul
# ---------------------------------------------------------------------------

def qmm(x, wq, scales, biases, dt: str, bits: int, group_size: int, row_chunk: int = 8192):
    """y = x . dequant(W)^T accumulated in fp64, and the tolerance scale T.

    x is [M, K] in the dtype.  Returns (y [M, N] float64, T [M, N] float64)
    with T[m, n] = sum_k |x[m, k]| * |w_hat[n, k]|.  No rounding is applied to
    y; the acceptance rule is |y_gpu - y| <= 4e-3 * T + 1e-3 elementwise.
    """
    x64 = to_f64(x, dt)
    M, K = x64.shape
    N = wq.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    T = np.empty((M, N), dtype=np.float64)
    ax = np.abs(x64)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        w64 = dequantize_exact(wq[r0:r1], scales[r0:r1], biases[r0:r1], dt, bits, group_size, K)
        y[:, r0:r1] = x64 @ w64.T
        T[:, r0:r1] = ax @ np.abs(w64).T
    return y, T


def qmm_batched(x, wq, scales, biases, dt: str, bits: int, group_size: int):
    """Batched product with weights per batch entry: y[b] = x[b] . dequant(W[b])^T.

    MLX issue #4720, "Describe the bug", singles out transposed, non-batched
    calls; this is the batched form of the same product.  x is [B, M, K],
    wq [B, N, words], scales and biases [B, N, K/gs]; entry b uses only the
    b-th slice of each.  Returns (y [B, M, N], T [B, M, N]) as :func:`qmm`
    does for each entry.
    """
    B = x.shape[0]
    M, N = x.shape[1], wq.shape[1]
    y = np.empty((B, M, N), dtype=np.float64)
    T = np.empty((B, M, N), dtype=np.float64)
    for b in range(B):
        y[b], T[b] = qmm(x[b], wq[b], scales[b], biases[b], dt, bits, group_size)
    return y, T


def qmm_nt(x, wq, scales, biases, dt: str, bits: int, group_size: int, N: int):
    """Non-transposed product y = x . dequant(W) with W stored [K, N].

    MLX issue #4720, "Describe the bug", concerns calls with transposed
    weights; the other orientation (``transpose=False``) keeps W as [K, N],
    quantized along its last axis: row k of W is packed and grouped along N
    exactly as a row of the transposed layout is along K (``wq`` [K, N*bits/32],
    ``scales`` and ``biases`` [K, N/gs]).  x is [M, K].  Returns
    (y [M, N], T [M, N]) with T[m, n] = sum_k |x[m, k]| |w_hat[k, n]|, fp64,
    unrounded, as :func:`qmm`.
    """
    x64 = to_f64(x, dt)
    w64 = dequantize_exact(wq, scales, biases, dt, bits, group_size, N)  # [K, N]
    return x64 @ w64, np.abs(x64) @ np.abs(w64)


TOL_REL = 4e-3
TOL_ABS = 1e-3


def within_tolerance(y_gpu: np.ndarray, y_o: np.ndarray, T: np.ndarray):
    """Elementwise acceptance test; returns (ok, worst |err| / bound)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    bound = TOL_REL * T + TOL_ABS
    err = np.abs(y_gpu - y_o)
    ok = bool(np.all(np.isfinite(y_gpu)) and np.all(err <= bound))
    worst = float(np.max(err / bound)) if err.size else 0.0
    return ok, worst

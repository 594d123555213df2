"""Pins for the oracle's matmul y = x . dequant(W)^T (fp64 accumulation).

Checked against exact rational arithmetic on tiny inputs (with an
independent big-integer unpack), one-hot rows recovering dequantized
weights, the all-ones closed form, zero inputs, linearity and inert
zero-padded rows."""

from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import qmm_oracle as O


def bigint_unpack_row(words, bits, K):
    v = 0
    for i, w in enumerate(words):
        v |= int(w) << (32 * i)
    return [(v >> (bits * k)) & ((1 << bits) - 1) for k in range(K)]


def make(dt, bits, gs, M, N, K, seed):
    w = synth.to_oracle(synth.normal((N, K), 0.02, dt, seed))
    x = synth.to_oracle(synth.normal((M, K), 1.0, dt, seed + 1))
    wq, sc, bi = O.quantize(w, dt, bits, gs)
    return x, wq, sc, bi


@pytest.mark.parametrize("dt,bits,gs", [("f16", 4, 32), ("bf16", 6, 64), ("f16", 8, 32), ("bf16", 4, 128)])
def test_exact_rationals(dt, bits, gs):
    M, N, K = 2, 3, 2 * gs
    x, wq, sc, bi = make(dt, bits, gs, M, N, K, 31)
    y, T = O.qmm(x, wq, sc, bi, dt, bits, gs)
    xf = O.to_f64(x, dt)
    s = O.to_f64(sc, dt)
    b = O.to_f64(bi, dt)
    for n in range(N):
        q = bigint_unpack_row(wq[n], bits, K)
        wh = [Fraction(float(s[n, k // gs])) * q[k] + Fraction(float(b[n, k // gs])) for k in range(K)]
        for m in range(M):
            exact = sum(Fraction(float(xf[m, k])) * wh[k] for k in range(K))
            tabs = sum(abs(Fraction(float(xf[m, k])) * wh[k]) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= K * Fraction(2) ** -52 * tabs
            assert abs(Fraction(float(T[m, n])) - tabs) <= K * Fraction(2) ** -52 * tabs


@pytest.mark.parametrize("dt,bits,gs", [("f16", 4, 64), ("bf16", 8, 128), ("f16", 6, 32)])
def test_one_hot_rows_recover_dequantized_weights(dt, bits, gs):
    N, K = 5, 2 * gs
    _, wq, sc, bi = make(dt, bits, gs, 1, N, K, 41)
    one = 1.0
    xs = np.zeros((K, K), dtype=np.float32)
    np.fill_diagonal(xs, one)
    x = O.f32_to_dt_rne(xs, dt)
    y, _ = O.qmm(x, wq, sc, bi, dt, bits, gs)
    s = O.to_f64(sc, dt)
    b = O.to_f64(bi, dt)
    for n in range(N):
        q = bigint_unpack_row(wq[n], bits, K)
        for k in range(K):
            want = Fraction(float(s[n, k // gs])) * q[k] + Fraction(float(b[n, k // gs]))
            assert Fraction(float(y[k, n])) == want


def test_all_ones_closed_form():
    dt, bits, gs = "f16", 4, 64
    N, K = 7, 256
    _, wq, sc, bi = make(dt, bits, gs, 1, N, K, 51)
    x = O.f32_to_dt_rne(np.ones((1, K), np.float32), dt)
    y, _ = O.qmm(x, wq, sc, bi, dt, bits, gs)
    s = O.to_f64(sc, dt)
    b = O.to_f64(bi, dt)
    for n in range(N):
        q = bigint_unpack_row(wq[n], bits, K)
        want = sum(Fraction(float(s[n, g])) * sum(q[g * gs:(g + 1) * gs]) + gs * Fraction(float(b[n, g]))
                   for g in range(K // gs))
        assert abs(Fraction(float(y[0, n])) - want) <= Fraction(2) ** -40


def test_zero_input_gives_zero():
    x, wq, sc, bi = make("bf16", 6, 32, 3, 9, 128, 61)
    y, T = O.qmm(np.zeros_like(x), wq, sc, bi, "bf16", 6, 32)
    assert np.all(y == 0) and np.all(T == 0)


def test_linearity_and_padded_rows():
    dt, bits, gs = "f16", 4, 64
    x, wq, sc, bi = make(dt, bits, gs, 4, 33, 256, 71)
    y, _ = O.qmm(x, wq, sc, bi, dt, bits, gs)
    # padding with zero rows leaves the real rows bit-for-bit unchanged
    xp = np.concatenate([x, np.zeros((3, 256), np.float16)], axis=0)
    yp, _ = O.qmm(xp, wq, sc, bi, dt, bits, gs)
    assert np.array_equal(yp[:4], y) and np.all(yp[4:] == 0)
    # row permutation commutes; scaling a row by 2 (exact) scales the result
    yr, _ = O.qmm(x[::-1].copy(), wq, sc, bi, dt, bits, gs)
    assert np.array_equal(yr, y[::-1])
    y2, _ = O.qmm((x.astype(np.float32) * 2).astype(np.float16), wq, sc, bi, dt, bits, gs)
    assert np.allclose(y2, 2 * y, rtol=1e-12, atol=1e-12)


def test_tolerance_rule():
    y_o = np.array([[1.0, -2.0]])
    T = np.array([[10.0, 10.0]])
    ok, worst = O.within_tolerance(y_o + 0.04, y_o, T)     # bound is 0.041
    assert ok and worst < 1
    ok, _ = O.within_tolerance(y_o + 0.05, y_o, T)
    assert not ok
    ok, _ = O.within_tolerance(np.array([[np.nan, -2.0]]), y_o, T)
    assert not ok


# ---------------------------------------------------------------------------
# batched form: one weight matrix per batch entry
# ---------------------------------------------------------------------------

def _scaled(a, dt, factor):
    """a * factor in the dtype (a power of two: exact for these magnitudes)."""
    return O.f32_to_dt_rne((O.to_f32(a, dt) * np.float32(factor)).astype(np.float32), dt)


@pytest.mark.parametrize("dt,bits,gs", [("f16", 4, 64), ("bf16", 8, 32), ("bf16", 6, 128)])
def test_batched_entries_use_their_own_weights_and_rows(dt, bits, gs):
    """Entry b with weights 2^b W quantizes to the same codes with 2^b the
    scales and biases, so its output is exactly 2^b times entry 0's; with
    activations 2^b x likewise.  A batched product that reads another
    entry's weights or rows breaks one of the two."""
    B, M, N, K = 4, 3, 5, 2 * gs
    w = synth.to_oracle(synth.normal((N, K), 0.02, dt, 81))
    x = synth.to_oracle(synth.normal((M, K), 1.0, dt, 82))
    ws = [_scaled(w, dt, 2.0 ** b) for b in range(B)]
    qs = [O.quantize(wb, dt, bits, gs) for wb in ws]
    for b in range(1, B):
        assert np.array_equal(qs[b][0], qs[0][0])
        assert np.array_equal(O.to_f64(qs[b][1], dt), 2.0 ** b * O.to_f64(qs[0][1], dt))
    wq, sc, bi = (np.stack([q[i] for q in qs]) for i in range(3))
    y, T = O.qmm_batched(np.stack([x] * B), wq, sc, bi, dt, bits, gs)
    assert y.shape == (B, M, N) and T.shape == (B, M, N)
    for b in range(B):
        assert np.array_equal(y[b], 2.0 ** b * y[0]) and np.array_equal(T[b], 2.0 ** b * T[0])
    xs = np.stack([_scaled(x, dt, 2.0 ** b) for b in range(B)])
    y2, _ = O.qmm_batched(xs, np.stack([qs[0][0]] * B), np.stack([qs[0][1]] * B), np.stack([qs[0][2]] * B),
                          dt, bits, gs)
    for b in range(B):
        assert np.array_equal(y2[b], 2.0 ** b * y2[0])
    assert np.array_equal(y2[0], y[0])


def test_batched_exact_rationals():
    """Independent entries against exact rational sums (big-integer unpack)."""
    dt, bits, gs = "f16", 4, 32
    B, M, N, K = 3, 2, 3, 64
    xs, wqs, scs, bis = [], [], [], []
    for b in range(B):
        x, wq, sc, bi = make(dt, bits, gs, M, N, K, 90 + 2 * b)
        xs.append(x); wqs.append(wq); scs.append(sc); bis.append(bi)
    y, _ = O.qmm_batched(np.stack(xs), np.stack(wqs), np.stack(scs), np.stack(bis), dt, bits, gs)
    for b in range(B):
        xf, s, bb = O.to_f64(xs[b], dt), O.to_f64(scs[b], dt), O.to_f64(bis[b], dt)
        for n in range(N):
            q = bigint_unpack_row(wqs[b][n], bits, K)
            wh = [Fraction(float(s[n, k // gs])) * q[k] + Fraction(float(bb[n, k // gs])) for k in range(K)]
            for m in range(M):
                exact = sum(Fraction(float(xf[m, k])) * wh[k] for k in range(K))
                tabs = sum(abs(Fraction(float(xf[m, k])) * wh[k]) for k in range(K))
                assert abs(Fraction(float(y[b, m, n])) - exact) <= K * Fraction(2) ** -52 * tabs


# ---------------------------------------------------------------------------
# non-transposed form: W stored [K, N], quantized along N
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt,bits,gs", [("f16", 4, 32), ("bf16", 6, 64), ("bf16", 8, 128)])
def test_nt_exact_rationals(dt, bits, gs):
    """Tiny non-transposed products against exact rational sums, with an
    independent big-integer unpack of each row k of W [K, N]."""
    M, K, N = 2, 3, 2 * gs
    w = synth.to_oracle(synth.normal((K, N), 0.02, dt, 101))
    x = synth.to_oracle(synth.normal((M, K), 1.0, dt, 102))
    wq, sc, bi = O.quantize(w, dt, bits, gs)
    assert wq.shape[0] == K and sc.shape == (K, N // gs)
    y, T = O.qmm_nt(x, wq, sc, bi, dt, bits, gs, N)
    assert y.shape == (M, N)
    xf, s, b = O.to_f64(x, dt), O.to_f64(sc, dt), O.to_f64(bi, dt)
    rows = [bigint_unpack_row(wq[k], bits, N) for k in range(K)]
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(xf[m, k])) * (Fraction(float(s[k, n // gs])) * rows[k][n]
                                                   + Fraction(float(b[k, n // gs]))) for k in range(K)]
            exact, tabs = sum(terms), sum(abs(t) for t in terms)
            assert abs(Fraction(float(y[m, n])) - exact) <= K * Fraction(2) ** -52 * tabs
            assert abs(Fraction(float(T[m, n])) - tabs) <= K * Fraction(2) ** -52 * tabs


def test_nt_one_hot_rows_recover_weight_rows():
    """x = e_k picks row k of the dequantized [K, N] weights, which is the
    dequantizer's output for that row (exact in fp64, then rounded once)."""
    dt, bits, gs = "f16", 4, 64
    K, N = 24, 192
    w = synth.to_oracle(synth.normal((K, N), 0.02, dt, 111))
    wq, sc, bi = O.quantize(w, dt, bits, gs)
    x = np.zeros((K, K), np.float16)
    x[np.arange(K), np.arange(K)] = 1
    y, _ = O.qmm_nt(x, wq, sc, bi, dt, bits, gs, N)
    d = O.dequantize(wq, sc, bi, dt, bits, gs, N)  # [K, N] in the dtype
    assert np.array_equal(O.f32_to_dt_rne(y.astype(np.float32), dt).view(np.uint16), d.view(np.uint16))


def test_nt_against_transposed_product_of_the_transpose():
    """With the dequantized weights in hand, x . W_hat equals the transposed
    product against W_hat^T: quantizing W_hat^T [N, K] along K with one group
    per row segment reproduces the same values when every group of W_hat^T
    is built from values that are already on a grid.  Here: W chosen so that
    each [K, N] group holds exactly the values s*q + b of an integer grid,
    and groups along both axes coincide (gs = K = N)."""
    dt, bits, gs = "f16", 8, 64
    K = N = 64
    rng = np.random.default_rng(5)
    # one scale and bias for the whole matrix: every row and column group
    # quantizes back to the same grid, whichever axis it runs along
    q = rng.integers(0, 256, size=(K, N))
    q[:, 0], q[:, 1] = 0, 255  # each row reaches both ends of the grid
    q[0, :], q[1, :] = 0, 255  # ... and each column
    q[0, 1] = q[1, 0] = 0
    q[1, 1] = q[0, 0] = 255
    s, b = np.float16(2.0 ** -10), np.float16(-0.125)
    w = (np.float16(s) * q.astype(np.float16) + b).astype(np.float16)
    x = synth.to_oracle(synth.normal((3, K), 1.0, dt, 121))
    wq, sc, bi = O.quantize(w, dt, bits, gs)
    wqt, sct, bit = O.quantize(np.ascontiguousarray(w.T), dt, bits, gs)
    y_nt, _ = O.qmm_nt(x, wq, sc, bi, dt, bits, gs, N)
    y_t, _ = O.qmm(x, wqt, sct, bit, dt, bits, gs)
    assert np.allclose(y_nt, y_t, rtol=1e-12, atol=1e-12)
    assert np.allclose(y_nt, O.to_f64(x, dt) @ w.astype(np.float64), rtol=1e-12, atol=1e-12)

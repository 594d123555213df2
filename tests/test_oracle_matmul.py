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

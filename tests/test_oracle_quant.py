"""Pins for the oracle's quantizer and dequantizer.

Checked against: hand-worked examples (golden file), brute-force nearest grid
points, the half-step round-trip bound, exact constant groups, library
rounding routines (torch / struct) for the dtype conversions, and an
exhaustive enumeration of the dtype for the round-up conversion.
"""

import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import qmm_oracle as O

COMBOS = [(dt, bits, gs) for dt in ("f16", "bf16") for bits in (4, 6, 8) for gs in (32, 64, 128)]


def dt_from_bits(hexes, dt):
    u = np.array([int(h, 16) for h in hexes], dtype=np.uint16)
    return u.view(np.float16) if dt == "f16" else u


def dt_bits(a, dt):
    a = np.asarray(a)
    return a.view(np.uint16) if dt == "f16" else a.astype(np.uint16)


# --------------------------------------------------------------- conversions

def test_rne_matches_torch():
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-8, 5, 20000),
        # exact halfway points between neighbouring bf16 / fp16 values
        (np.arange(1, 4000, dtype=np.uint32) << 15 | 0x3F800000).view(np.float32),
        (np.arange(1, 4000, dtype=np.uint32) << 12 | 0x3F800000).view(np.float32),
    ]).astype(np.float32)
    t = torch.from_numpy(f)
    assert np.array_equal(O.f32_to_dt_rne(f, "f16"), t.to(torch.float16).numpy())
    assert np.array_equal(O.f32_to_dt_rne(f, "bf16"), t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_f16_rne_matches_struct():
    rng = np.random.default_rng(2)
    f = (rng.standard_normal(3000) * 3).astype(np.float32)
    want = np.array([struct.unpack("<H", struct.pack("<e", float(v)))[0] for v in f], dtype=np.uint16)
    assert np.array_equal(O.f32_to_dt_rne(f, "f16").view(np.uint16), want)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_round_up_is_smallest_value_not_below(dt):
    """RU(f) is the smallest finite dtype value >= f, by enumerating the dtype."""
    pats = np.arange(0, 0x7C00 if dt == "f16" else 0x7F80, dtype=np.uint32).astype(np.uint16)
    vals = O.to_f32(pats.view(np.float16) if dt == "f16" else pats, dt)
    order = np.argsort(vals, kind="stable")
    sorted_vals = vals[order]
    rng = np.random.default_rng(3)
    f = np.abs(rng.standard_normal(20000).astype(np.float32)) * np.float32(10.0) ** rng.integers(-9, 4, 20000)
    f = np.concatenate([f, sorted_vals[:2000], np.array([0.0], np.float32)]).astype(np.float32)
    if dt == "f16":
        f = f[f <= 65504]
    idx = np.searchsorted(sorted_vals, f, side="left")
    want = sorted_vals[idx]
    got = O.to_f32(O.f32_to_dt_ru(f, dt), dt)
    assert np.array_equal(got, want)


# --------------------------------------------------------------- worked examples

def test_worked_examples(golden):
    rows = golden("quant_worked_examples.txt")
    assert [r[0] for r in rows] == ["A", "B", "C", "D"]
    for name, dt, bits, gs, w, s, b, words, deq in rows:
        bits, gs = int(bits), int(gs)
        wv = dt_from_bits(w.split(), dt).reshape(1, gs)
        wq, sc, bi = O.quantize(wv, dt, bits, gs)
        assert int(dt_bits(sc, dt)[0, 0]) == int(s, 16), name
        assert int(dt_bits(bi, dt)[0, 0]) == int(b, 16), name
        assert [int(x) for x in wq[0]] == [int(x, 16) for x in words.split()], name
        d = O.dequantize(wq, sc, bi, dt, bits, gs, gs)
        assert [int(x) for x in dt_bits(d, dt)[0]] == [int(x, 16) for x in deq.split()], name


def test_round_up_changes_example_b():
    """Nearest-even scale would be 0x3044 and dequantize +1 to 0.99951172;
    the round-up scale 0x3045 gives 1.0009766 (guards against RNE)."""
    w = np.tile(np.array([-1, 1], dtype=np.float16), 16).reshape(1, 32)
    _, sc, _ = O.quantize(w, "f16", 4, 32)
    assert sc.view(np.uint16)[0, 0] == 0x3045
    assert O.f32_to_dt_rne(np.float32(2) / np.float32(15), "f16").view(np.uint16) == 0x3044


# --------------------------------------------------------------- properties

def exact_w_hat(wq, sc, bi, dt, bits, gs, K):
    q = O.unpack(wq, bits, K).astype(np.float64)
    s = np.repeat(O.to_f64(sc, dt), gs, axis=1)
    b = np.repeat(O.to_f64(bi, dt), gs, axis=1)
    return s * q + b, q, s, b


@pytest.mark.parametrize("dt,bits,gs", COMBOS)
def test_round_trip_bound(dt, bits, gs):
    """|w - (s*q + b)| <= s/2 (+ fp32 slack), for normal, outlier, tiny-range
    and constant groups; and the dtype-rounded dequant adds at most half an ulp."""
    K = 2 * gs
    N = 64
    Q = (1 << bits) - 1
    ws = [
        synth.normal((N, K), 0.02, dt, 11),
        synth.normal((N, K), 0.02, dt, 12, outlier_frac=0.05),
        synth.special_groups("tiny", N, K, gs, dt, 13),
        synth.special_groups("constant", N, K, gs, dt, 14),
        synth.special_groups("mixed", N, K, gs, dt, 15),
    ]
    for wt in ws:
        w = synth.to_oracle(wt)
        wq, sc, bi = O.quantize(w, dt, bits, gs)
        w64 = O.to_f64(w, dt)
        what, q, s, b = exact_w_hat(wq, sc, bi, dt, bits, gs, K)
        assert q.min() >= 0 and q.max() <= Q
        bound = s / 2 + 2.0 ** -20 * Q * s
        assert np.all(np.abs(w64 - what) <= bound)
        # q(min) == 0 in every group
        lo_pos = np.argmin(w64.reshape(N, -1, gs), axis=-1)
        qg = q.reshape(N, -1, gs)
        assert np.all(np.take_along_axis(qg, lo_pos[..., None], -1) == 0)
        # constant groups are exact
        const = (w64.reshape(N, -1, gs).max(-1) == w64.reshape(N, -1, gs).min(-1))
        assert np.all((s.reshape(N, -1, gs)[..., 0] == 0) == const)
        assert np.array_equal(what.reshape(N, -1, gs)[const], w64.reshape(N, -1, gs)[const])
        # dtype-rounded dequantization
        d = O.to_f64(O.dequantize(wq, sc, bi, dt, bits, gs, K), dt)
        ulp = np.spacing(np.abs(d).astype(np.float16 if dt == "f16" else np.float32)).astype(np.float64)
        if dt == "bf16":
            ulp = ulp * 2.0 ** 16
        assert np.all(np.abs(d - what) <= ulp / 2 + 2.0 ** -24 * np.abs(what) + 1e-30)


@pytest.mark.parametrize("dt,bits", [(dt, b) for dt in ("f16", "bf16") for b in (4, 6, 8)])
def test_brute_force_nearest_grid_point(dt, bits):
    """Every q is a nearest grid point of the stored scale: no q' in [0, Q]
    is closer in exact rational arithmetic by more than fp32 rounding."""
    gs = 32
    Q = (1 << bits) - 1
    w = synth.to_oracle(synth.normal((6, gs), 0.5, dt, 21 + bits))
    wq, sc, bi = O.quantize(w, dt, bits, gs)
    q = O.unpack(wq, bits, gs)
    wf = O.to_f64(w, dt)
    for n in range(w.shape[0]):
        s = Fraction(float(O.to_f64(sc, dt)[n, 0]))
        b = Fraction(float(O.to_f64(bi, dt)[n, 0]))
        slack = Fraction(2) ** -20 * Q * s
        for k in range(gs):
            wk = Fraction(float(wf[n, k]))
            best = min(abs(wk - (s * qq + b)) for qq in range(Q + 1))
            assert abs(wk - (s * int(q[n, k]) + b)) <= best + slack


def test_dequantize_against_independent_rounding():
    """RNE_dt(fl32(s*q + b)) from exact rationals, rounded with struct (fp32,
    fp16) and torch (bf16), matches the oracle's dequantize."""
    rng = np.random.default_rng(5)
    for dt, bits, gs in [("f16", 4, 64), ("bf16", 8, 32), ("f16", 6, 128), ("bf16", 4, 32)]:
        w = synth.to_oracle(synth.normal((16, 2 * gs), 0.3, dt, int(rng.integers(1000))))
        wq, sc, bi = O.quantize(w, dt, bits, gs)
        d = O.dequantize(wq, sc, bi, dt, bits, gs, 2 * gs)
        q = O.unpack(wq, bits, 2 * gs)
        s = O.to_f64(sc, dt)
        b = O.to_f64(bi, dt)
        for n in range(16):
            for k in range(0, 2 * gs, 7):
                exact = Fraction(float(s[n, k // gs])) * int(q[n, k]) + Fraction(float(b[n, k // gs]))
                f32 = struct.unpack("<f", struct.pack("<f", float(exact)))[0]
                if dt == "f16":
                    want = struct.unpack("<H", struct.pack("<e", f32))[0]
                    got = int(d.view(np.uint16)[n, k])
                else:
                    want = int(torch.tensor([f32], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
                    got = int(d[n, k])
                assert got == want


def test_q_of_max_is_not_always_Q(golden):
    """With round-up scales q(max) can fall one short of Q (example D)."""
    rows = {r[0]: r for r in golden("quant_worked_examples.txt")}
    assert rows["D"][7].split()[0] == "000000FE"


def test_signed_zero_minimum_gives_positive_zero_bias():
    """A group whose minimum is zero stores bias +0 whatever the order of -0/+0."""
    for first in (-0.0, 0.0):
        w = np.array([[first, -first] + [0.5] * 30], dtype=np.float16)
        _, _, bi = O.quantize(w, "f16", 4, 32)
        assert bi.view(np.uint16)[0, 0] == 0x0000

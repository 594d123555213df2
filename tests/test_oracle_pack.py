"""Pins for the oracle's packing: closed-form words and an independent
big-integer bitstream (value k at bits [bits*k, bits*k + bits), LE words)."""

import numpy as np
import pytest

from oracle import qmm_oracle as O


def bigint_pack_row(q, bits):
    """Independent definition: one Python integer holds the row's bitstream."""
    v = 0
    for k, qk in enumerate(q):
        v |= int(qk) << (bits * k)
    nwords = len(q) * bits // 32
    return [(v >> (32 * i)) & 0xFFFFFFFF for i in range(nwords)]


def bigint_unpack_row(words, bits, K):
    v = 0
    for i, w in enumerate(words):
        v |= int(w) << (32 * i)
    return [(v >> (bits * k)) & ((1 << bits) - 1) for k in range(K)]


def test_closed_form_words(golden):
    rows = golden("pack_words.txt")
    assert len(rows) >= 8
    for bits, vals, words in rows:
        bits = int(bits)
        q = np.array([[int(v) for v in vals.split()]], dtype=np.int32)
        want = np.array([[int(w, 16) for w in words.split()]], dtype=np.uint32)
        got = O.pack(q, bits)
        assert np.array_equal(got, want), (bits, vals, [hex(x) for x in got[0]])
        assert np.array_equal(O.unpack(want, bits, q.shape[1]), q)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_matches_bigint_bitstream(bits):
    rng = np.random.default_rng(bits)
    K = 192
    q = rng.integers(0, 1 << bits, size=(7, K))
    got = O.pack(q, bits)
    for r in range(q.shape[0]):
        assert list(got[r]) == bigint_pack_row(q[r], bits)
        assert list(O.unpack(got[r:r + 1], bits, K)[0]) == bigint_unpack_row(got[r], bits, K)


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_every_value_at_every_position(bits):
    """Each code value placed at each position of one packing unit, the rest
    random, survives pack -> unpack and lands in the right bits."""
    rng = np.random.default_rng(100 + bits)
    unit = 16 if bits == 6 else 32 // bits * 4   # values per 3 words (6-bit) / per 4 words
    rows = []
    for pos in range(unit):
        for val in range(1 << bits):
            r = rng.integers(0, 1 << bits, size=unit)
            r[pos] = val
            rows.append(r)
    q = np.array(rows)
    words = O.pack(q, bits)
    assert np.array_equal(O.unpack(words, bits, unit), q)
    for i in range(0, len(rows), 97):
        assert list(words[i]) == bigint_pack_row(q[i], bits)


def test_word_counts():
    assert O.packed_words(4, 4096) == 512
    assert O.packed_words(8, 4096) == 1024
    assert O.packed_words(6, 4096) == 768
    assert O.packed_words(6, 64) == 12


def test_weight_bytes_from_issue(golden):
    for N, K, bits, gs, nbytes in golden("weight_bytes.txt"):
        assert O.weight_bytes(int(N), int(K), int(bits), int(gs)) == int(nbytes)

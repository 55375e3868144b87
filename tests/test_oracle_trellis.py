"""Pins of the oracle's trellis codebook and decoders (CPU only)."""

import os

import numpy as np
import pytest

from oracle import trellis

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def test_codebook_test_vectors():
    for s, v in _rows("codebook_values.txt"):
        assert trellis.codebook(int(s, 16)) * 8192 == int(v)


def test_codebook_closed_form_properties():
    v = trellis.codebook(np.arange(65536)) * 8192
    # every value is an integer multiple of 2^-13 (exact in fp16)
    assert np.all(v == np.round(v))
    # magnitudes 2^(e-3) (1 + m/1024), e in 0..3, m in 0..1023:
    # [1024, 8 * 2047] / 8192
    a = np.abs(v)
    assert a.min() == 1024 and a.max() == 8 * 2047
    # the hash is a bijection of 16-bit states and bits 12..14 of h are
    # unused: every (sign, e, m) appears exactly 8 times
    vals, counts = np.unique(v, return_counts=True)
    assert len(vals) == 2 * 4 * 1024 and np.all(counts == 8)
    # sign is bit 15 of a bijection: exact zero mean
    assert v.sum() == 0
    # mean square: (1/4) sum_e 4^(e-3) * mean_m (1 + m/1024)^2
    m = np.arange(1024)
    ms = np.mean([4.0 ** (e - 3) for e in range(4)]) * np.mean((1 + m / 1024) ** 2)
    assert abs(np.mean((v / 8192) ** 2) - ms) < 1e-12
    # fp16 representability of every codebook value
    f = (v / 8192).astype(np.float16).astype(np.float64)
    assert np.array_equal(f, v / 8192)


@pytest.mark.parametrize("K", range(2, 9))
def test_tile_test_vectors(K):
    row = [r for r in _rows("tile_vectors.txt") if int(r[0]) == K][0]
    b = np.array([(37 * j + 11) % 256 for j in range(32 * K)], dtype=np.uint8)
    words = b.view("<u2")[None, :]
    for dec in (trellis.decode_tiles_window, trellis.decode_tiles_shift):
        W = dec(words, K)[0] * 8192
        got = [W[0, 0], W[1, 0], W[0, 1], W[15, 15], W.sum(), (W * W).sum()]
        assert [int(round(g)) for g in got] == [int(x) for x in row[1:]]


@pytest.mark.parametrize("K", range(2, 9))
def test_two_decoders_agree(K):
    rng = np.random.default_rng(K)
    words = rng.integers(0, 65536, size=(64, 16 * K), dtype=np.uint16)
    a = trellis.decode_tiles_window(words, K)
    b = trellis.decode_tiles_shift(words, K)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("K", [2, 3, 4, 5, 8])
def test_constant_streams(K):
    zero = np.zeros((1, 16 * K), np.uint16)
    ones = np.full((1, 16 * K), 0xFFFF, np.uint16)
    # all states 0 -> h = 0 -> 1/8; all states 0xFFFF -> h = 0x61C9 -> 1481/8192
    for dec in (trellis.decode_tiles_window, trellis.decode_tiles_shift):
        assert np.all(dec(zero, K) == 0.125)
        assert np.all(dec(ones, K) == 1481 / 8192)


@pytest.mark.parametrize("K", [3, 4, 7])
def test_single_bit_lands_in_its_windows(K):
    # A single set stream bit j lies in the 16-bit windows of the consecutive
    # states covering it (tail-biting included), at bit j - (iK + K - 16).
    L = 256 * K
    for j in (0, 5, L - 1, L // 2 + 3):
        bits = np.zeros(L, np.uint8)
        bits[j] = 1
        words = np.packbits(bits, bitorder="little").view("<u2")[None, :]
        s = trellis.tile_states_shift(words, K)[0]
        nz = np.nonzero(s)[0]
        # windows advance by K bits, so a bit sits in 16/K of them (rounded)
        assert len(nz) in (16 // K, -(-16 // K))
        for i in range(256):
            t = (j - (i * K + K - 16)) % L
            expect = (1 << t) if t < 16 else 0
            assert s[i] == expect


def test_tensor_order_is_out_major():
    # words [out/16][in/16][16K]: only tile (kt=2, nt=1) all-ones.
    K, fin, fout = 4, 64, 48
    w = np.zeros(trellis.tensor_words(fin, fout, K), np.uint16)
    kt_n = fin // 16
    start = (1 * kt_n + 2) * 16 * K
    w[start:start + 16 * K] = 0xFFFF
    W = trellis.dequantize(w, fin, fout, K)
    # every all-zero tile decodes to the constant 1/8, the all-ones tile to
    # the constant 1481/8192
    expect = np.full((fin, fout), 0.125)
    expect[32:48, 16:32] = 1481 / 8192
    assert np.array_equal(W, expect)
    assert np.array_equal(trellis.dequantize(w, fin, fout, K, "window"), W)


def test_golden_files_match_their_generator():
    # the stored vectors are exactly what the independent bit-by-bit
    # generator beside them prints
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_vectors", os.path.join(GOLDEN, "make_vectors.py"))
    mv = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mv)
    assert mv.stored_lines("codebook_values.txt") == mv.codebook_lines()
    assert mv.stored_lines("tile_vectors.txt") == mv.tile_lines()

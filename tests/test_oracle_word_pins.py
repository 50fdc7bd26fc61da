"""Pins of the oracle's word layout for a native integer all-reduce (CPU only).

The layout puts floor(32 / W) biased W-bit fields (code + M) in each 32-bit
word, so that the plain word-wise uint32 SUM of a collective adds every
field exactly ("Global-QSGD: Practical Floatless Quantization ...", Sec. 6:
the codes are reduced by the collective's own integer sum).  The pins check
the oracle against what does not depend on it: the exact integer sum of the
codes, a Python big-integer construction of each row from the layout's
definition, and the minimal-width rule that makes the sum exact.
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import SCHEME_E, SCHEME_L


def _bigint_row(codes_row, W, M, row_bytes):
    """The row as one little-endian integer, built from the definition:
    field j = code_j + M at bit 32 (j // f) + W (j % f)."""
    f = 32 // W
    v = 0
    for j, c in enumerate(codes_row):
        v += (int(c) + M) << (32 * (j // f) + W * (j % f))
    return v.to_bytes(row_bytes, "little")


@pytest.mark.parametrize("W", [2, 3, 5, 7, 8, 9, 11, 13, 16, 17, 31, 32])
def test_layout_matches_big_integer_construction(W):
    M = (1 << (W - 2)) if W > 2 else 1  # codes in [-M, M], 2M < 2^W
    rng = np.random.default_rng(W)
    n, d = 3, 97
    codes = rng.integers(-M, M + 1, size=(n, d), dtype=np.int64).astype(np.int32)
    words = oracle.pack_words(codes, W, M)
    rb = oracle.word_row_bytes(d, W)
    assert words.shape == (n, rb // 4) and rb % 16 == 0
    for i in range(n):
        assert words[i].tobytes() == _bigint_row(codes[i], W, M, rb)
    # pad: no more 16-byte groups than the fields need
    f = 32 // W
    assert (rb - 16) * 8 < -(-d // f) * 32 <= rb * 8


@pytest.mark.parametrize("n,s,scheme", [(1, 1, SCHEME_L), (2, 1, SCHEME_L), (2, 3, SCHEME_L),
                                        (3, 2, SCHEME_L), (3, 3, SCHEME_E), (4, 1, SCHEME_L),
                                        (2, 4, SCHEME_E), (5, 2, SCHEME_L)])
def test_word_sum_is_exact_for_every_code_tuple(n, s, scheme):
    """Every tuple of n codes in [-M, M], at every field position of a word,
    summed word-wise modulo 2^32 and unpacked, gives the exact integer sum."""
    M = oracle.top_code(s, scheme)
    W = oracle.min_code_bits(n, s, scheme)
    f = oracle.word_fields(W)
    tuples = np.array(list(itertools.product(range(-M, M + 1), repeat=n)), dtype=np.int32).T
    for shift in range(f):  # the tuples start at every field position
        codes = np.concatenate([np.zeros((n, shift), np.int32), tuples], axis=1)
        d = codes.shape[1]
        total = oracle.unpack_word_sums(oracle.sum_words(oracle.pack_words(codes, W, M)),
                                        n, d, W, M)
        assert np.array_equal(total, codes.astype(np.int64).sum(axis=0))


@pytest.mark.parametrize("n,s,scheme", [(2, 3, SCHEME_L), (3, 7, SCHEME_L), (8, 127, SCHEME_L),
                                        (16, 8, SCHEME_E), (64, 3, SCHEME_L), (8, 15, SCHEME_L)])
def test_minimal_width_is_the_exactness_boundary(n, s, scheme):
    """At the minimal width every field sum fits; one bit less and the
    all-(+M) and all-(-M) columns no longer come back."""
    M = oracle.top_code(s, scheme)
    W = oracle.min_code_bits(n, s, scheme)
    d = 2 * oracle.word_fields(W) + 1
    for sign in (1, -1):
        codes = np.full((n, d), sign * M, dtype=np.int32)
        ok = oracle.unpack_word_sums(oracle.sum_words(oracle.pack_words(codes, W, M)), n, d, W, M)
        assert np.all(ok == sign * n * M)
    if W > 2:
        Wl = W - 1
        codes = np.full((n, d), M, dtype=np.int32)
        bad = oracle.unpack_word_sums(oracle.sum_words(oracle.pack_words(codes, Wl, M)),
                                      n, d, Wl, M)
        assert not np.all(bad == n * M)


def test_native_word_sum_equals_big_integer_sum():
    """Fields never carry into the next word: the word-wise uint32 sum of
    the rows is the big-integer sum of the rows."""
    n, s = 8, 127
    M, W = s, oracle.min_code_bits(n, s, SCHEME_L)
    rng = np.random.default_rng(5)
    d = 1001
    codes = rng.integers(-M, M + 1, size=(n, d)).astype(np.int32)
    codes[:, :7] = M
    words = oracle.pack_words(codes, W, M)
    rb = oracle.word_row_bytes(d, W)
    big = sum(int.from_bytes(words[i].tobytes(), "little") for i in range(n))
    assert oracle.sum_words(words).tobytes() == big.to_bytes(rb, "little")


@pytest.mark.parametrize("key", [1, 2])
def test_word_path_gives_the_same_mean(key):
    """Quantize, pack to words, sum the words, unpack, dequantize: the same
    code sums and mean as the direct integer sum."""
    w = wl.WORKLOADS[key]
    d = 20_000
    x = wl.generate(w, d=d)
    scheme = SCHEME_L if w.scheme == "L" else SCHEME_E
    N, _ = oracle.global_norm(x, w.q, w.p)
    codes = oracle.quantize(x, N, w.s, scheme, w.seed)
    M = oracle.top_code(w.s, scheme)
    W = oracle.min_code_bits(w.n, w.s, scheme)
    sums = oracle.unpack_word_sums(oracle.sum_words(oracle.pack_words(codes, W, M)),
                                   w.n, d, W, M)
    assert np.array_equal(sums, oracle.sum_codes(codes))
    assert np.array_equal(oracle.dequantize(sums, w.n, N, w.s, scheme),
                          oracle.dequantize(oracle.sum_codes(codes), w.n, N, w.s, scheme))

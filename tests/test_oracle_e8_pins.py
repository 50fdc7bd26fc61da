"""Pins of the oracle's 8-bit exponential-dithering wire format and its
re-rounding tree reduction ("Global-QSGD: Practical Floatless Quantization
for Distributed Learning with Theoretical Guarantees", Sec. 4 worked example:
1 sign bit and 7 level bits; Sec. 6: custom reduction inside the Allreduce).

Checked against the format's definition (explicit code table), exact
rationals (unbiasedness of one re-rounding, found threshold by bisection),
exact enumeration of every rounding path of a small tree, and Monte Carlo.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

TWO32 = 1 << 32


def threshold(v):
    """F of one re-rounding: the smallest u that rounds down (bisection on u)."""
    hi_code = oracle.e8_round(v, 0)
    lo, hi = 0, TWO32
    while lo < hi:
        mid = (lo + hi) // 2
        if oracle.e8_round(v, mid) == hi_code:
            lo = mid + 1
        else:
            hi = mid
    return lo


def test_code_table():
    assert oracle.e8_value(0x00) == 0.0
    assert oracle.e8_value(0x80) == 0.0
    assert oracle.e8_value(0x01) == 1.0 and oracle.e8_value(0x81) == -1.0
    assert oracle.e8_value(0x02) == 0.5 and oracle.e8_value(0x83) == -0.25
    assert oracle.e8_value(0x7F) == 2.0 ** -126 and oracle.e8_value(0xFF) == -(2.0 ** -126)
    vals = {oracle.e8_value(c) for c in range(256)}
    assert len(vals) == 255  # +-2^-m for m < 127, and one zero


@pytest.mark.parametrize("m", [0, 1, 5, 60, 125, 126])
def test_levels_are_fixed_points(m):
    for sign in (1.0, -1.0):
        v = sign * 2.0 ** -m
        for u in (0, 1, 12345, TWO32 - 1):
            assert oracle.e8_value(oracle.e8_round(v, u)) == v
    assert oracle.e8_round(0.0, 0) == 0 and oracle.e8_round(-0.0, 0) == 0


@pytest.mark.parametrize("v", [0.3, -0.7, 0.75, 1e-3, -3.3e-20, 2.0 ** -126 * 0.3,
                               2.0 ** -126 * 1.7, 0.999999, 2.0 ** -40 * 1.1])
def test_one_rerounding_is_unbiased(v):
    F = threshold(v)
    up = oracle.e8_value(oracle.e8_round(v, 0))
    down = oracle.e8_value(oracle.e8_round(v, TWO32 - 1))
    assert abs(down) <= abs(v) <= abs(up)
    gap = Fraction(up) - Fraction(down)
    e = Fraction(down) + gap * Fraction(F, TWO32)
    assert abs(e - Fraction(v)) <= abs(gap) / TWO32
    # neighbours on the grid: powers of two one apart, or 0 and 2^-126
    if down != 0:
        assert up == 2 * down
    else:
        assert abs(up) == 2.0 ** -126


def test_pair_reduction_special_cases():
    d = 40
    rng = np.random.default_rng(1)
    a = rng.integers(0, 256, size=d).astype(np.uint8)
    assert np.array_equal(
        np.vectorize(oracle.e8_value)(oracle.e8_reduce_pair(a, a, 7, 1, 0)),
        np.vectorize(oracle.e8_value)(a))                  # average of equal codes
    neg = a ^ np.uint8(0x80)
    z = oracle.e8_reduce_pair(a, neg, 7, 1, 0)
    assert not np.vectorize(oracle.e8_value)(z).any()      # opposite codes cancel
    k = np.arange(1, 41, dtype=np.uint8)                   # 2^(1-k) with 0 -> 2^-k exactly
    h = oracle.e8_reduce_pair(k, np.zeros(d, np.uint8), 3, 2, 5)
    assert np.array_equal(h, k + 1)


def _leaf_dist(xv, N):
    """[(value, probability)] of the quantized leaf of one coordinate."""
    pre, sigma, _ = oracle.scale_params(N, 1, 127, oracle.SCHEME_E)
    t = np.float32(np.float32(abs(np.float32(xv)) * pre) * sigma)
    t = min(float(t), 1.0)
    up = oracle.e8_value(oracle.e8_round(t, 0))
    down = oracle.e8_value(oracle.e8_round(t, TWO32 - 1))
    F = threshold(t)
    s = -1.0 if np.signbit(np.float32(xv)) else 1.0
    out = [(s * up, Fraction(F, TWO32)), (s * down, 1 - Fraction(F, TWO32))]
    return [(v, p) for v, p in out if p]


def _round_dist(v):
    up = oracle.e8_value(oracle.e8_round(v, 0))
    down = oracle.e8_value(oracle.e8_round(v, TWO32 - 1))
    F = threshold(v)
    out = [(up, Fraction(F, TWO32)), (down, 1 - Fraction(F, TWO32))]
    return [(u, p) for u, p in out if p]


def _tree_dist(leaves):
    """Exact distribution of the root of the averaging tree with re-rounding."""
    level = leaves
    while len(level) > 1:
        nxt = []
        for a, b in zip(level[0::2], level[1::2]):
            dist = {}
            for (va, pa), (vb, pb) in itertools.product(a, b):
                for vr, pr in _round_dist(0.5 * (va + vb)):
                    dist[vr] = dist.get(vr, 0) + pa * pb * pr
            nxt.append(list(dist.items()))
        level = nxt
    return level[0]


@pytest.mark.parametrize("n", [2, 4])
def test_tree_matches_exact_path_enumeration(n):
    x = np.array([[0.61], [-0.23], [0.9], [0.05]][:n], np.float32)
    N, _ = oracle.global_norm(x, 2, 2)
    root = _tree_dist([_leaf_dist(x[i, 0], N) for i in range(n)])
    assert sum(p for _, p in root) == 1
    ev = sum(Fraction(v) * p for v, p in root)
    truth = sum(Fraction(float(x[i, 0])) for i in range(n)) / n / Fraction(float(N))
    assert abs(float(ev - truth)) < 1e-6 * abs(float(truth))   # unbiased (fp32 scale bound)
    # the sampled tree follows that distribution (chi-square over the support)
    seeds = 4000
    xs = np.repeat(x, 8, axis=1)  # 8 coordinates share one Philox block per seed
    counts = {}
    for seed in range(seeds):
        r = oracle.e8_tree(oracle.e8_quantize(xs, N, seed), seed)
        for c in r:
            v = oracle.e8_value(int(c))
            counts[v] = counts.get(v, 0) + 1
    tot = seeds * 8
    assert set(counts) <= {v for v, _ in root}
    chi2 = sum((counts.get(v, 0) - tot * float(p)) ** 2 / (tot * float(p)) for v, p in root)
    assert chi2 < 30 + 3 * len(root)


def test_pipeline_pieces_compose_and_power_of_two_only():
    x = wl.random_rows(4, 100, seed=6)
    N, root, mean = oracle.e8_compress_mean(x, 2, 2, seed=3)
    codes = oracle.e8_quantize(x, N, 3)
    assert np.array_equal(oracle.e8_tree(codes, 3), root)
    l1a = oracle.e8_reduce_pair(codes[0], codes[1], 3, 1, 0)
    l1b = oracle.e8_reduce_pair(codes[2], codes[3], 3, 1, 1)
    assert np.array_equal(oracle.e8_reduce_pair(l1a, l1b, 3, 2, 0), root)
    assert np.array_equal(mean, (float(N) * np.vectorize(oracle.e8_value)(root)).astype(np.float32))
    with pytest.raises(ValueError):
        oracle.e8_tree(np.zeros((3, 8), np.uint8), 0)
    assert np.array_equal(oracle.e8_tree(codes[:1], 3), codes[0])


def test_quantize_matches_the_fixed_point_exponential_levels():
    # for |x|/N >= 2^-30 the 8-bit format and the fixed-point codes (s = 31)
    # pick the same level with the same uniforms
    x = (wl.random_rows(3, 500, seed=2) * np.float32(0.3)).astype(np.float32)
    N, _ = oracle.global_norm(x, 2, 2)
    c8 = np.vectorize(oracle.e8_value)(oracle.e8_quantize(x, N, 11))
    cf = oracle.quantize(x, N, 31, oracle.SCHEME_E, 11) / 2.0 ** 30
    big = np.abs(x) / float(N) >= 2.0 ** -29
    assert big.sum() > 1000 and np.array_equal(c8[big], cf[big])


def test_rerounding_variance_grows_like_one_plus_log2_n():
    # measured property of this reading of the tree: every level adds about as
    # much variance to the mean as the initial quantization (iid workers)
    rng = np.random.default_rng(0)
    n, d = 8, 128
    x = rng.standard_normal((n, d)).astype(np.float32)
    N, _ = oracle.global_norm(x, 2, 2)
    xbar = x.astype(np.float64).mean(0)
    val = np.vectorize(oracle.e8_value)
    once, tree = [], []
    for seed in range(150):
        codes = oracle.e8_quantize(x, N, seed)
        once.append((((val(codes) * float(N)).mean(0) - xbar) ** 2).sum())
        tree.append(((val(oracle.e8_tree(codes, seed)) * float(N) - xbar) ** 2).sum())
    ratio = np.mean(tree) / np.mean(once)
    assert 3.0 < ratio < 5.0  # 1 + log2(8) = 4, far above (9/8)^3 = 1.42


def test_column_pipeline_equals_whole_pipeline():
    x = wl.random_rows(8, 300, seed=12, scale=0.4)
    N, root, mean = oracle.e8_compress_mean(x, 2, 2, seed=21)
    cols = np.array([0, 7, 8, 150, 299])
    r2, m2 = oracle.e8_compress_cols(x, N, 21, cols)
    assert np.array_equal(r2, root[cols]) and np.array_equal(m2, mean[cols])

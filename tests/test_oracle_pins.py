"""Pins of the CPU oracle to facts fixed outside it (CPU only).

Each test checks the oracle against something it does not compute itself:
published known-answer values, library routines, closed forms, brute force
on tiny inputs, exact enumeration with rationals, or the worked example of
"Global-QSGD: Practical Floatless Quantization for Distributed Learning with
Theoretical Guarantees".  A dropped term, a wrong sign or index, a swapped
comparison or a transposed operand in the oracle fails at least one of them.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle import SCHEME_E, SCHEME_L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
INF = math.inf
TWO32 = 1 << 32


# ---------------------------------------------------------------------------
# Philox4x32-10: published known answers (SC'11 reference implementation)

def _kat_rows():
    rows = []
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                w = [int(t, 16) for t in line.split()]
                rows.append((w[0:4], w[4:6], w[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expect", _kat_rows())
def test_philox_known_answers(ctr, key, expect):
    assert list(oracle.philox4x32_10(ctr, key)) == expect


def test_uniform_halves_are_uniform_and_distinct():
    # chi-square on the top byte of the high and low 16-bit halves, across
    # elements of one row, and pairwise distinctness across workers and seeds
    us = np.array([oracle.uniform32(7, 0, j) for j in range(1 << 14)], dtype=np.uint64)
    for part in (us >> 24, (us >> 8) & 0xFF):
        counts = np.bincount(part.astype(np.int64), minlength=256)
        exp = us.size / 256
        chi2 = float(((counts - exp) ** 2 / exp).sum())
        assert chi2 < 360.0  # 255 dof: p ~ 1e-4 threshold
    a = [oracle.uniform32(7, 0, j) for j in range(64)]
    b = [oracle.uniform32(7, 1, j) for j in range(64)]
    c = [oracle.uniform32(8, 0, j) for j in range(64)]
    assert len(set(a)) == 64 and set(a).isdisjoint(b) and set(a).isdisjoint(c)


def test_uniform_consumes_both_draws_of_a_block():
    # the 8 elements of a block use 8 different 16-bit halves of draw A (high
    # halves of u) and of draw B (low halves); every half appears once
    ctrA = [0, 0, 3, 0]
    ctrB = [0, 0, 3, 1]
    A = oracle.philox4x32_10(ctrA, [5, 0])
    B = oracle.philox4x32_10(ctrB, [5, 0])
    halvesA = sorted(int(w >> (16 * h)) & 0xFFFF for w in A for h in (0, 1))
    halvesB = sorted(int(w >> (16 * h)) & 0xFFFF for w in B for h in (0, 1))
    us = [oracle.uniform32(5, 3, j) for j in range(8)]
    assert sorted(u >> 16 for u in us) == halvesA
    assert sorted(u & 0xFFFF for u in us) == halvesB


# ---------------------------------------------------------------------------
# (q,p)-norm, Sec. 2: library routines and closed forms

def _fsum_sq(v):
    return math.fsum(float(t) * float(t) for t in v)


@pytest.mark.parametrize("n,d", [(1, 1), (3, 17), (4, 1000), (7, 333)])
def test_norm_matches_exactly_rounded_reference(n, d):
    x = wl.random_rows(n, d, seed=n * 100 + d, scale=0.37)
    rows = [x[i].astype(np.float64) for i in range(n)]
    ref = {
        (2.0, 2.0): math.sqrt(math.fsum(_fsum_sq(r) for r in rows)),
        (2.0, INF): math.sqrt(max(_fsum_sq(r) for r in rows)),
        (INF, INF): max(float(np.abs(r).max()) for r in rows),
        (INF, 2.0): math.sqrt(math.fsum(float(np.abs(r).max()) ** 2 for r in rows)),
    }
    for (q, p), v in ref.items():
        N, _ = oracle.global_norm(x, q, p)
        assert N == np.float32(v), (q, p)
    # and numpy's own norm of the flattened vector for q = p = 2
    N22, _ = oracle.global_norm(x, 2, 2)
    assert abs(float(N22) - np.linalg.norm(x.astype(np.float64).ravel())) <= 1e-7 * float(N22)


def test_norm_closed_forms():
    n, d = 5, 12
    ones = np.ones((n, d), np.float32)
    assert oracle.global_norm(ones, 2, 2)[0] == np.float32(math.sqrt(n * d))
    assert oracle.global_norm(ones, 2, INF)[0] == np.float32(math.sqrt(d))
    assert oracle.global_norm(ones, INF, INF)[0] == np.float32(1.0)
    assert oracle.global_norm(ones, INF, 2)[0] == np.float32(math.sqrt(n))
    assert oracle.global_norm(np.array([[3.0, -4.0]], np.float32), 2, 2)[0] == np.float32(5.0)
    # rows [3,4] and [0,-12]: (2,2)-norm 13, (2,inf)-norm 12, (inf,2)-norm sqrt(4^2 + 12^2)
    x = np.array([[3.0, 4.0], [0.0, -12.0]], np.float32)
    assert oracle.global_norm(x, 2, 2)[0] == np.float32(13.0)
    assert oracle.global_norm(x, 2, INF)[0] == np.float32(12.0)
    assert oracle.global_norm(x, INF, 2)[0] == np.float32(math.sqrt(160.0))
    assert oracle.global_norm(np.zeros((2, 3), np.float32), 2, 2)[0] == 0.0


def test_norm_widens_bf16_exactly():
    torch = pytest.importorskip("torch")
    x = wl.random_rows(3, 50, seed=11, dtype="bf16", scale=3.0)
    ref32 = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    for q, p in [(2, 2), (2, INF), (INF, INF), (INF, 2)]:
        assert oracle.global_norm(x, q, p)[0] == oracle.global_norm(ref32, q, p)[0]


# ---------------------------------------------------------------------------
# Code width: the exact sum of n codes in [-M, M] must fit

def _brute_min_bits(n, M):
    for W in range(1, 64):
        if -(1 << (W - 1)) <= -n * M and n * M <= (1 << (W - 1)) - 1:
            return W


def test_min_code_bits_configs_and_brute_force():
    # the five workloads: 6, 11, 13, 8, 9 bits (the GPT-2-medium one is
    # ceil(log2(8*15+1))+1 = 8)
    got = [oracle.min_code_bits(w.n, w.s, SCHEME_L if w.scheme == "L" else SCHEME_E)
           for w in wl.WORKLOADS.values()]
    assert got == [6, 11, 13, 8, 9]
    for n in (1, 2, 3, 7, 8, 64, 1000):
        for s in (1, 2, 3, 7, 15, 127, 255):
            assert oracle.min_code_bits(n, s, SCHEME_L) == _brute_min_bits(n, s)
        for s in range(1, 12):
            assert oracle.min_code_bits(n, s, SCHEME_E) == _brute_min_bits(n, 1 << (s - 1))


# ---------------------------------------------------------------------------
# Packing: library routines for byte-multiple widths, brute force otherwise

def _brute_pack_row(codes, W):
    bits = []
    for c in codes:
        f = int(c) & ((1 << W) - 1)
        bits.extend((f >> b) & 1 for b in range(W))
    nbytes = ((len(bits) + 127) // 128) * 16
    out = bytearray(nbytes)
    for k, b in enumerate(bits):
        if b:
            out[k // 8] |= 1 << (k % 8)
    return bytes(out)


@pytest.mark.parametrize("W", [8, 16, 32])
def test_pack_byte_widths_equal_plain_integer_arrays(W):
    rng = np.random.default_rng(W)
    lim = (1 << (W - 1)) - 1
    codes = rng.integers(-lim, lim + 1, size=(3, 37)).astype(np.int32)
    packed = oracle.pack(codes, W)
    np_t = {8: np.int8, 16: np.int16, 32: np.int32}[W]
    for i in range(3):
        raw = codes[i].astype(np_t).tobytes()
        assert packed[i, :len(raw)].tobytes() == raw
        assert not packed[i, len(raw):].any()


@pytest.mark.parametrize("W", list(range(2, 33)))
def test_pack_brute_force_and_roundtrip(W):
    rng = np.random.default_rng(100 + W)
    lim = (1 << (W - 1)) - 1
    for d in (1, 5, 32, 33, 70):
        codes = rng.integers(-lim - 1 if W < 32 else -lim, lim + 1, size=(2, d)).astype(np.int32)
        packed = oracle.pack(codes, W)
        for i in range(2):
            assert packed[i].tobytes() == _brute_pack_row(codes[i], W)
        assert np.array_equal(oracle.unpack(packed, 2, d, W), codes)


# ---------------------------------------------------------------------------
# Levels and rounding, Sec. 3: deterministic cases

def test_L_exact_levels_are_deterministic():
    s, n = 7, 1
    N = np.float32(7.0)  # sigma = s / N = 1, so t = |x| exactly
    for k in range(s + 1):
        for sign in (1.0, -1.0):
            lo, hi, F = oracle.bracket(sign * k, N, n, s, SCHEME_L)
            assert (lo, F) == (k, 0)
            for u in (0, 1, 12345, TWO32 - 1):
                assert oracle.code(sign * k, N, n, s, SCHEME_L, u) == int(sign * k)


def test_E_exact_levels_are_deterministic():
    s, n = 8, 1
    N = np.float32(1.0)  # sigma = 1, r = |x|
    for k in range(s):
        x = 2.0 ** -k
        lo, hi, F = oracle.bracket(x, N, n, s, SCHEME_E)
        assert (lo, F) == (1 << (s - 1 - k), 0)
        for u in (0, 99, TWO32 - 1):
            assert oracle.code(-x, N, n, s, SCHEME_E, u) == -(1 << (s - 1 - k))


def test_max_element_under_inf_norm_is_top_level():
    x = np.array([[0.25, -3.0, 1.0], [2.5, 0.0, -0.5]], np.float32)
    for scheme, s in ((SCHEME_L, 5), (SCHEME_E, 6)):
        N, _ = oracle.global_norm(x, INF, INF)
        codes = oracle.quantize(x, N, s, scheme, seed=3)
        assert codes[0, 1] == -oracle.top_code(s, scheme)
        assert np.abs(codes).max() <= oracle.top_code(s, scheme)


def test_zeros_signed_zero_and_zero_norm():
    x = np.array([[0.0, -0.0, 1.0, -2.0]], np.float32)
    N, _ = oracle.global_norm(x, 2, 2)
    for seed in range(20):
        c = oracle.quantize(x, N, 3, SCHEME_L, seed)
        assert c[0, 0] == 0 and c[0, 1] == 0
    z = np.zeros((3, 9), np.float32)
    z[1, 4] = -0.0
    for scheme in (SCHEME_L, SCHEME_E):
        N, sums, mean = oracle.compress_mean(z, 4, 2, 2, scheme, seed=1)
        assert N == 0 and not sums.any() and not mean.any()


def test_denormal_inputs_and_tiny_norm():
    # all-denormal input: N < 2^-64, so the exact 2^64 pre-scale keeps sigma finite;
    # values equal to N map to the top level
    tiny = np.float32(1e-41)
    x = np.array([[tiny, -tiny, 0.0]], np.float32)
    N, _ = oracle.global_norm(x, INF, INF)
    assert N == tiny
    pre, sigma, _ = oracle.scale_params(N, 1, 5, SCHEME_L)
    assert pre == np.float32(2.0 ** 64) and np.isfinite(sigma)
    c = oracle.quantize(x, N, 5, SCHEME_L, seed=0)
    assert list(c[0]) == [5, -5, 0]
    c = oracle.quantize(x, N, 5, SCHEME_E, seed=0)
    assert list(c[0]) == [16, -16, 0]


# ---------------------------------------------------------------------------
# Unbiasedness (Definitions 2.1/2.2, lemma of Sec. 3): exact enumeration

def _exact_value(m, N, s, scheme):
    M = s if scheme == SCHEME_L else 1 << (s - 1)
    return Fraction(float(N)) * m / M


@pytest.mark.parametrize("scheme,s,q,p", [(SCHEME_L, 3, 2, 2), (SCHEME_L, 7, 2, INF),
                                          (SCHEME_E, 4, 2, 2), (SCHEME_E, 3, INF, INF),
                                          (SCHEME_L, 1, INF, 2)])
def test_unbiased_by_enumeration(scheme, s, q, p):
    x = np.array([[0.3, -1.7, 0.01], [2.2, -0.05, 0.9], [0.0, 1.1, -0.6]], np.float32)
    n, d = x.shape
    N, _ = oracle.global_norm(x, q, p)
    br = [[oracle.bracket(x[i, j], N, n, s, scheme) for j in range(d)] for i in range(n)]
    for j in range(d):
        # every up/down outcome of the n coordinates that form mean_j
        expect = Fraction(0)
        for outcome in itertools.product((0, 1), repeat=n):
            prob = Fraction(1)
            tot = 0
            for i, up in enumerate(outcome):
                lo, hi, F = br[i][j]
                pu = Fraction(F, TWO32)
                prob *= pu if up else 1 - pu
                m = hi if up else lo
                tot += -m if np.signbit(x[i, j]) else m
            expect += prob * _exact_value(tot, N, s, scheme) / n
        truth = sum(Fraction(float(x[i, j])) for i in range(n)) / n
        # bias allowed: fp32 rounding of sigma and of |x| sigma (2^-23 relative)
        # and the 32-bit threshold (2^-32 of one level gap per coordinate)
        slack = sum(abs(Fraction(float(x[i, j]))) for i in range(n)) * Fraction(1, 1 << 22) / n
        slack += Fraction(float(N)) * Fraction(1, 1 << 31)
        assert abs(expect - truth) <= slack


def test_round_up_frequency_matches_threshold():
    # the sampled codes pick the upper level with probability F / 2^32
    x = np.full((1, 4096), 0.3, np.float32)
    x[0, ::2] = 1.3
    N = np.float32(2.0)
    s = 4
    seeds = 40
    ups = {0.3: 0, 1.3: 0}
    tot = {0.3: 0, 1.3: 0}
    for seed in range(seeds):
        c = oracle.quantize(x, N, s, SCHEME_L, seed)
        for v in (0.3, 1.3):
            lo, hi, F = oracle.bracket(v, N, 1, s, SCHEME_L)
            sel = np.isclose(x[0], v)
            ups[v] += int((c[0, sel] == hi).sum())
            tot[v] += int(sel.sum())
    for v in (0.3, 1.3):
        lo, hi, F = oracle.bracket(v, N, 1, s, SCHEME_L)
        pr = F / TWO32
        k, m = ups[v], tot[v]
        sd = math.sqrt(m * pr * (1 - pr))
        assert abs(k - m * pr) < 5 * sd, (v, k, m * pr)


# ---------------------------------------------------------------------------
# Variance and sparsity theorem of Sec. 3 (reconstructed bounds), Monte Carlo

def omega_L(D, s):
    """QSGD bound on R^D (standard dithering, global norm <= l2 norm)."""
    return min(D / s ** 2, math.sqrt(D) / s)


def omega_E(D, s):
    """Natural/exponential dithering bound on R^D with levels 2^-k, k < s."""
    c = 2.0 ** (1 - s)
    return 1.0 / 8.0 + min(math.sqrt(D) * c, D * c * c)


def _exact_variance(x, N, s, scheme):
    n, d = x.shape
    V = Fraction(0)
    for i in range(n):
        for j in range(d):
            lo, hi, F = oracle.bracket(x[i, j], N, n, s, scheme)
            pu = Fraction(F, TWO32)
            gap = _exact_value(hi - lo, N, s, scheme)
            V += gap * gap * pu * (1 - pu)
    return V


@pytest.mark.parametrize("scheme,s,q,p", [(SCHEME_L, 2, 2, 2), (SCHEME_L, 5, INF, INF),
                                          (SCHEME_E, 3, 2, 2), (SCHEME_E, 5, 2, INF)])
def test_variance_closed_form_monte_carlo_and_bound(scheme, s, q, p):
    x = wl.random_rows(3, 40, seed=77, scale=0.5)
    n, d = x.shape
    N, _ = oracle.global_norm(x, q, p)
    V = float(_exact_variance(x, N, s, scheme))
    # Monte Carlo: squared error of the dequantized concatenated vector
    M = oracle.top_code(s, scheme)
    unit = float(N) / M
    errs = []
    for seed in range(1500):
        c = oracle.quantize(x, N, s, scheme, seed)
        errs.append(float(((c.astype(np.float64) * unit - x.astype(np.float64)) ** 2).sum()))
    errs = np.array(errs)
    assert abs(errs.mean() - V) < 5 * errs.std() / math.sqrt(errs.size)
    # the mean over workers has variance V / n^2 (independent workers)
    xsq = float((x.astype(np.float64) ** 2).sum())
    bound = (omega_L if scheme == SCHEME_L else omega_E)(n * d, s)
    assert V <= bound * xsq * (1 + 1e-6)


def test_variance_bound_nearly_tight_for_E():
    # every r at 2^e (1 + 1/3): the per-coordinate variance is r^2 / 8, the worst case
    s = 6
    r = np.float32(0.5 * (1 + 1 / 3))
    x = np.full((2, 8), r, np.float32)
    x[0, 0] = 1.0  # makes N = 1 under (inf, inf)
    N, _ = oracle.global_norm(x, INF, INF)
    V = float(_exact_variance(x, N, s, SCHEME_E))
    xsq = float((x.astype(np.float64) ** 2).sum())
    assert V <= omega_E(16, s) * xsq
    assert V >= 0.9 * (xsq - 1.0) / 8.0


def test_sparsity_expectation_and_bound():
    s = 2
    x = wl.random_rows(2, 500, seed=5)
    n, d = x.shape
    N, _ = oracle.global_norm(x, 2, 2)
    E0 = 0.0
    for i in range(n):
        for j in range(d):
            lo, hi, F = oracle.bracket(x[i, j], N, n, s, SCHEME_L)
            E0 += 1.0 if lo >= 1 else F / TWO32
    nnz = [int((oracle.quantize(x, N, s, SCHEME_L, seed) != 0).sum()) for seed in range(300)]
    nnz = np.array(nnz, np.float64)
    assert abs(nnz.mean() - E0) < 5 * nnz.std() / math.sqrt(nnz.size) + 1e-9
    D = n * d
    assert E0 <= s * s + s * math.sqrt(D)


# ---------------------------------------------------------------------------
# Reduction property (lemma of Sec. 3: n workers behave as one vector of nd)

@pytest.mark.parametrize("q", [2.0, INF])
@pytest.mark.parametrize("scheme,s", [(SCHEME_L, 5), (SCHEME_E, 6)])
def test_reduction_property(q, scheme, s):
    x = wl.random_rows(4, 30, seed=21, scale=0.2)
    n, d = x.shape
    Ng, _ = oracle.global_norm(x, q, q)
    N1, _ = oracle.global_norm(x.reshape(1, n * d), q, q)
    assert Ng == N1
    for i in range(n):
        for j in range(d):
            assert oracle.bracket(x[i, j], Ng, n, s, scheme)[:3] == \
                oracle.bracket(x.reshape(-1)[i * d + j], N1, 1, s, scheme)[:3]


def test_single_worker_global_equals_local_qsgd():
    x = wl.random_rows(1, 300, seed=8)
    s = 3
    N, sums, mean = oracle.compress_mean(x, s, 2, 2, SCHEME_L, seed=9)
    norms, codes, lmean = oracle.qsgd_local_mean(x, s, seed=9)
    assert norms[0] == N
    assert np.array_equal(codes[0].astype(np.int64), sums)
    assert np.array_equal(lmean, mean)


# ---------------------------------------------------------------------------
# Dequantization and the pipeline

def test_mean_is_exact_rational_rounded():
    x = wl.random_rows(5, 64, seed=31)
    for scheme, s in ((SCHEME_L, 9), (SCHEME_E, 7)):
        N, sums, mean = oracle.compress_mean(x, s, 2, 2, scheme, seed=4)
        M = oracle.top_code(s, scheme)
        for j in range(64):
            exact = Fraction(float(N)) * int(sums[j]) / (5 * M)
            got = Fraction(float(mean[j]))
            ulp = Fraction(float(np.spacing(np.float32(abs(float(exact))) or np.float32(1e-45))))
            assert abs(got - exact) <= ulp


def test_pipeline_pieces_compose():
    x = wl.random_rows(6, 129, seed=2, scale=3.0)
    s, scheme, seed = 11, SCHEME_L, 12
    N, sums, mean = oracle.compress_mean(x, s, 2, INF, scheme, seed)
    codes = oracle.quantize(x, N, s, scheme, seed)
    W = oracle.min_code_bits(6, s, scheme)
    back = oracle.unpack(oracle.pack(codes, W), 6, 129, W)
    assert np.array_equal(back, codes)
    assert np.array_equal(oracle.sum_codes(codes), sums)
    assert np.array_equal(oracle.dequantize(sums, 6, N, s, scheme), mean)
    cols = np.array([0, 5, 128, 64])
    cs, cm = oracle.compress_mean_cols(x, N, s, scheme, seed, cols)
    assert np.array_equal(cs, sums[cols]) and np.array_equal(cm, mean[cols])


def test_bf16_pipeline_equals_widened_fp32():
    xb = wl.random_rows(3, 80, seed=3, dtype="bf16", scale=0.1)
    xf = wl.bf16_bits_to_f32(xb)
    a = oracle.compress_mean(xb, 15, 2, 2, SCHEME_L, seed=5)
    b = oracle.compress_mean(xf, 15, 2, 2, SCHEME_L, seed=5)
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


# ---------------------------------------------------------------------------
# Worked example of Sec. 4 pins the exponential-dithering bound's form

def test_worked_example_sec4():
    vals = {}
    with open(os.path.join(GOLDEN, "worked_example_sec4.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    n, d = vals["n"], vals["d"]
    s = (1 << vals["level_bits"]) - 1  # 2^7 codes: level 0 and 2^-k, k = 0..s-1
    # the page's factor is 1 + n^0.17 * omega_E(n d): the bound used above on R^{nd}
    printed = n ** 1.17 * (1 / (8 * n) + math.sqrt(d) / (math.sqrt(n) * 2.0 ** (s - 1)))
    assert printed == pytest.approx(n ** 0.17 * omega_E(n * d, s), rel=1e-12)
    assert round(100 * printed) == vals["iteration_increase_pct"]
    assert 100 * (1 - vals["bits_sent"] / vals["bits_dense"]) == vals["communication_saved_pct"]


# ---------------------------------------------------------------------------
# The synthetic inputs are reproducible and prefix-stable

@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_workload_prefix_stable(key):
    w = wl.WORKLOADS[key]
    a = wl.generate(w, d=3000, threads=1)
    b = wl.generate(w, d=1000, threads=2)
    assert a.shape == (w.n, 3000)
    assert np.array_equal(a[:, :1000], b)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 7
    v[:4] = [0.0, -0.0, 1e-40, 3.0e38]
    ours = wl.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# Rounding of the scale can push |x| sigma above the top level: the clamp

def _find_overshooting_norm(s):
    # a norm N for which fp32(N * fp32(s / N)) > s, found by search
    rng = np.random.default_rng(s)
    for v in rng.uniform(0.5, 4.0, size=200000).astype(np.float32):
        sig = np.float32(s / float(v))
        if np.float32(v * sig) > np.float32(s):
            return v
    raise AssertionError("no overshooting norm found")


@pytest.mark.parametrize("s", [3, 7, 127])
def test_top_level_clamp(s):
    N = _find_overshooting_norm(s)
    lo, hi, F = oracle.bracket(N, N, 1, s, SCHEME_L)
    assert (lo, F) == (s, 0)
    x = np.array([[N, -N, 0.5 * N]], np.float32)
    for seed in range(10):
        c = oracle.quantize(x, N, s, SCHEME_L, seed)
        assert c[0, 0] == s and c[0, 1] == -s
    # a NaN coordinate stays on the grid too
    c = oracle.quantize(np.array([[np.nan, 1.0]], np.float32), np.float32(1.0), s, SCHEME_L, 0)
    assert abs(int(c[0, 0])) <= s


# ---------------------------------------------------------------------------
# Local-norm QSGD ablation with several workers

def test_local_qsgd_exact_levels_give_the_exact_mean():
    # row norms 5 and 13 with s = 5 and s = 13 multiples: every |x|/N_i * s is an integer
    x = np.array([[3.0, -4.0, 0.0], [0.0, 5.0, -12.0]], np.float32)
    s = 65  # both 3/5, 4/5 and 5/13, 12/13 land on multiples of 1/65
    norms, codes, mean = oracle.qsgd_local_mean(x, s, seed=1)
    assert list(norms) == [5.0, 13.0]
    assert codes.tolist() == [[39, -52, 0], [0, 25, -60]]
    assert np.array_equal(mean, x.mean(axis=0))


def test_local_qsgd_unbiased_monte_carlo():
    x = wl.random_rows(4, 6, seed=19)
    s = 2
    means = np.array([oracle.qsgd_local_mean(x, s, seed)[2] for seed in range(3000)], np.float64)
    truth = x.astype(np.float64).mean(axis=0)
    se = means.std(axis=0) / math.sqrt(means.shape[0])
    assert np.all(np.abs(means.mean(axis=0) - truth) < 5 * se + 1e-7)


def test_row_parallel_norm_equals_whole_norm():
    x = wl.random_rows(6, 999, seed=44)
    for q, p in [(2, 2), (2, INF), (INF, INF), (INF, 2)]:
        a = oracle.global_norm(x, q, p)
        b = oracle.global_norm_rows(x, q, p, threads=3)
        assert a[0] == b[0] and np.array_equal(a[1], b[1])


def test_local_ablation_pieces_compose():
    x = wl.random_rows(5, 301, seed=45)
    norms, codes, mean = oracle.qsgd_local_mean(x, 4, seed=2)
    assert np.array_equal(oracle.local_norms(x, threads=2), norms)
    cols = np.array([0, 17, 300, 150])
    c2, m2 = oracle.qsgd_local_cols(x, norms, 4, 2, cols)
    assert np.array_equal(c2, codes[:, cols]) and np.array_equal(m2, mean[cols])


# ---------------------------------------------------------------------------
# General real orders (Sec. 2 allows p in (1, inf) and inf)

@pytest.mark.parametrize("q,p", [(1.0, 1.0), (1.5, 3.0), (3.0, INF), (INF, 1.5), (2.0, 4.0),
                                 (7.25, 2.0), (1.0, INF)])
def test_general_orders_against_numpy(q, p):
    x = wl.random_rows(5, 200, seed=int(10 * min(q, 99.0) + p if p < INF else 3), scale=0.3)
    N, _ = oracle.global_norm(x, q, p)
    xr = x.astype(np.float64)
    w = np.array([np.linalg.norm(xr[i], ord=q) for i in range(5)])
    ref = np.linalg.norm(w, ord=p)
    assert abs(float(N) - ref) <= 2 ** -23 * ref  # one fp32 rounding of a ~1e-15-accurate value


def test_general_orders_closed_forms():
    x = np.array([[3.0, -4.0, 0.0], [1.0, 1.0, -2.0]], np.float32)
    assert oracle.global_norm(x, 1.0, 1.0)[0] == np.float32(11.0)       # sum of |x|
    assert oracle.global_norm(x, 1.0, INF)[0] == np.float32(7.0)        # max row l1
    assert oracle.global_norm(x, INF, 1.0)[0] == np.float32(6.0)        # 4 + 2
    assert oracle.global_norm(x, 3.0, 3.0)[0] == np.float32((27 + 64 + 1 + 1 + 8) ** (1 / 3))
    # the {2, inf} pairs keep their exact forms
    assert oracle.global_norm(x, 2.0, 2.0)[0] == np.float32(math.sqrt(31.0))
    # norms decrease with the order
    y = wl.random_rows(3, 50, seed=3)
    vals = [float(oracle.global_norm(y, q, q)[0]) for q in (1.0, 1.5, 2.0, 3.0, 8.0, INF)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))

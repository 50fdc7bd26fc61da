"""GPU parity of the zero-code skip in the word layout (gq_norm_term_bounds,
gq_compress_words_skip): the per-device step of the sharded path, where a
device sums its own workers' codes into uint32 words for the integer
all-reduce.

The skip changes which coordinates are read, never what is computed, so
each case checks the skipped word row against the oracle's word-wise sum of
its packed codes and against the same pass reading every coordinate
(gq_compress_words_from_norm), bit for bit; the bounds against numpy's
rounding-up of each span's largest |x|; and the term against gq_norm_term.
Cases cover every fields-per-word count, both accumulators of bf16
standard dithering, more than 64 rows on one device, shards at non-zero
worker offsets whose sums add up to the whole, inf and NaN inputs, norms
below 2^-64, and all-zero rows.
"""
import math
import sys
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import allreduce_compatible_gradient_amd as gq  # noqa: E402
import oracle  # noqa: E402
import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu
SCH = {"L": oracle.SCHEME_L, "E": oracle.SCHEME_E}
DEV = "cuda:0"
INF = math.inf


def log(msg):
    print(f"[gpu-words-skip {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def words_host(t):
    return host(t).view(np.uint32)


def numpy_bounds(x):
    """Per (row, 512-coordinate span): the high half of max(bits & 0x7FFFFFFF)
    rounded up, bf16 inputs widened to their fp32 patterns first."""
    n, d = x.shape
    bits = (x.astype(np.uint32) << np.uint32(16)) if x.dtype == np.uint16 else x.view(np.uint32)
    spans = -(-d // 512)
    row = np.zeros((n, spans * 512), dtype=np.uint32)
    row[:, :d] = bits & np.uint32(0x7FFFFFFF)
    m = row.reshape(n, spans, 512).max(axis=2).astype(np.uint64)
    return ((m + 0xFFFF) >> 16).astype(np.uint16)


def M_of(s, scheme):
    return s if scheme == "L" else 1 << (s - 1)


def shard_words(x, xd, s, q, p, scheme, seed, W, norm, worker_base, tag):
    """One device's step on its rows xd (host copy x): term and bounds in one
    pass, then the word row with and without the skip.  Returns the skipped
    row; asserts the bounds, the term and skip == dense."""
    n, d = x.shape
    term, bounds = gq.gq_norm_term_bounds(xd, q, p)
    plain = gq.gq_norm_term(xd, q, p)
    t0, t1 = host(term)[0], host(plain)[0]
    assert t0 == t1 or (np.isnan(t0) and np.isnan(t1)), (tag, t0, t1)
    if d > 0:
        stride = -(-d // 8192) * 16
        got_b = host(bounds)[: 2 * n * stride].view(np.uint16).reshape(n, stride)[:, : -(-d // 512)]
        assert np.array_equal(got_b, numpy_bounds(x)), tag
    skip = gq.gq_compress_words_skip(xd, s, scheme, norm, bounds, seed, W,
                                     worker_base=worker_base)
    dense = gq.gq_compress_words_from_norm(xd, s, scheme, norm, seed, W, worker_base=worker_base)
    hs = words_host(skip)
    assert np.array_equal(hs, words_host(dense)), (tag, "skip vs dense")
    return hs


def check_words(x, s, q, p, scheme, seed, W, tag, worker_base=0):
    """The device holds every row: skipped row == dense row == the oracle's.
    W None: the minimal width for n rows."""
    n, d = x.shape
    if W is None:
        W = gq.gq_min_code_bits(n, s, scheme)
    xd = to_dev(x)
    norm = gq.gq_global_norm(xd, q, p)
    N = np.float32(host(norm)[0])
    got = shard_words(x, xd, s, q, p, scheme, seed, W, norm, worker_base, tag)
    if worker_base == 0:
        ocodes = oracle.quantize(x, N, s, SCH[scheme], seed)
        expect = oracle.sum_words(oracle.pack_words(ocodes, W, M_of(s, scheme)))
        assert np.array_equal(got, expect), (tag, "skip vs oracle")
        nz = np.count_nonzero(ocodes)
    else:
        nz = -1
    log(f"{tag}: n={n} d={d} {scheme} s={s} W={W} base={worker_base}: N={float(N):.4g}, "
        f"{nz} non-zero codes: bit-exact")


def make(kind, n, d, dtype, seed):
    x = wl.random_rows(n, d, seed=seed, scale=0.01)
    rng = np.random.default_rng(seed)
    if kind == "mixed":
        # a few spans of a few rows hold values near or above N / s: dense spans
        for _ in range(3):
            x[rng.integers(0, n), rng.integers(0, d)] = np.float32(50.0)
    elif kind == "heavy":
        m = rng.random((n, d)) < 0.001
        x[m] *= np.float32(100.0)
    return wl.f32_to_bf16_bits(x) if dtype == "bf16" else x


# (n, s, scheme, W): every fields-per-word count (W 2..32 gives 16, 10, 8,
# 6, 5, 4, 3, 2, 1 fields), both schemes
WORD_CASES = [
    (1, 1, "L", 2), (1, 1, "L", 3), (2, 1, "L", 4), (3, 1, "L", 5), (4, 3, "L", 6),
    (6, 3, "L", 7), (9, 7, "L", 8), (4, 15, "L", 9), (8, 127, "L", 11), (16, 8, "E", 13),
    (5, 3, "E", 16), (8, 127, "L", 17), (16, 8, "E", 24), (3, 7, "L", 32),
]


@pytest.mark.parametrize("n,s,scheme,W", WORD_CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["plain", "mixed"])
def test_words_skip_matches_oracle_and_dense(n, s, scheme, W, dtype, kind):
    assert W >= oracle.min_code_bits(n, s, SCH[scheme])
    for d in (1, 513, 6001, 20_483):
        x = make(kind, n, d, dtype, seed=n * 100 + d + W)
        check_words(x, s, 2.0, 2.0, scheme, 3 + W, W, f"{kind}/{dtype}/d={d}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_rows_on_one_device(dtype):
    """70 rows (thresholds are shared 64 rows at a time), at worker offset
    0 against the oracle and at offset 1000 against the dense pass; bf16 with
    L and a small n M takes the packed 16-bit accumulators."""
    n, d = 70, 9000
    x = make("mixed", n, d, dtype, seed=70)
    for scheme, s in (("L", 3), ("E", 5)):
        W = gq.gq_min_code_bits(n, s, scheme)
        check_words(x, s, 2.0, 2.0, scheme, 17, W, f"many/{dtype}")
        check_words(x, s, 2.0, 2.0, scheme, 17, W, f"many/{dtype}", worker_base=1000)


@pytest.mark.parametrize("scheme,s,q,p", [("L", 15, 2.0, 2.0), ("E", 8, 2.0, INF),
                                          ("L", 127, INF, INF)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shards_add_up_to_the_whole(scheme, s, q, p, dtype):
    """Three devices: each computes its term and bounds, the terms combine
    as the all-reduce of a double would, N follows from the combined term;
    each device's skipped word row at its worker offset, summed word-wise
    over the devices, is the oracle's sum over all workers at that N, and
    gq_dequantize_words of it is the oracle's mean at that N."""
    n, d = 9, 40_003
    W = gq.gq_min_code_bits(n, s, scheme)
    x = make("heavy", n, d, dtype, seed=123)
    xd = to_dev(x)
    cuts = ((0, 4), (4, 5), (5, 9))
    terms = [host(gq.gq_norm_term_bounds(xd[a:b].clone(), q, p)[0])[0] for a, b in cuts]
    comb = max(terms) if math.isinf(p) else sum(terms)  # an all-reduce of one double
    norm = gq.gq_norm_from_term(torch.tensor([comb], dtype=torch.float64, device=DEV), q, p)
    N = np.float32(host(norm)[0])
    total = np.zeros(gq.gq_word_row_bytes(d, W) // 4, dtype=np.uint64)
    for a, b in cuts:
        total += shard_words(x[a:b], xd[a:b].clone(), s, q, p, scheme, 8, W, norm, a,
                             f"shard {a}:{b}")
    total = (total & 0xFFFFFFFF).astype(np.uint32)  # a uint32 SUM wraps modulo 2^32
    M = M_of(s, scheme)
    ocodes = oracle.quantize(x, N, s, SCH[scheme], 8)
    assert np.array_equal(total, oracle.sum_words(oracle.pack_words(ocodes, W, M)))
    sums = oracle.unpack_word_sums(total, n, d, W, M)
    wt = torch.from_numpy(total.view(np.int32)).to(DEV)
    mean = host(gq.gq_dequantize_words(wt, n, d, s, scheme, W, norm))
    assert np.array_equal(mean.view(np.uint32),
                          oracle.dequantize(sums, n, N, s, SCH[scheme]).view(np.uint32))
    log(f"shards {scheme} s={s} q={q} p={p} {dtype}: N={float(N):.6g}, "
        f"{np.count_nonzero(sums)} non-zero sums: bit-exact")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_non_finite_tiny_and_zero_rows(dtype):
    """NaN and inf make their spans dense; a norm below 2^-64 takes the exact
    pre-scale in the thresholds as in the codes; all-zero rows give the bias
    only; a scaled sigma that overflows fp32 reads everything."""
    n, d = 3, 5000
    x = wl.random_rows(n, d, seed=4, scale=1e-3)
    x[1, 700] = np.float32(np.nan)
    x[2, 4099] = np.float32(-np.nan)
    xb = wl.f32_to_bf16_bits(x) if dtype == "bf16" else x
    check_words(xb, 7, INF, INF, "L", 5, None, f"nan/{dtype}")
    check_words(xb, 8, INF, 2.0, "E", 6, 11, f"nan-E/{dtype}")
    y = x.copy()
    y[np.isnan(y)] = 0.0
    y[0, 3] = np.float32(np.inf)
    yb = wl.f32_to_bf16_bits(y) if dtype == "bf16" else y
    check_words(yb, 7, INF, INF, "L", 7, None, f"inf/{dtype}")
    scale = 1e-41 if dtype == "f32" else 1e-39
    rng = np.random.default_rng(31)
    t = (rng.standard_normal((3, 3001)) * scale).astype(np.float32)
    tb = wl.f32_to_bf16_bits(t) if dtype == "bf16" else t
    check_words(tb, 7, 2.0, 2.0, "L", 4, None, f"tiny-L/{dtype}")
    check_words(tb, 9, 2.0, 2.0, "E", 4, None, f"tiny-E/{dtype}")
    z = np.zeros((4, 3000), dtype=np.float32)
    check_words(wl.f32_to_bf16_bits(z) if dtype == "bf16" else z, 7, 2.0, 2.0, "L", 1, None,
                f"zeros/{dtype}")
    o = np.zeros((1, 600), dtype=np.float32)
    o[0, [3, 300, 599]] = np.float32(2.0 ** -149) * np.array([1, -1, 1], dtype=np.float32)
    check_words(o, 31, 2.0, 2.0, "E", 8, 32, "sigma-overflow")


def test_int_accumulator():
    """n M > 2^24 (E, s = 16, 600 rows): one field per word, the int32
    accumulator, with the skip."""
    x = make("mixed", 600, 2500, "f32", seed=600)
    check_words(x, 16, 2.0, 2.0, "E", 9, None, "int-acc")


def test_empty_rows_and_rejects():
    xd = torch.zeros((3, 0), dtype=torch.float32, device=DEV)
    term, bounds = gq.gq_norm_term_bounds(xd, 2.0, 2.0)
    assert host(term)[0] == 0.0
    norm = torch.zeros(1, dtype=torch.float32, device=DEV)
    assert gq.gq_compress_words_skip(xd, 7, "L", norm, bounds, 1, 6).numel() == 0
    x = torch.zeros((2, 1000), dtype=torch.float32, device=DEV)
    nb = gq.gq_span_bounds_bytes(2, 1000)
    big = torch.zeros(nb + 16, dtype=torch.uint8, device=DEV)
    _, b = gq.gq_norm_term_bounds(x, 2.0, 2.0, bounds=big[:nb])
    with pytest.raises(gq.GQError):
        gq.gq_compress_words_skip(x, 7, "L", norm, big[2:2 + nb], 1, 6)  # not 16-byte aligned
    with pytest.raises(gq.GQError):
        gq.gq_compress_words_skip(x, 7, "L", norm, b, 1, 4)  # W below the width rule
    with pytest.raises(gq.GQError):
        gq.gq_norm_term_bounds(x, 2.0, 2.0, bounds=big[2:2 + nb])
    torch.cuda.synchronize()

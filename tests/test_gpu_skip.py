"""GPU parity of the zero-code skip (gq_global_norm_bounds, gq_compress_mean_skip
and gq_compress_mean with its full workspace).

The skip changes which coordinates the fused pass reads, never what it
computes, so every case is checked three ways: against the CPU oracle,
against the same pass reading every coordinate (gq_compress_mean_from_norm),
and -- for the span bounds themselves -- against the bf16 rounding-up of each
span's largest |x| computed in numpy.  Cases aim at the skip's own edges:
spans where some t reaches the first level (dense) beside sparse ones, inf
and NaN inputs, more than 64 workers (thresholds are shared 64 rows at a
time), ragged rows, norms below 2^-64 (the exact pre-scale), a scaled sigma
that overflows fp32, bf16 inputs on both accumulators, code sums, and
sparse spans where most groups pass (the per-wave candidate queue filled
and drained thousands of times).
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
    print(f"[gpu-skip {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


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


def numpy_bounds(x: np.ndarray) -> np.ndarray:
    """Per (row, 512-coordinate span): the high half of max(bits & 0x7FFFFFFF)
    rounded up, bf16 inputs widened to their fp32 patterns first."""
    n, d = x.shape
    bits = (x.astype(np.uint32) << np.uint32(16)) if x.dtype == np.uint16 else x.view(np.uint32)
    spans = -(-d // 512)
    out = np.empty((n, spans), dtype=np.uint16)
    for i in range(n):
        row = np.zeros(spans * 512, dtype=np.uint32)
        row[:d] = bits[i] & np.uint32(0x7FFFFFFF)
        m = row.reshape(spans, 512).max(axis=1).astype(np.uint64)
        out[i] = ((m + 0xFFFF) >> 16).astype(np.uint16)
    return out


def check_all(x, s, q, p, scheme, seed, tag, want_sums=False, nan_mean=False):
    """nan_mean: N is inf, so the mean holds 0 * inf = NaN, whose sign bit the
    host and the device may set differently; there the mean is compared with
    the oracle's as values (NaN equal to NaN) and the code sums exactly."""
    n, d = x.shape
    N, sums, mean = oracle.compress_mean(x, s, q, p, SCH[scheme], seed)
    xd = to_dev(x)
    norm, bounds = gq.gq_global_norm_bounds(xd, q, p)
    gN = np.float32(host(norm)[0])
    assert gN == N or (np.isnan(gN) and np.isnan(N)), (tag, gN, N)
    stride = -(-d // 8192) * 16  # entries per row: the spans padded to 16
    got_b = host(bounds)[: 2 * n * stride].view(np.uint16).reshape(n, stride)[:, : -(-d // 512)]
    assert np.array_equal(got_b, numpy_bounds(x)), tag
    W = gq.gq_min_code_bits(n, s, scheme)
    skip, csum = gq.gq_compress_mean_skip(xd, s, scheme, seed, norm, bounds, code_bits=W,
                                          want_code_sum=want_sums)
    dense, dsum = gq.gq_compress_mean_from_norm(xd, s, scheme, seed, norm, code_bits=W,
                                                want_code_sum=want_sums)
    whole, wnorm, _ = gq.gq_compress_mean(xd, s, q, p, scheme, seed)
    hs, hd, hw = host(skip), host(dense), host(whole)
    if nan_mean:
        assert np.array_equal(hs, mean, equal_nan=True), (tag, "skip vs oracle")
    else:
        assert np.array_equal(hs.view(np.uint32), mean.view(np.uint32)), (tag, "skip vs oracle")
    assert np.array_equal(hd.view(np.uint32), hs.view(np.uint32)), (tag, "dense vs skip")
    assert np.array_equal(hw.view(np.uint32), hs.view(np.uint32)), (tag, "whole vs skip")
    if want_sums:
        assert np.array_equal(host(csum), oracle.pack_row(sums, W)), (tag, "code sums")
        assert np.array_equal(host(dsum), host(csum)), (tag, "dense code sums")
    dense_spans = (got_b >= 0x7F80).mean()
    log(f"{tag}: n={n} d={d} {scheme} s={s} q={q} p={p}: N={float(N):.4g}, "
        f"{np.count_nonzero(sums)} non-zero sums, inf/NaN spans {dense_spans:.3f}: bit-exact")


CASES = [
    # (n, d, dtype, scheme, s, q, p, kind)
    (4, 65_536, "f32", "L", 7, 2.0, 2.0, "plain"),
    (3, 1, "f32", "L", 7, 2.0, 2.0, "plain"),
    (5, 7, "f32", "E", 8, 2.0, 2.0, "plain"),
    (2, 511, "f32", "L", 127, 2.0, INF, "plain"),
    (2, 513, "bf16", "L", 15, 2.0, 2.0, "plain"),
    (7, 2049, "f32", "E", 8, INF, 2.0, "plain"),
    (9, 10_007, "bf16", "E", 6, 2.0, 2.0, "plain"),
    (65, 3000, "f32", "L", 3, 2.0, 2.0, "plain"),
    (130, 1030, "f32", "E", 5, 2.0, 2.0, "mixed"),
    (130, 2048, "bf16", "L", 3, 2.0, 2.0, "mixed"),
    (70, 4100, "bf16", "E", 8, INF, INF, "mixed"),
    (16, 8192, "f32", "L", 7, 2.0, 2.0, "mixed"),
    (8, 100_003, "f32", "E", 8, 2.0, 2.0, "heavy"),
    (8, 100_000, "bf16", "L", 15, 2.0, 2.0, "heavy"),
    (4, 4096, "f32", "L", 1, 2.0, 2.0, "mixed"),
    (3, 9000, "f32", "L", 127, 1.5, 3.0, "mixed"),
    (600, 2500, "f32", "E", 16, 2.0, 2.0, "mixed"),  # n M > 2^24: the int32 accumulator
    # sparse spans whose thresholds let most groups through: thousands of
    # queue entries per span, the candidate ring wrapping many times
    (200, 1030, "f32", "L", 1, 2.0, INF, "plain"),
    (200, 2048, "bf16", "L", 1, 2.0, INF, "plain"),
    (150, 700, "f32", "E", 3, 2.0, INF, "plain"),
]


def make(kind, n, d, dtype, seed):
    x = wl.random_rows(n, d, seed=seed, scale=0.01)
    if kind == "mixed":
        # a few spans of a few rows hold values near or above N / s: dense spans
        rng = np.random.default_rng(seed)
        for _ in range(3):
            i, j = rng.integers(0, n), rng.integers(0, d)
            x[i, j] = np.float32(50.0)
    elif kind == "heavy":
        # Laplace-like tails: 0.1% of entries scaled by 100
        rng = np.random.default_rng(seed)
        m = rng.random((n, d)) < 0.001
        x[m] *= np.float32(100.0)
    return wl.f32_to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("n,d,dtype,scheme,s,q,p,kind", CASES)
def test_skip_matches_oracle_and_dense(n, d, dtype, scheme, s, q, p, kind):
    x = make(kind, n, d, dtype, seed=n * 1000 + d)
    check_all(x, s, q, p, scheme, 11 + n, f"{kind}/{dtype}", want_sums=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_inf_and_nan_make_their_spans_dense(dtype):
    """A NaN lands on the top level and an inf makes N inf: the bound of
    their span must mark it dense (patterns >= 0x7F80), whatever the norm."""
    n, d = 3, 5000
    x = wl.random_rows(n, d, seed=4, scale=1e-3)
    x[1, 700] = np.float32(np.nan)
    x[2, 4099] = np.float32(-np.nan)
    xb = wl.f32_to_bf16_bits(x) if dtype == "bf16" else x
    # q = inf drops the NaN from N (fmax), so the rest of the row stays sparse
    check_all(xb, 7, INF, INF, "L", 5, f"nan/{dtype}")
    check_all(xb, 8, INF, 2.0, "E", 6, f"nan-E/{dtype}")
    y = x.copy()
    y[np.isnan(y)] = 0.0
    y[0, 3] = np.float32(np.inf)
    yb = wl.f32_to_bf16_bits(y) if dtype == "bf16" else y
    check_all(yb, 7, INF, INF, "L", 7, f"inf/{dtype}", want_sums=True, nan_mean=True)


@pytest.mark.parametrize("scheme,s", [("L", 7), ("E", 8)])
def test_tiny_norms_prescale(scheme, s):
    """N below 2^-64: |x| is pre-scaled by 2^64 before sigma, in the bounds'
    thresholds as in the codes."""
    x = (wl.random_rows(6, 3001, seed=9, scale=1.0) * np.float32(1e-38)).astype(np.float32)
    x[2, 10] = np.float32(3e-38)
    check_all(x, s, 2.0, 2.0, scheme, 3, f"tiny/{scheme}")


def test_scaled_sigma_overflow_reads_everything():
    """E with s = 31 and N near 2^-146: sigma 2^(s+15) overflows fp32, so
    every span is read (the skip is off) -- still the oracle's results."""
    x = np.zeros((1, 600), dtype=np.float32)
    x[0, [3, 300, 599]] = np.float32(2.0 ** -149) * np.array([1, -1, 1], dtype=np.float32)
    check_all(x, 31, 2.0, 2.0, "E", 8, "sigma-overflow")


def test_all_zero_and_single_worker():
    z = np.zeros((4, 3000), dtype=np.float32)
    check_all(z, 7, 2.0, 2.0, "L", 1, "zeros")
    one = wl.random_rows(1, 70_001, seed=3, scale=0.5)
    check_all(one, 127, 2.0, INF, "L", 2, "one-worker")


def check_local(x, s, seed, tag, vs_oracle=True):
    """The local-norm ablation with the zero-code skip (full workspace)
    against the same call reading every coordinate (smallest workspace) and
    the oracle: norms, per-worker codes and mean.  vs_oracle False: only the
    two device calls are compared (a worker's inf gives N_i = inf on the
    device and NaN in the oracle's compensated sum, a difference of the
    norm, not of the skip)."""
    n, d = x.shape
    onorms, ocodes, omean = oracle.qsgd_local_mean(x, s, seed)
    xd = to_dev(x)
    W = gq.gq_min_code_bits(1, s, "L")
    small = torch.empty(gq.gq_workspace_bytes(n, d), dtype=torch.uint8, device=DEV)
    skip_m, skip_n, skip_c = gq.gq_qsgd_local_mean(xd, s, seed, code_bits=W, want_codes=True)
    full_m, full_n, full_c = gq.gq_qsgd_local_mean(xd, s, seed, code_bits=W, want_codes=True,
                                                   workspace=small)
    hs, hf = host(skip_m), host(full_m)
    assert np.array_equal(hs.view(np.uint32), hf.view(np.uint32)), (tag, "skip vs every coordinate")
    assert np.array_equal(host(skip_n).view(np.uint32), host(full_n).view(np.uint32)), (tag, "norms")
    assert np.array_equal(host(skip_c), host(full_c)), (tag, "codes")
    if vs_oracle:
        assert np.array_equal(host(skip_n).view(np.uint32), onorms.view(np.uint32)), (tag, "norms")
        assert np.array_equal(host(skip_c), oracle.pack(ocodes, W)), (tag, "codes vs oracle")
        assert np.array_equal(hs.view(np.uint32), omean.view(np.uint32)), (tag, "mean vs oracle")
    log(f"ablation {tag}: n={n} d={d} s={s}: bit-exact")


@pytest.mark.parametrize("n,d,dtype,kind", [(4, 65_536, "f32", "plain"), (3, 1, "f32", "plain"),
                                            (70, 4100, "f32", "mixed"), (9, 10_007, "bf16", "heavy"),
                                            (130, 1030, "bf16", "mixed")])
def test_local_ablation_skip(n, d, dtype, kind):
    check_local(make(kind, n, d, dtype, seed=n * 77 + d), 3, 9 + n, f"{kind}/{dtype}")


def test_local_ablation_skip_edges():
    """A worker of zeros (norm 0: no codes), one with an inf (kappa_i inf:
    its zero codes add 0 * inf = NaN, so it is read whole), tiny norms."""
    x = wl.random_rows(5, 5000, seed=12, scale=1e-3)
    x[1] = 0.0
    check_local(x, 3, 4, "zero worker")
    y = x.copy()
    y[3, 17] = np.float32(np.inf)
    check_local(y, 3, 5, "inf worker", vs_oracle=False)
    z = (wl.random_rows(4, 3001, seed=13) * np.float32(1e-38)).astype(np.float32)
    check_local(z, 7, 6, "tiny norms")

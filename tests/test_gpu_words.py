"""GPU parity of the word layout for a native integer all-reduce.

floor(32 / W) fields of code + M per 32-bit word, so that a plain uint32
SUM over the rows adds every code exactly.  Bar: words, summed words and
code sums bit-exact against the oracle; the mean bit-exact against the
oracle's dequantization of the same sums (and against the fused path at
full size).  Inputs come from the seeded generators of workloads.py; only
the oracle computes expected values.
"""
import math
import os
import sys
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import allreduce_compatible_gradient_amd as gq  # noqa: E402
import oracle  # noqa: E402
import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu
INF = math.inf
SCH = {"L": oracle.SCHEME_L, "E": oracle.SCHEME_E}
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-words {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def u32(a: np.ndarray) -> torch.Tensor:
    """uint32 words to a device int32 tensor of the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(DEV)


def words_host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint32)


def M_of(s, scheme):
    return s if scheme == "L" else 1 << (s - 1)


# (n, s, scheme): the widths tried run from the minimal one up to 32, so
# that every fields-per-word count (16, 10, 8, 6, 5, 4, 3, 2, 1) occurs
SETS = [(1, 1, "L"), (3, 7, "L"), (8, 127, "L"), (16, 8, "E"), (5, 3, "E")]
WIDTHS = [2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 13, 16, 17, 24, 32]
SHAPES = [(1, 1), (3, 17), (4, 4096), (2, 6001), (5, 12290)]


def _cases():
    out = []
    for n0, s, scheme in SETS:
        Wmin = oracle.min_code_bits(n0, s, SCH[scheme])
        for W in WIDTHS:
            if W >= Wmin:
                out.append((n0, s, scheme, W))
    return out


@pytest.mark.parametrize("n0,s,scheme,W", _cases())
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_words_match_oracle(n0, s, scheme, W, dtype):
    for n, d in SHAPES:
        n = min(n, n0)
        seed = 7 * n + d + W
        x = wl.random_rows(n, d, seed=seed, dtype=dtype, scale=0.3)
        xd = to_dev(x)
        norm = gq.gq_global_norm(xd, 2.0, 2.0)
        N = np.float32(host(norm)[0])
        M = M_of(s, scheme)
        ocodes = oracle.quantize(x, N, s, SCH[scheme], seed)
        owords = oracle.pack_words(ocodes, W, M)
        gw = gq.gq_quantize_words(xd, s, scheme, norm, seed, W)
        assert np.array_equal(words_host(gw), owords), (n, d)
        # the sum and dequantization kernels take the oracle's words as input
        osum = oracle.sum_words(owords)
        gsum = gq.gq_sum_words(u32(owords), n, d, W)
        assert np.array_equal(words_host(gsum), osum), (n, d)
        sums = oracle.unpack_word_sums(osum, n, d, W, M)
        assert np.array_equal(sums, oracle.sum_codes(ocodes))
        gmean = gq.gq_dequantize_words(u32(osum), n, d, s, scheme, W, norm)
        assert np.array_equal(host(gmean), oracle.dequantize(sums, n, N, s, SCH[scheme])), (n, d)


@pytest.mark.parametrize("n0,s,scheme,W", [c for c in _cases() if c[0] > 1 or c[3] <= 4])
def test_compress_words_equals_the_summed_rows(n0, s, scheme, W):
    """One pass over a device's rows: the word-wise sum of its rows' words,
    bit-exact against the oracle, for every fields-per-word count."""
    for n, d in SHAPES:
        n = min(n, n0)
        seed = 11 * n + d + W
        x = wl.random_rows(n, d, seed=seed, scale=0.3)
        xd = to_dev(x)
        norm = gq.gq_global_norm(xd, 2.0, 2.0)
        N = np.float32(host(norm)[0])
        M = M_of(s, scheme)
        ocodes = oracle.quantize(x, N, s, SCH[scheme], seed)
        expect = oracle.sum_words(oracle.pack_words(ocodes, W, M))
        got = gq.gq_compress_words_from_norm(xd, s, scheme, norm, seed, W)
        assert np.array_equal(words_host(got), expect), (n, d)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_device_sums_add_up_to_the_whole(dtype):
    """Three devices' summed rows (their workers at their global offsets),
    added word-wise as the all-reduce would, give the sum over all workers,
    and gq_dequantize_words of it the fused path's mean."""
    n, d, s, scheme = 9, 40_003, 15, "L"
    W = gq.gq_min_code_bits(n, s, scheme)
    x = wl.random_rows(n, d, seed=123, dtype=dtype, scale=0.2)
    xd = to_dev(x)
    norm = gq.gq_global_norm(xd, 2.0, 2.0)
    parts = [words_host(gq.gq_compress_words_from_norm(xd[a:b].clone(), s, scheme, norm, 8, W,
                                                       worker_base=a))
             for a, b in ((0, 4), (4, 5), (5, 9))]
    total = (parts[0].astype(np.uint64) + parts[1] + parts[2]).astype(np.uint32)  # mod 2^32
    whole = words_host(gq.gq_compress_words_from_norm(xd, s, scheme, norm, 8, W))
    assert np.array_equal(total, whole)
    mean = gq.gq_dequantize_words(u32(total), n, d, s, scheme, W, norm)
    fmean, _, _ = gq.gq_compress_mean(xd, s, 2.0, 2.0, scheme, 8)
    assert np.array_equal(host(mean), host(fmean))


def test_zero_norm_gives_the_bias_only():
    """N = 0: every code is 0, so each field holds M and the mean is 0."""
    n, d, s, W = 3, 5000, 7, 6
    xd = torch.zeros((n, d), dtype=torch.float32, device=DEV)
    norm = gq.gq_global_norm(xd, 2.0, 2.0)
    gw = words_host(gq.gq_quantize_words(xd, s, "L", norm, 1, W))
    assert np.array_equal(gw, oracle.pack_words(np.zeros((n, d), np.int32), W, s))
    gsum = gq.gq_sum_words(u32(gw), n, d, W)
    mean = host(gq.gq_dequantize_words(gsum, n, d, s, "L", W, norm))
    assert np.all(mean == 0)


def test_shards_summed_together_reproduce_the_whole():
    """Workers quantized in shards (worker_base = their global index), the
    rows of every shard summed as one all-reduce would: the same words and
    the same mean as one call over all workers."""
    n, d, s, scheme = 7, 30_011, 127, "L"
    W = gq.gq_min_code_bits(n, s, scheme)
    x = wl.random_rows(n, d, seed=99, scale=0.1)
    xd = to_dev(x)
    norm = gq.gq_global_norm(xd, 2.0, INF)
    whole = gq.gq_quantize_words(xd, s, scheme, norm, 5, W)
    parts = [gq.gq_quantize_words(xd[a:b].clone(), s, scheme, norm, 5, W, worker_base=a)
             for a, b in ((0, 3), (3, 4), (4, 7))]
    assert np.array_equal(words_host(torch.cat(parts)), words_host(whole))
    gsum = gq.gq_sum_words(torch.cat(parts), n, d, W)
    mean = gq.gq_dequantize_words(gsum, n, d, s, scheme, W, norm)
    fmean, _, _ = gq.gq_compress_mean(xd, s, 2.0, INF, scheme, 5)
    assert np.array_equal(host(mean), host(fmean))


def _sample_cols(d, rng, k=20000):
    edge = np.concatenate([np.arange(0, min(d, 4100)), np.arange(max(0, d - 4100), d)])
    return np.unique(np.concatenate([edge, rng.integers(0, d, size=k)]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", [2, 3, 4, 5])
def test_workload_full_size(key):
    """Full-size workloads at the minimal width (11 and 13 bits, 2 fields per
    word; 8 bits from bf16 input, 4 per word; 9 bits, 3 per word): the word
    path's sums and mean equal the fused path's at every coordinate, and
    sampled columns equal the oracle's at the device's norm."""
    w = wl.WORKLOADS[key]
    threads = min(16, os.cpu_count() or 1)
    log(f"workload {key} {w.name}: generating {w.input_bytes / 1e9:.2f} GB")
    x = wl.generate(w, threads=threads)
    xd = to_dev(x)
    W = gq.gq_min_code_bits(w.n, w.s, w.scheme)
    M = M_of(w.s, w.scheme)
    fmean, norm, fsum = gq.gq_compress_mean(xd, w.s, w.q, w.p, w.scheme, w.seed, code_bits=32,
                                            want_code_sum=True)
    words = gq.gq_quantize_words(xd, w.s, w.scheme, norm, w.seed, W)
    wsum = gq.gq_sum_words(words, w.n, w.d, W)
    mean = gq.gq_dequantize_words(wsum, w.n, w.d, w.s, w.scheme, W, norm)
    csum = gq.gq_compress_words_from_norm(xd, w.s, w.scheme, norm, w.seed, W)
    assert torch.equal(csum, wsum)
    log("unpacking")
    sums = oracle.unpack_word_sums(words_host(wsum), w.n, w.d, W, M)
    assert np.array_equal(sums, host(fsum).view(np.int32)[: w.d].astype(np.int64))
    gmean = host(mean)
    assert np.array_equal(gmean, host(fmean))
    log("sampled oracle columns")
    cols = _sample_cols(w.d, np.random.default_rng(key))
    N = np.float32(host(norm)[0])
    osums, omean = oracle.compress_mean_cols(x, N, w.s, SCH[w.scheme], w.seed, cols)
    assert np.array_equal(sums[cols], osums)
    assert np.array_equal(gmean[cols], omean)
    del xd, x, words
    torch.cuda.empty_cache()
    log(f"workload {key} ok")

"""GPU parity of the word layout for a native integer all-reduce.

floor(32 / W) fields of code + M per 32-bit word, so that a plain uint32
SUM over the rows adds every code exactly.  Bar: words, summed words and
code sums bit-exact against the oracle; the mean bit-exact against the
oracle's dequantization of the same sums.  Full-size workloads are checked
at every coordinate in test_gpu_full_size.py.  Inputs come from the seeded generators of workloads.py; only
the oracle computes expected values.
"""
import math

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
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compress_words_equals_the_summed_rows(n0, s, scheme, W, dtype):
    """One pass over a device's rows: the word-wise sum of its rows' words,
    bit-exact against the oracle, for every fields-per-word count (bf16
    standard dithering takes the packed 16-bit accumulators)."""
    for n, d in SHAPES:
        n = min(n, n0)
        seed = 11 * n + d + W
        x = wl.random_rows(n, d, seed=seed, dtype=dtype, scale=0.3)
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


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_subnormal_inputs_take_the_exact_prescale(dtype):
    """N < 2^-64: |x| and N are scaled by 2^64 first; the word path's words,
    one-pass row and mean are the oracle's bit for bit."""
    rng = np.random.default_rng(31)
    # subnormal values (bf16 keeps 7 fraction bits, so a larger scale)
    scale = 1e-41 if dtype == "f32" else 1e-39
    x = (rng.standard_normal((3, 3001)) * scale).astype(np.float32)
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    xd = to_dev(x)
    for scheme, s in (("L", 7), ("E", 9)):
        W = gq.gq_min_code_bits(3, s, scheme)
        M = M_of(s, scheme)
        norm = gq.gq_global_norm(xd, 2.0, 2.0)
        N = np.float32(host(norm)[0])
        assert N < 2.0 ** -64
        ocodes = oracle.quantize(x, N, s, SCH[scheme], 4)
        assert np.any(ocodes != 0)
        owords = oracle.pack_words(ocodes, W, M)
        assert np.array_equal(words_host(gq.gq_quantize_words(xd, s, scheme, norm, 4, W)), owords)
        osum = oracle.sum_words(owords)
        assert np.array_equal(words_host(gq.gq_compress_words_from_norm(xd, s, scheme, norm, 4, W)),
                              osum)
        mean = gq.gq_dequantize_words(u32(osum), 3, 3001, s, scheme, W, norm)
        sums = oracle.unpack_word_sums(osum, 3, 3001, W, M)
        assert np.array_equal(host(mean), oracle.dequantize(sums, 3, N, s, SCH[scheme]))


def test_non_finite_inputs_stay_in_their_fields():
    """NaN and +-inf inputs give codes in [-M, M], so every field stays in
    [0, 2M] and no field carries into its neighbour."""
    x = wl.random_rows(4, 4096, seed=9)
    x[0, 5] = np.nan
    x[1, 100] = np.inf
    x[2, 2000] = -np.inf
    xd = to_dev(x)
    norm = gq.gq_global_norm(xd, INF, INF)
    for scheme, s in (("L", 7), ("E", 6)):
        W = gq.gq_min_code_bits(4, s, scheme)
        M = M_of(s, scheme)
        f = oracle.word_fields(W)
        rows = words_host(gq.gq_quantize_words(xd, s, scheme, norm, 1, W))
        for r in rows:
            fields = (r[:, None] >> (W * np.arange(f, dtype=np.uint32))) & ((1 << W) - 1)
            assert fields.max() <= 2 * M
        total = words_host(gq.gq_compress_words_from_norm(xd, s, scheme, norm, 1, W))
        sums = oracle.unpack_word_sums(total, 4, 4096, W, M)
        assert np.abs(sums).max() <= 4 * M


def test_empty_rows_launch_nothing():
    xd = torch.zeros((3, 0), dtype=torch.float32, device=DEV)
    norm = torch.zeros(1, dtype=torch.float32, device=DEV)
    assert gq.gq_quantize_words(xd, 7, "L", norm, 1, 6).numel() == 0
    assert gq.gq_compress_words_from_norm(xd, 7, "L", norm, 1, 6).numel() == 0
    assert gq.gq_dequantize_words(torch.zeros(0, dtype=torch.int32, device=DEV), 3, 0, 7, "L", 6,
                                  norm).numel() == 0
    torch.cuda.synchronize()


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

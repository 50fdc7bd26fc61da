"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Bar: integer codes and code sums bit-exact; the norm within 1e-6 relative
(the fp64 sums are taken in different orders; the fp32 norm then agrees to
the bit unless the exact value sits within ~1e-15 of an fp32 rounding
boundary) and, because every code and mean depends on the norm's bits, the
dequantized means are compared bit-exactly too.  Inputs come from the
seeded generators of workloads.py and only the oracle computes expected
values.
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
INF = math.inf
SCH = {"L": oracle.SCHEME_L, "E": oracle.SCHEME_E}
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-parity {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


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


def check_norm(gN, N):
    gN = np.float32(gN)
    assert abs(float(gN) - float(N)) <= 1e-6 * abs(float(N)) or gN == N, (gN, N)
    assert gN == N, f"norm differs in the last bits: {gN!r} vs {N!r}"


def M_of(s, scheme):
    return s if scheme == "L" else 1 << (s - 1)


# ---------------------------------------------------------------------------
# Small shapes: several tiles, ragged tails, every scheme, norm and dtype

SHAPES = [(1, 1), (3, 17), (4, 2048), (4, 2049), (2, 6000), (5, 4104), (7, 10007), (16, 24)]
CASES = [("L", 7, 2.0, 2.0), ("L", 127, 2.0, INF), ("E", 8, 2.0, 2.0), ("E", 5, INF, INF),
         ("L", 3, INF, 2.0), ("E", 12, 2.0, INF)]


@pytest.mark.parametrize("n,d", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scheme,s,q,p", CASES)
def test_fused_and_unfused_match_oracle(n, d, dtype, scheme, s, q, p):
    seed = 1000 * n + d
    x = wl.random_rows(n, d, seed=seed, dtype=dtype, scale=0.3)
    W = gq.gq_min_code_bits(n, s, scheme)
    N, sums, mean = oracle.compress_mean(x, s, q, p, SCH[scheme], seed)
    xd = to_dev(x)
    # fused path
    gmean, gnorm, gsum = gq.gq_compress_mean(xd, s, q, p, scheme, seed, code_bits=W,
                                             want_code_sum=True)
    check_norm(host(gnorm)[0], N)
    assert np.array_equal(host(gsum), oracle.pack(sums.astype(np.int32), W)[0])
    assert np.array_equal(host(gmean), mean)
    # unfused path: norm, codes, integer sum, dequantize
    norm = gq.gq_global_norm(xd, q, p)
    check_norm(host(norm)[0], N)
    codes = gq.gq_quantize(xd, s, scheme, norm, seed, W)
    ocodes = oracle.quantize(x, N, s, SCH[scheme], seed)
    assert np.array_equal(host(codes), oracle.pack(ocodes, W))
    # the sum and dequantization kernels take the oracle's packed codes as input
    packed = torch.from_numpy(oracle.pack(ocodes, W)).to(DEV)
    csum = gq.gq_reduce_codes(packed, n, d, W)
    assert np.array_equal(host(csum), oracle.pack(sums.astype(np.int32), W)[0])
    dmean = gq.gq_dequantize(torch.from_numpy(oracle.pack(sums.astype(np.int32), W)[0]).to(DEV),
                             n, d, s, scheme, W, norm)
    assert np.array_equal(host(dmean), mean)


@pytest.mark.parametrize("scheme,s,n", [("L", 3, 4), ("E", 4, 3), ("L", 100, 2)])
def test_every_code_width(scheme, s, n):
    d = 5000
    x = wl.random_rows(n, d, seed=s, scale=2.0)
    N, sums, _ = oracle.compress_mean(x, s, 2, 2, SCH[scheme], 3)
    ocodes = oracle.quantize(x, N, s, SCH[scheme], 3)
    xd = to_dev(x)
    norm = gq.gq_global_norm(xd, 2, 2)
    for W in range(gq.gq_min_code_bits(n, s, scheme), 33):
        codes = gq.gq_quantize(xd, s, scheme, norm, 3, W)
        assert np.array_equal(host(codes), oracle.pack(ocodes, W)), W
        csum = gq.gq_reduce_codes(codes, n, d, W)
        assert np.array_equal(host(csum), oracle.pack(sums.astype(np.int32), W)[0]), W
        _, _, fsum = gq.gq_compress_mean(xd, s, 2, 2, scheme, 3, code_bits=W, want_code_sum=True)
        assert np.array_equal(host(fsum), host(csum)), W


@pytest.mark.parametrize("n,s", [(1, 32767), (2, 16383), (2, 16384), (3, 10922), (9, 3641)])
def test_packed_int16_sum_limits(n, s):
    """bf16 standard dithering sums pairs of coordinates in int16 lanes while
    n s < 2^15: sums at +-n s exactly (every input at the norm, q = p = inf),
    mixed signs, ties and a ragged tail, on both sides of the limit."""
    d = 4099
    x = wl.random_rows(n, d, seed=s, dtype="f32", scale=1.0)
    x[:, :300] = 8.0   # the largest magnitude: t = s exactly, sum n s
    x[:, 300:600] = -8.0
    x[0, 600] = 8.0
    x = wl.f32_to_bf16_bits(x)
    W = gq.gq_min_code_bits(n, s, "L")
    for q, p, seed in ((INF, INF, 5), (2.0, 2.0, 6), (INF, 2.0, 2**64 - 3)):
        N, sums, mean = oracle.compress_mean(x, s, q, p, SCH["L"], seed)
        gmean, gnorm, gsum = gq.gq_compress_mean(to_dev(x), s, q, p, "L", seed, code_bits=W,
                                                 want_code_sum=True)
        check_norm(host(gnorm)[0], N)
        if q == INF and p == INF:
            assert sums[:300].tolist() == [n * s] * 300 and sums[300:600].tolist() == [-n * s] * 300
        assert np.array_equal(host(gsum), oracle.pack(sums.astype(np.int32), W)[0])
        assert np.array_equal(host(gmean), mean)


@pytest.mark.parametrize("n,d,scheme,s,q,p", [(3000, 37, "L", 5, 2.0, 2.0),
                                               (2049, 130, "E", 6, INF, INF),
                                               (1500, 4100, "L", 127, 2.0, INF)])
def test_many_workers(n, d, scheme, s, q, p):
    """More workers than the finalize block has threads: its rows go in
    several passes; the fused pass walks thousands of rows per coordinate."""
    x = wl.random_rows(n, d, seed=n, scale=0.1)
    W = gq.gq_min_code_bits(n, s, scheme)
    N, sums, mean = oracle.compress_mean(x, s, q, p, SCH[scheme], 9)
    xd = to_dev(x)
    gmean, gnorm, gsum = gq.gq_compress_mean(xd, s, q, p, scheme, 9, code_bits=W,
                                             want_code_sum=True)
    check_norm(host(gnorm)[0], N)
    assert np.array_equal(host(gsum), oracle.pack(sums.astype(np.int32), W)[0])
    assert np.array_equal(host(gmean), mean)
    if scheme == "L" and q == 2.0 and p == 2.0:
        norms, codes, lmean = oracle.qsgd_local_mean(x, s, 9)
        gl, gn, _ = gq.gq_qsgd_local_mean(xd, s, 9)
        assert np.array_equal(host(gn), norms)
        assert np.array_equal(host(gl), lmean)


@pytest.mark.parametrize("scheme,s,n", [("E", 28, 3), ("L", 1 << 23, 4), ("E", 26, 9),
                                         ("L", 5_000_000, 7)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_int32_accumulator_above_2_24(scheme, s, n, dtype):
    """Sums of magnitude up to n M > 2^24 are no longer exact in fp32, so the
    fused pass and the one-pass word row (one field per word at these widths)
    accumulate in int32: every entry point that takes that branch, at the
    minimal width and at 32 bits, against the oracle."""
    d = 6151
    M = M_of(s, scheme)
    assert n * M > 1 << 24
    x = wl.random_rows(n, d, seed=s + n, dtype="f32", scale=0.5)
    x[:, :64] = 4.0  # t at the top level in every row: sums of +-n M
    x[1, :32] = -4.0
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    seed = 0x0123456789ABCDEF + n
    N, sums, mean = oracle.compress_mean(x, s, INF, INF, SCH[scheme], seed)
    assert np.abs(sums).max() > 1 << 24
    codes = oracle.quantize(x, N, s, SCH[scheme], seed)
    Wmin = gq.gq_min_code_bits(n, s, scheme)
    xd = to_dev(x)
    for W in sorted({Wmin, 32}):
        gmean, gnorm, gsum = gq.gq_compress_mean(xd, s, INF, INF, scheme, seed, code_bits=W,
                                                 want_code_sum=True)
        check_norm(host(gnorm)[0], N)
        assert np.array_equal(host(gsum), oracle.pack(sums.astype(np.int32), W)[0]), W
        assert np.array_equal(host(gmean), mean), W
        fmean, fsum = gq.gq_compress_mean_from_norm(xd, s, scheme, seed, gnorm, code_bits=W,
                                                    want_code_sum=True)
        assert np.array_equal(host(fsum), host(gsum)) and np.array_equal(host(fmean), mean), W
        owords = oracle.pack_words(codes, W, M)
        one = gq.gq_compress_words_from_norm(xd, s, scheme, gnorm, seed, W)
        assert np.array_equal(host(one).view(np.uint32), oracle.sum_words(owords)), W
        words = gq.gq_quantize_words(xd, s, scheme, gnorm, seed, W)
        assert np.array_equal(host(words).view(np.uint32), owords), W
        wmean = gq.gq_dequantize_words(one, n, d, s, scheme, W, gnorm)
        assert np.array_equal(host(wmean), mean), W


def staged_matches(staged: np.ndarray, sums: np.ndarray) -> bool:
    """gq_compress_sums8's buffer against the oracle's exact sums: the group
    mask (bit g = group g holds a non-zero sum; the bits past the last group
    in its word zero) and the bytes of the marked groups (the sum, or -128
    beyond [-127, 127])."""
    d = sums.size
    groups = -(-d // 8)
    words = -(-d // 512)  # the mask's 64-bit words (its 16-byte padding is not written)
    mb = (words * 8 + 15) // 16 * 16
    bits = np.unpackbits(staged[:words * 8].view(np.uint8), bitorder="little")
    padded = np.zeros(groups * 8, np.int64)
    padded[:d] = sums
    nzg = (padded.reshape(groups, 8) != 0).any(axis=1)
    if not (np.array_equal(bits[:groups].astype(bool), nzg) and not bits[groups:].any()):
        return False
    cols = np.flatnonzero(np.repeat(nzg, 8)[:d])
    want = np.where(np.abs(sums) <= 127, sums, -128).astype(np.int8)
    return np.array_equal(staged[mb:mb + d].view(np.int8)[cols], want[cols])


@pytest.mark.parametrize("n,d,scheme,s,q,p,escapes", [(16, 7001, "E", 8, INF, INF, True),
                                                       (32, 10_007, "L", 3, 2.0, 2.0, False),
                                                       (40, 4104, "E", 8, 2.0, INF, True),
                                                       (64, 2049, "L", 127, INF, 2.0, True),
                                                       (33, 16_384, "E", 5, INF, INF, True),
                                                       (48, 5000, "L", 1 << 20, 2.0, 2.0, True),
                                                       (32, 7, "L", 7, 2.0, 2.0, False)])
def test_staged_sums_for_many_workers(n, d, scheme, s, q, p, escapes):
    """The staged compress step (gq_compress_sums8, gq_dequantize_sums8): the
    pass stages a bit per 8-coordinate group and 1-byte sums of the non-zero
    groups, and a second kernel writes the mean.  Sums outside [-127, 127]
    (the first 300 coordinates sit at the top level in every row, so they
    sum to +-n M; the E rows flip signs) take the escape and are recomputed
    from x.  Against the oracle, and gq_compress_mean with the larger
    workspace (the zero-code skip; those first spans are dense) and with the
    smallest one (every coordinate read)."""
    x = wl.random_rows(n, d, seed=n * 7 + d, scale=0.2)
    x[:, : min(d, 300)] = 2.0
    if scheme == "E":
        x[::3, : min(d, 100)] = -2.0
    N, sums, mean = oracle.compress_mean(x, s, q, p, SCH[scheme], 17)
    # escaped sums (beyond one byte) beside plain ones where the case asks for them
    assert ((np.abs(sums) > 127).any() and (np.abs(sums) <= 127).any()) == escapes
    xd = to_dev(x)
    big = torch.empty(gq.gq_compress_workspace_bytes(n, d), dtype=torch.uint8, device=DEV)
    small = torch.empty(gq.gq_workspace_bytes(n, d), dtype=torch.uint8, device=DEV)
    # room for the span bounds of the zero-code skip
    assert big.numel() == small.numel() + -(-gq.gq_span_bounds_bytes(n, d) // 256) * 256
    gmean, gnorm, _ = gq.gq_compress_mean(xd, s, q, p, scheme, 17, workspace=big)
    check_norm(host(gnorm)[0], N)
    assert np.array_equal(host(gmean), mean)
    one, _, _ = gq.gq_compress_mean(xd, s, q, p, scheme, 17, workspace=small)
    assert np.array_equal(host(one), mean)
    # the two staged kernels through their own entry points, fp32 and bf16;
    # the staging buffer starts full of garbage (unmarked groups stay unread)
    b8 = torch.full((gq.gq_sums8_bytes(d),), 0x7F, dtype=torch.uint8, device=DEV)
    gq.gq_compress_sums8(xd, s, scheme, 17, gnorm, sums8=b8)
    assert staged_matches(host(b8), sums)
    assert np.array_equal(host(gq.gq_dequantize_sums8(xd, s, scheme, 17, gnorm, b8)), mean)
    xb = wl.f32_to_bf16_bits(x)
    Nb, sb, meanb = oracle.compress_mean(xb, s, q, p, SCH[scheme], 19)
    xbd = to_dev(xb)
    nb = gq.gq_global_norm(xbd, q, p)
    check_norm(host(nb)[0], Nb)
    b8 = gq.gq_compress_sums8(xbd, s, scheme, 19, nb)
    assert staged_matches(host(b8), sb)
    assert np.array_equal(host(gq.gq_dequantize_sums8(xbd, s, scheme, 19, nb, b8)), meanb)
    # all-zero input: every bit clear, nothing else written, mean zero
    z = torch.zeros((n, d), dtype=torch.float32, device=DEV)
    zn = gq.gq_global_norm(z, q, p)
    gq.gq_compress_sums8(z, s, scheme, 3, zn, sums8=b8)
    assert staged_matches(host(b8), np.zeros(d, np.int64))
    assert not host(gq.gq_dequantize_sums8(z, s, scheme, 3, zn, b8)).any()
    # subnormal inputs (the exact pre-scale) on the same path
    y = (x * np.float32(1e-40)).astype(np.float32)
    N2, _, mean2 = oracle.compress_mean(y, s, q, p, SCH[scheme], 18)
    g2, n2, _ = gq.gq_compress_mean(to_dev(y), s, q, p, scheme, 18, workspace=big)
    check_norm(host(n2)[0], N2)
    assert np.array_equal(host(g2), mean2)


def test_worker_base_shards_reproduce_the_whole():
    n, d, s = 6, 3000, 9
    x = wl.random_rows(n, d, seed=5)
    N, _ = oracle.global_norm(x, 2, 2)
    W = gq.gq_min_code_bits(n, s, "L")
    whole = oracle.pack(oracle.quantize(x, N, s, SCH["L"], 77), W)
    xd = to_dev(x)
    norm = gq.gq_global_norm(xd, 2, 2)
    for r in range(n):  # each "rank" quantizes its own row with its global index
        part = gq.gq_quantize(xd[r:r + 1].contiguous(), s, "L", norm, 77, W, worker_base=r)
        assert np.array_equal(host(part)[0], whole[r])


# ---------------------------------------------------------------------------
# Edge cases

def test_zero_input_and_empty_rows():
    x = np.zeros((3, 4100), np.float32)
    x[1, 7] = -0.0
    xd = to_dev(x)
    for scheme, s in (("L", 5), ("E", 6)):
        W = gq.gq_min_code_bits(3, s, scheme)
        mean, norm, csum = gq.gq_compress_mean(xd, s, 2, 2, scheme, 1, code_bits=W,
                                               want_code_sum=True)
        assert host(norm)[0] == 0 and not host(mean).any() and not host(csum).any()
        codes = gq.gq_quantize(xd, s, scheme, norm, 1, W)
        assert not host(codes).any()
    # d == 0: the norm is 0 and nothing else is touched
    e = torch.empty((2, 0), dtype=torch.float32, device=DEV)
    mean, norm, _ = gq.gq_compress_mean(e, 3, 2, 2, "L", 0)
    assert host(norm)[0] == 0 and mean.numel() == 0


def test_subnormal_inputs_use_the_exact_prescale():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((3, 3000)) * 1e-41).astype(np.float32)  # all subnormal
    assert np.all(np.abs(x[x != 0]) < np.finfo(np.float32).tiny)
    for scheme, s, q, p in (("L", 7, 2, 2), ("E", 9, INF, INF), ("L", 2, 2, INF)):
        N, sums, mean = oracle.compress_mean(x, s, q, p, SCH[scheme], 4)
        assert N < 2.0 ** -64
        W = gq.gq_min_code_bits(3, s, scheme)
        gmean, gnorm, gsum = gq.gq_compress_mean(to_dev(x), s, q, p, scheme, 4, code_bits=W,
                                                 want_code_sum=True)
        check_norm(host(gnorm)[0], N)
        assert np.array_equal(host(gsum), oracle.pack(sums.astype(np.int32), W)[0])
        assert np.array_equal(host(gmean), mean)


def test_exact_levels_and_max_element():
    # q = p = inf with max |x| = 8: x = k exactly gives code k (L, s = 8)
    x = np.tile(np.arange(-8, 9, dtype=np.float32), (2, 64))
    n, d = x.shape
    xd = to_dev(x)
    W = gq.gq_min_code_bits(n, 8, "L")
    for seed in range(3):
        mean, norm, csum = gq.gq_compress_mean(xd, 8, INF, INF, "L", seed, code_bits=W,
                                               want_code_sum=True)
        assert host(norm)[0] == 8.0
        expect = (x.astype(np.int64).sum(axis=0)).astype(np.int32)
        assert np.array_equal(host(csum), oracle.pack(expect, W)[0])
        assert np.array_equal(host(mean), x.mean(axis=0))


def test_non_finite_inputs_stay_on_the_grid():
    x = wl.random_rows(4, 4096, seed=9)
    x[0, 5] = np.nan
    x[1, 100] = np.inf
    x[2, 2000] = -np.inf
    for scheme, s in (("L", 7), ("E", 6)):
        W = gq.gq_min_code_bits(4, s, scheme)
        xd = to_dev(x)
        norm = gq.gq_global_norm(xd, INF, INF)
        codes = gq.gq_quantize(xd, s, scheme, norm, 1, W)
        c = oracle.unpack(host(codes), 4, 4096, W)
        assert np.abs(c).max() <= M_of(s, scheme)


def test_repeated_calls_are_bit_identical():
    w = wl.WORKLOADS[1]
    x = wl.generate(w)
    xd = to_dev(x)
    outs = [gq.gq_compress_mean(xd, w.s, w.q, w.p, w.scheme, w.seed, code_bits=8,
                                want_code_sum=True) for _ in range(3)]
    ref = [host(t) for t in outs[0]]
    for o in outs[1:]:
        for a, b in zip(ref, o):
            assert np.array_equal(a, host(b))


# ---------------------------------------------------------------------------
# Local-norm QSGD ablation

@pytest.mark.parametrize("n,d,dtype", [(1, 100, "f32"), (4, 4099, "f32"), (8, 16384, "bf16")])
def test_local_qsgd_matches_oracle(n, d, dtype):
    s = 3
    x = wl.random_rows(n, d, seed=n + d, dtype=dtype)
    norms, codes, mean = oracle.qsgd_local_mean(x, s, 12)
    W = gq.gq_min_code_bits(1, s, "L")
    gmean, gnorms, gcodes = gq.gq_qsgd_local_mean(to_dev(x), s, 12, code_bits=W, want_codes=True)
    gn = host(gnorms)
    for i in range(n):
        check_norm(gn[i], norms[i])
    assert np.array_equal(host(gcodes), oracle.pack(codes, W))
    assert np.array_equal(host(gmean), mean)


# ---------------------------------------------------------------------------
# Inputs above 256 MiB take the one-shot norm pass (16 KB blocks, a middle
# reduction): ragged, unaligned and aligned rows, every kind of order, and
# the per-worker norms of the ablation; the bf16 case (just above 1 GiB,
# ragged rows) reads two groups per thread.

@pytest.mark.timeout(600)
@pytest.mark.parametrize("n,d,dtype,q,p", [(3, 89_478_487, "f32", 2.0, 2.0),
                                           (5, 53_687_093, "f32", INF, 2.0),
                                           (1, 268_435_464, "f32", 2.0, INF),
                                           (4, 67_108_869, "f32", 1.5, 3.0),
                                           (5, 107_374_185, "bf16", INF, 2.0)])
def test_large_input_norm(n, d, dtype, q, p):
    log(f"large-input norm n={n} d={d} {dtype} q={q} p={p}")
    x = np.empty((n, d), np.float32)
    for i in range(n):
        x[i] = wl.random_rows(1, d, seed=d + i, scale=0.01)[0]
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    N, _ = oracle.global_norm_rows(x, q, p, threads=min(16, n))
    xd = to_dev(x)
    gN = np.float32(host(gq.gq_global_norm(xd, q, p))[0])
    assert abs(float(gN) - float(N)) <= 1e-6 * float(N)
    assert gN == N, f"norm differs in the last bit ({gN!r} vs {N!r})"
    if q == 2.0 and p == 2.0:
        _, gnorms, _ = gq.gq_qsgd_local_mean(xd, 3, 1)
        assert np.array_equal(host(gnorms), oracle.local_norms(x, threads=n))
    del xd, x
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# General real orders (fp64 pow): the norm within 1e-6 relative; codes and
# means bit-exact against the oracle at the device's norm

@pytest.mark.parametrize("q,p", [(1.0, 1.0), (1.5, 3.0), (3.0, INF), (INF, 1.5), (2.0, 4.0),
                                 (7.25, 2.0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_general_orders(q, p, dtype):
    n, d, s = 6, 5003, 15
    x = wl.random_rows(n, d, seed=int(10 * min(q, 9)) + 3, dtype=dtype, scale=0.5)
    N, sums, mean = oracle.compress_mean(x, s, q, p, oracle.SCHEME_L, 8)
    W = gq.gq_min_code_bits(n, s, "L")
    gmean, gnorm, gsum = gq.gq_compress_mean(to_dev(x), s, q, p, "L", 8, code_bits=W,
                                             want_code_sum=True)
    gN = np.float32(host(gnorm)[0])
    assert abs(float(gN) - float(N)) <= 1e-6 * float(N)
    if gN != N:
        # fp64 pow of the device library and of the host libm may differ by
        # an ulp, which can move the fp32 norm by its last bit; every code is
        # a function of the norm's bits, so compare at the device's norm
        log(f"q={q} p={p} {dtype}: norm differs in the last bit ({gN!r} vs {N!r})")
        ocodes = oracle.quantize(x, gN, s, oracle.SCHEME_L, 8)
        sums = oracle.sum_codes(ocodes)
        mean = oracle.dequantize(sums, n, gN, s, oracle.SCHEME_L)
    assert np.array_equal(host(gsum), oracle.pack(sums.astype(np.int32), W)[0])
    assert np.array_equal(host(gmean), mean)

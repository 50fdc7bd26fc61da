"""GPU parity over a seeded random sweep of the whole parameter space.

Each case draws its own worker count, row length (log-uniform, so tiny rows,
single tiles, ragged tails and multi-tile rows all occur), input dtype,
scheme, s, (q, p) orders, 64-bit seed, code width between the minimum and
32, input scale (down to far below 2^-64, which takes the exact pre-scale),
and input structure (exact zeros, repeated values, sign flips, exact
levels).  Every entry point is compared with the oracle on the same inputs:
bit-exact for codes, code sums and means; the norm within 1e-6 relative.
Where the fp32 norm differs from the oracle's in its last bit (possible for
the fp64 pow orders, and with probability ~1e-7 otherwise), the codes and
means are compared with the oracle evaluated at the device's norm, since
every code is a function of the norm's bits.
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
DEV = "cuda:0"
SCH = {"L": oracle.SCHEME_L, "E": oracle.SCHEME_E}
ORDERS = [1.0, 1.5, 2.0, 2.0, 3.0, INF, INF]
# 60 cases by default; GQ_SWEEP_CASES widens the sweep for a longer run
N_CASES = int(os.environ.get("GQ_SWEEP_CASES", "60"))


def log(msg):
    print(f"[gpu-sweep {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def draw_case(k: int) -> dict:
    rng = np.random.default_rng([0x5EED, k])
    n = int(rng.integers(1, 21))
    d = int(math.exp(rng.uniform(0.0, math.log(40000.0))))
    dtype = "bf16" if rng.random() < 0.4 else "f32"
    scheme = "E" if rng.random() < 0.4 else "L"
    if scheme == "L":
        s = max(1, int(math.exp(rng.uniform(0.0, math.log(5000.0)))))
    else:
        s = int(rng.integers(1, 17))
    q, p = float(rng.choice(ORDERS)), float(rng.choice(ORDERS))
    seed = int(rng.integers(0, 2**63, dtype=np.int64)) * 2 + int(rng.integers(0, 2))
    scale = 10.0 ** rng.uniform(-30.0, 3.0) if rng.random() < 0.3 else 10.0 ** rng.uniform(-3, 1)
    x = wl.random_rows(n, d, seed=1000 + k, dtype="f32", scale=scale)
    # structure: exact zeros, a repeated value, sign flips
    x[rng.random((n, d)) < rng.uniform(0.0, 0.3)] = 0.0
    if d > 4:
        x[:, rng.integers(0, d, size=max(1, d // 50))] = x[0, 0]
    x *= np.where(rng.random((n, d)) < 0.5, -1.0, 1.0).astype(np.float32)
    if dtype == "bf16":
        x = wl.f32_to_bf16_bits(x)
    Wmin = gq.gq_min_code_bits(n, s, scheme)
    W = int(rng.integers(Wmin, 33))
    # about one case in eight sums beyond 2^24 (the int32 accumulators of
    # the fused pass and the one-pass word row)
    if n >= 2 and rng.random() < 0.125:
        if scheme == "L":
            lo, hi = (1 << 24) // n + 1, min(1 << 24, (2**31 - 1) // n)
            s = int(math.exp(rng.uniform(math.log(lo), math.log(hi))))
        else:
            ss = [t for t in range(1, 32) if (1 << 24) < n * (1 << (t - 1)) < 2**31]
            s = int(rng.choice(ss))
        W = int(rng.integers(gq.gq_min_code_bits(n, s, scheme), 33))
    return dict(n=n, d=d, dtype=dtype, scheme=scheme, s=s, q=q, p=p, seed=seed, W=W, x=x)


def oracle_at(x, N, c):
    """Codes, sums and mean of the oracle at a given fp32 norm."""
    codes = oracle.quantize(x, N, c["s"], SCH[c["scheme"]], c["seed"])
    sums = oracle.sum_codes(codes)
    mean = oracle.dequantize(sums, c["n"], N, c["s"], SCH[c["scheme"]])
    return codes, sums, mean


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_case(k):
    c = draw_case(k)
    n, d, s, W, x = c["n"], c["d"], c["s"], c["W"], c["x"]
    log(f"case {k}: n={n} d={d} {c['dtype']} {c['scheme']} s={s} q={c['q']} p={c['p']} W={W}")
    N, _ = oracle.global_norm(x, c["q"], c["p"])
    xd = to_dev(x)
    gmean, gnorm, gsum = gq.gq_compress_mean(xd, s, c["q"], c["p"], c["scheme"], c["seed"],
                                             code_bits=W, want_code_sum=True)
    gN = np.float32(host(gnorm)[0])
    if math.isfinite(N) and N != 0:
        assert abs(float(gN) - float(N)) <= 1e-6 * abs(float(N)), (gN, N)
    else:
        assert gN == N or (math.isnan(gN) and math.isnan(N))
    at = N if gN == N else gN
    codes, sums, mean = oracle_at(x, at, c)
    assert np.array_equal(host(gsum), oracle.pack(sums.astype(np.int32), W)[0])
    assert np.array_equal(host(gmean), mean)
    # unfused entry points on the same norm
    norm = gq.gq_global_norm(xd, c["q"], c["p"])
    assert np.float32(host(norm)[0]) == gN
    gcodes = gq.gq_quantize(xd, s, c["scheme"], norm, c["seed"], W)
    assert np.array_equal(host(gcodes), oracle.pack(codes, W))
    csum = gq.gq_reduce_codes(gcodes, n, d, W)
    assert np.array_equal(host(csum), host(gsum))
    dmean = gq.gq_dequantize(csum, n, d, s, c["scheme"], W, norm)
    assert np.array_equal(host(dmean), mean)
    fmean, fsum = gq.gq_compress_mean_from_norm(xd, s, c["scheme"], c["seed"], norm, code_bits=W,
                                                want_code_sum=True)
    assert np.array_equal(host(fmean), mean) and np.array_equal(host(fsum), host(gsum))
    # a shard: the last worker quantized alone at its global index
    part = gq.gq_quantize(xd[n - 1:n].clone(), s, c["scheme"], norm, c["seed"], W,
                          worker_base=n - 1)
    assert np.array_equal(host(part)[0], oracle.pack(codes, W)[n - 1])
    # the word layout for a native uint32 SUM: rows, their sum, the one-pass
    # row and the mean from it
    M = oracle.top_code(s, SCH[c["scheme"]])
    owords = oracle.pack_words(codes, W, M)
    words = gq.gq_quantize_words(xd, s, c["scheme"], norm, c["seed"], W)
    assert np.array_equal(host(words).view(np.uint32), owords)
    wsum = gq.gq_sum_words(words, n, d, W)
    assert np.array_equal(host(wsum).view(np.uint32), oracle.sum_words(owords))
    one = gq.gq_compress_words_from_norm(xd, s, c["scheme"], norm, c["seed"], W)
    assert np.array_equal(host(one), host(wsum))
    wmean = gq.gq_dequantize_words(wsum, n, d, s, c["scheme"], W, norm)
    assert np.array_equal(host(wmean), mean)


@pytest.mark.parametrize("k", range(0, N_CASES, 4))
def test_random_case_many_workers(k):
    """32 to 79 fp32 workers: the path that stages 1-byte sums (with escapes
    for sums beyond [-127, 127]) between the pass and the mean."""
    rng = np.random.default_rng([0x5EED, 7, k])
    n = int(rng.integers(32, 80))
    d = int(math.exp(rng.uniform(0.0, math.log(20000.0))))
    scheme = "E" if rng.random() < 0.4 else "L"
    s = int(rng.integers(1, 13)) if scheme == "E" else max(1, int(math.exp(rng.uniform(0, 7))))
    q, p = float(rng.choice(ORDERS)), float(rng.choice(ORDERS))
    seed = int(rng.integers(0, 2**63, dtype=np.int64))
    x = wl.random_rows(n, d, seed=5000 + k, dtype="f32", scale=10.0 ** rng.uniform(-3, 1))
    x[rng.random((n, d)) < 0.2] = 0.0
    if rng.random() < 0.5 and d > 8:  # some columns at one value: large sums, escapes
        x[:, rng.integers(0, d, size=max(1, d // 10))] = np.abs(x).max()
    log(f"many-workers case {k}: n={n} d={d} {scheme} s={s} q={q} p={p}")
    N, _ = oracle.global_norm(x, q, p)
    gmean, gnorm, _ = gq.gq_compress_mean(to_dev(x), s, q, p, scheme, seed)
    gN = np.float32(host(gnorm)[0])
    assert abs(float(gN) - float(N)) <= 1e-6 * abs(float(N)) or gN == N
    _, _, mean = oracle_at(x, N if gN == N else gN, dict(s=s, scheme=scheme, seed=seed, n=n))
    assert np.array_equal(host(gmean), mean)


@pytest.mark.parametrize("k", range(0, N_CASES, 3))
def test_random_case_local_and_e8(k):
    c = draw_case(k)
    n, d, x, seed = c["n"], c["d"], c["x"], c["seed"]
    s = min(c["s"], 200)
    xd = to_dev(x)
    norms, codes, mean = oracle.qsgd_local_mean(x, s, seed)
    W = gq.gq_min_code_bits(1, s, "L")
    lmean, lnorms, lcodes = gq.gq_qsgd_local_mean(xd, s, seed, code_bits=W, want_codes=True)
    gn = host(lnorms)
    if not np.array_equal(gn, norms):
        # a last-bit difference of some worker's norm: both within 1e-6, and
        # the codes and mean compared with the oracle at the device's norms
        assert np.all(np.abs(gn.astype(np.float64) - norms) <= 1e-6 * np.abs(norms))
        codes, mean = oracle.qsgd_local_cols(x, gn, s, seed, np.arange(d))
    assert np.array_equal(host(lcodes), oracle.pack(codes, W))
    assert np.array_equal(host(lmean), mean)
    # 8-bit format: the tree needs a power-of-two worker count
    m = 1 << (n.bit_length() - 1)
    xm = np.ascontiguousarray(x[:m])
    N, root, emean = oracle.e8_compress_mean(xm, c["q"], c["p"], seed)
    gmean, gnorm, groot = gq.gq_e8_compress_mean(to_dev(xm), c["q"], c["p"], seed, want_root=True)
    gN = np.float32(host(gnorm)[0])
    if gN != N:
        assert abs(float(gN) - float(N)) <= 1e-6 * abs(float(N))
        ecodes = oracle.e8_quantize(xm, gN, seed)
        root = oracle.e8_tree(ecodes, seed)
        emean = oracle.e8_dequantize(root, gN)
    assert np.array_equal(host(groot)[:d], root)
    assert np.array_equal(host(gmean), emean)
    if m >= 2:
        # two devices of m / 2 workers: subtrees at their offsets, then the top pair
        h = m // 2
        xmd = to_dev(xm)
        roots = [gq.gq_e8_subtree(gq.gq_e8_quantize(xmd[r * h:(r + 1) * h].clone(), gnorm, seed,
                                                    worker_base=r * h), h, d, seed, r * h)
                 for r in range(2)]
        top = gq.gq_e8_reduce_pair(roots[0], roots[1], d, seed, h.bit_length(), 0)
        assert np.array_equal(host(top)[:d], root)

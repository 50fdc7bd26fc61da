"""The path split over shards of workers, as each device of a data-parallel
job would run it, checked on one GPU.

Each shard computes its fp64 norm term (gq_norm_term); the terms are
combined on the host as one all-reduce of a double would (sum for finite p,
max for p = inf); N follows from the combined term (gq_norm_from_term).
Every shard then quantizes its rows at their global worker indices, the
integer code rows are summed across shards as the integer all-reduce
would, and gq_dequantize gives the mean.  All of it is compared with the
oracle run on the whole input at the same N: codes, sums and mean
bit-exact; the terms and N within the tolerances the header states.
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
DEV = "cuda:0"
SCH = {"L": oracle.SCHEME_L, "E": oracle.SCHEME_E}


def log(msg):
    print(f"[gpu-shards {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


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


def expected_term(pw, q, p):
    """The shard term from the oracle's per-worker partials (sum of |x|^q,
    or max |x| for q = inf), combined as the header defines it."""
    pw = np.asarray(pw, dtype=np.float64)
    if q == INF:
        w = pw
    elif q == 2.0:
        w = np.sqrt(pw)
    else:
        w = pw ** (1.0 / q)
    if p == INF:
        if q == 2.0:
            return float(pw.max())          # max_i S_i, the root comes later
        return float(w.max())
    if p == 2.0:
        return float(pw.sum()) if q == 2.0 else float((w * w).sum())
    return float((w ** p).sum())


SPLITS = [(0, 3), (3, 4), (4, 7)]


@pytest.mark.parametrize("q,p", [(2.0, 2.0), (INF, 2.0), (2.0, INF), (INF, INF),
                                 (1.5, 3.0), (3.0, INF), (1.0, 2.0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sharded_norm(q, p, dtype):
    n, d = 7, 5003
    x = wl.random_rows(n, d, seed=31 + int(min(q, 9.0) * 3) + int(min(p, 9.0)), dtype=dtype)
    xd = to_dev(x)
    log(f"norm q={q} p={p} {dtype}")
    N_full = np.float32(host(gq.gq_global_norm(xd, q, p))[0])
    N_or, pw = oracle.global_norm(x, q, p)
    # one shard holding every row: the same N bit for bit
    T = gq.gq_norm_term(xd, q, p)
    assert np.float32(host(gq.gq_norm_from_term(T, q, p))[0]) == N_full
    assert abs(host(T)[0] - expected_term(pw, q, p)) <= 1e-12 * expected_term(pw, q, p)
    # three shards
    terms = []
    for a, b in SPLITS:
        t = host(gq.gq_norm_term(xd[a:b].clone(), q, p))[0]
        assert abs(t - expected_term(pw[a:b], q, p)) <= 1e-12 * expected_term(pw[a:b], q, p)
        terms.append(float(t))
    comb = max(terms) if p == INF else math.fsum(terms)
    Nsh = np.float32(host(gq.gq_norm_from_term(
        torch.tensor([comb], dtype=torch.float64, device=DEV), q, p))[0])
    assert abs(float(Nsh) - float(N_full)) <= 1e-6 * float(N_full)
    assert abs(float(Nsh) - float(N_or)) <= 1e-6 * float(N_or)
    if q == INF and p == INF:
        assert Nsh == N_full == N_or


@pytest.mark.parametrize("scheme,s,q,p,dtype", [("L", 127, 2.0, INF, "f32"),
                                                ("E", 8, 2.0, 2.0, "f32"),
                                                ("L", 15, 2.0, 2.0, "bf16"),
                                                ("L", 3, INF, INF, "f32")])
def test_sharded_path_reproduces_the_whole(scheme, s, q, p, dtype):
    n, d, seed = 7, 20011, 0xC0FFEE
    x = wl.random_rows(n, d, seed=77 + s, dtype=dtype)
    xd = to_dev(x)
    W = gq.gq_min_code_bits(n, s, scheme)
    log(f"path {scheme} s={s} q={q} p={p} {dtype} W={W}")
    terms = [float(host(gq.gq_norm_term(xd[a:b].clone(), q, p))[0]) for a, b in SPLITS]
    comb = max(terms) if p == INF else math.fsum(terms)
    norm = gq.gq_norm_from_term(torch.tensor([comb], dtype=torch.float64, device=DEV), q, p)
    Nsh = np.float32(host(norm)[0])
    codes = oracle.quantize(x, Nsh, s, SCH[scheme], seed)
    sums = oracle.sum_codes(codes)
    mean = oracle.dequantize(sums, n, Nsh, s, SCH[scheme])
    total = np.zeros(d, dtype=np.int64)
    for a, b in SPLITS:
        part = gq.gq_quantize(xd[a:b].clone(), s, scheme, norm, seed, W, worker_base=a)
        assert np.array_equal(host(part), oracle.pack(codes[a:b], W))
        total += oracle.unpack(host(part), b - a, d, W).astype(np.int64).sum(axis=0)
    assert np.array_equal(total, sums)
    # the summed row as the integer all-reduce would deliver it, then the mean
    packed = torch.from_numpy(oracle.pack(total.astype(np.int32)[None, :], W)[0]).to(DEV)
    gmean = gq.gq_dequantize(packed, n, d, s, scheme, W, norm)
    assert np.array_equal(host(gmean), mean)

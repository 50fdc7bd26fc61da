"""Seeded sweep of the zero-code skip against the same pass reading every
coordinate, on the GPU alone.

The skip (span bounds from pass 1, the per-wave candidate queue) must give
the bits of the dense pass for any input, so this sweep draws many shapes
and settings -- worker counts across the 64-row threshold chunks, ragged
and tiny rows, both schemes and input types, the orders the norm supports,
inputs from plain to heavy-tailed, tiny and spiky -- and compares the mean,
the code sums and the word-layout row of both paths bit for bit.  The
oracle itself is compared in the skip tests and the full-size tests; here
the dense pass (checked against the oracle elsewhere) is the reference, so
the sweep can afford hundreds of cases.
"""
import math
import sys
import time

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import allreduce_compatible_gradient_amd as gq  # noqa: E402
import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
INF = math.inf
CASES = 240


def log(msg):
    print(f"[gpu-skip-sweep {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()


def draw(rng):
    n = int(rng.choice([1, 2, 3, 7, 8, 15, 16, 33, 63, 64, 65, 100, 129, 200]))
    d = int(np.exp(rng.uniform(0.0, np.log(120_000))))
    dtype = "bf16" if rng.random() < 0.4 else "f32"
    scheme = "L" if rng.random() < 0.6 else "E"
    s = int(rng.choice([1, 2, 3, 7, 15, 127])) if scheme == "L" else int(rng.integers(1, 12))
    q = float(rng.choice([2.0, INF, 2.0, 1.5]))
    p = float(rng.choice([2.0, INF, 2.0, 3.0]))
    kind = str(rng.choice(["plain", "heavy", "spikes", "tiny", "rowscale"]))
    return n, d, dtype, scheme, s, q, p, kind


def make(n, d, dtype, kind, seed):
    rng = np.random.default_rng(seed)
    x = wl.random_rows(n, d, seed=seed, scale=0.01)
    if kind == "heavy":
        m = rng.random((n, d)) < 0.002
        x[m] *= np.float32(200.0)
    elif kind == "spikes":
        for _ in range(1 + n // 8):
            x[rng.integers(0, n), rng.integers(0, d)] = np.float32(rng.choice([-1, 1]) * 40.0)
    elif kind == "tiny":
        x = (x * np.float32(1e-36)).astype(np.float32)
    elif kind == "rowscale":
        x = (x * (10.0 ** rng.uniform(-3, 2, size=(n, 1)))).astype(np.float32)
    return wl.f32_to_bf16_bits(x) if dtype == "bf16" else x


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def test_skip_equals_dense_on_a_seeded_sweep():
    rng = np.random.default_rng(20261203)
    counts = {"queue_rows": 0, "cases": 0}
    for c in range(CASES):
        n, d, dtype, scheme, s, q, p, kind = draw(rng)
        W = gq.gq_min_code_bits(n, s, scheme)
        if W < 0 or W > 32:
            continue
        seed = 1000 + c
        x = make(n, d, dtype, kind, seed)
        xd = to_dev(x)
        tag = f"case {c}: n={n} d={d} {dtype} {scheme} s={s} q={q} p={p} {kind}"
        norm, bounds = gq.gq_global_norm_bounds(xd, q, p)
        skip, ssum = gq.gq_compress_mean_skip(xd, s, scheme, seed, norm, bounds, code_bits=W,
                                              want_code_sum=True)
        dense, dsum = gq.gq_compress_mean_from_norm(xd, s, scheme, seed, norm, code_bits=W,
                                                    want_code_sum=True)
        wskip = gq.gq_compress_words_skip(xd, s, scheme, norm, bounds, seed, W, worker_base=c)
        wdense = gq.gq_compress_words_from_norm(xd, s, scheme, norm, seed, W, worker_base=c)
        torch.cuda.synchronize()
        a, b = skip.cpu().numpy(), dense.cpu().numpy()
        # both paths share N; a NaN mean (inf or NaN input) has no defined sign
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)) or \
            np.array_equal(a, b, equal_nan=True), tag
        assert torch.equal(ssum, dsum), tag
        assert torch.equal(wskip, wdense), tag
        counts["cases"] += 1
    log(f"{counts['cases']} cases: skip == dense (mean, code sums, word rows)")
    assert counts["cases"] >= CASES * 3 // 4

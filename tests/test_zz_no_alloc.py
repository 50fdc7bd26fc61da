"""The no-allocation entry point against the entry point it mirrors.

gq_compress_mean_noalloc keeps the norm pass's partial sums, and the span
bounds of the zero-code skip, in the library's own device array instead of
a caller workspace.  Called through
the C ABI with preallocated outputs, it must give gq_compress_mean's norm,
mean and code sums bit for bit, on consecutive calls that reuse the array
with a smaller input each time: first above 1 GiB of fp32 (the one-shot
norm pass and its middle reduction), then a multi-tile ragged input, then
a bf16 input of a few tiles.
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
INF = math.inf
DEV = "cuda:0"


def log(msg):
    print(f"[gpu-noalloc {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()


def _dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


# (n, d, dtype, scheme, s, q, p), largest first: each call reuses the array
CALLS = [(2, 150_000_011, "f32", "L", 127, 2.0, INF),
         (8, 1_000_003, "f32", "E", 8, 2.0, 2.0),
         (3, 10_007, "bf16", "L", 15, INF, 2.0)]


def test_noalloc_matches_compress_mean_on_consecutive_calls():
    for k, (n, d, dtype, scheme, s, q, p) in enumerate(CALLS):
        log(f"call {k}: n={n} d={d} {dtype} {scheme} s={s} q={q} p={p}")
        assert gq.gq_workspace_bytes(n, d) <= gq.NOALLOC_SCRATCH_BYTES
        x = wl.random_rows(n, d, seed=100 + k, dtype=dtype, scale=0.05)
        xd = _dev(x)
        seed = 0xC0FFEE + k
        W = gq.gq_min_code_bits(n, s, scheme)
        rb = gq.gq_code_row_bytes(d, W)
        # the entry point with a workspace
        mean_a, norm_a, sum_a = gq.gq_compress_mean(xd, s, q, p, scheme, seed, code_bits=W,
                                                    want_code_sum=True)
        # the no-allocation one: outputs preallocated, filled with a pattern
        mean_b = torch.full((d,), float("nan"), dtype=torch.float32, device=DEV)
        norm_b = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
        sum_b = torch.full((rb,), 0xA5, dtype=torch.uint8, device=DEV)
        gq.gq_compress_mean_noalloc(xd, s, q, p, scheme, seed, mean=mean_b, norm=norm_b,
                                    code_bits=W, code_sum=sum_b)
        torch.cuda.synchronize()
        assert torch.equal(norm_a, norm_b), (norm_a.item(), norm_b.item())
        assert torch.equal(sum_a, sum_b)
        assert torch.equal(mean_a.view(torch.int32), mean_b.view(torch.int32))
        # without the code sums, on the same array again
        mean_c = torch.empty_like(mean_b)
        gq.gq_compress_mean_noalloc(xd, s, q, p, scheme, seed, mean=mean_c, norm=norm_b)
        torch.cuda.synchronize()
        assert torch.equal(mean_a.view(torch.int32), mean_c.view(torch.int32))
        del xd, mean_a, mean_b, mean_c, sum_a, sum_b
        torch.cuda.empty_cache()


def test_noalloc_rejects_what_the_array_cannot_hold():
    """A size beyond the array is refused with GQ_ERR_WORKSPACE and nothing
    is launched (the check precedes every HIP call)."""
    x = torch.zeros((3_000_000, 8), dtype=torch.float32, device=DEV)
    assert gq.gq_workspace_bytes(3_000_000, 8) > gq.NOALLOC_SCRATCH_BYTES
    mean = torch.empty(8, dtype=torch.float32, device=DEV)
    norm = torch.empty(1, dtype=torch.float32, device=DEV)
    with pytest.raises(gq.GQError) as e:
        gq.gq_compress_mean_noalloc(x, 3, 2.0, 2.0, "L", 1, mean=mean, norm=norm)
    assert e.value.status == 5

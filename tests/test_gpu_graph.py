"""The library only enqueues kernels (no memset, synchronization or
allocation), so its calls can be captured in a HIP graph and replayed.
Each replay is compared bit-exactly with the eager result, with eager work
and synchronizations between the replays, and the eager result with the
oracle."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import allreduce_compatible_gradient_amd as gq  # noqa: E402
import oracle  # noqa: E402
import workloads as wl  # noqa: E402

pytestmark = pytest.mark.gpu
INF = math.inf
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("n,d,s,q,p,scheme,W", [(4, 70_001, 7, 2.0, 2.0, "L", 6),
                                                (8, 300_000, 127, 2.0, INF, "L", 11),
                                                (16, 50_000, 8, 2.0, 2.0, "E", 13)])
def test_graph_replays_match_eager(n, d, s, q, p, scheme, W):
    x = wl.random_rows(n, d, seed=n + d)
    xd = torch.from_numpy(x).to(DEV)
    ws = torch.empty(gq.gq_workspace_bytes(n, d), dtype=torch.uint8, device=DEV)
    mean = torch.empty(d, dtype=torch.float32, device=DEV)
    norm = torch.empty(1, dtype=torch.float32, device=DEV)
    csum = torch.empty(gq.gq_code_row_bytes(d, W), dtype=torch.uint8, device=DEV)
    codes = torch.empty((n, gq.gq_code_row_bytes(d, W)), dtype=torch.uint8, device=DEV)
    csum2 = torch.empty_like(csum)
    mean2 = torch.empty_like(mean)
    rw = gq.gq_word_row_bytes(d, W) // 4
    words = torch.empty((n, rw), dtype=torch.int32, device=DEV)
    wsum = torch.empty(rw, dtype=torch.int32, device=DEV)
    mean3 = torch.empty_like(mean)
    seed = 1234

    def fused(st):
        gq.gq_compress_mean(xd, s, q, p, scheme, seed, code_bits=W, want_code_sum=True, mean=mean,
                            norm=norm, code_sum=csum, workspace=ws, stream=st)

    def unfused(st):
        gq.gq_quantize(xd, s, scheme, norm, seed, W, codes=codes, stream=st)
        gq.gq_reduce_codes(codes, n, d, W, code_sum=csum2, stream=st)
        gq.gq_dequantize(csum2, n, d, s, scheme, W, norm, mean=mean2, stream=st)
        gq.gq_quantize_words(xd, s, scheme, norm, seed, W, words=words, stream=st)
        gq.gq_sum_words(words, n, d, W, word_sum=wsum, stream=st)
        gq.gq_dequantize_words(wsum, n, d, s, scheme, W, norm, mean=mean3, stream=st)

    cur = torch.cuda.current_stream()
    fused(cur)
    unfused(cur)
    ref = [host(t).copy() for t in (mean, norm, csum, codes, csum2, mean2, words, wsum, mean3)]
    N, sums, omean = oracle.compress_mean(x, s, q, p, oracle.SCHEME_L if scheme == "L" else oracle.SCHEME_E,
                                          seed)
    assert np.float32(ref[1][0]) == N
    assert np.array_equal(ref[0], omean)
    assert np.array_equal(ref[8], omean)  # the word path gives the same mean

    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        fused(side)
        unfused(side)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        fused(side)
        unfused(side)
    for rep in range(3):
        for t in (mean, norm, csum, codes, csum2, mean2, words, wsum, mean3):
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        got = [host(t) for t in (mean, norm, csum, codes, csum2, mean2, words, wsum, mean3)]
        for a, b in zip(ref, got):
            assert np.array_equal(a, b), rep
        fused(cur)  # eager call between replays
        torch.cuda.synchronize()
    del graph


def test_skip_pass_and_noalloc_replay():
    """gq_compress_mean with the zero-code skip (span bounds written by
    pass 1 into the workspace) and the no-allocation entry point (bounds in
    its own scratch), captured together and replayed.  Bounds left in the
    workspace by another input must not leak into a replay; the first 64
    coordinates sit at the top level, so their spans are dense."""
    n, d, s = 40, 30_011, 5
    x = wl.random_rows(n, d, seed=77, scale=0.3)
    x[:, :64] = 3.0  # sums beyond one byte: escapes recomputed from x
    xd = torch.from_numpy(x).to(DEV)
    ws = torch.empty(gq.gq_compress_workspace_bytes(n, d), dtype=torch.uint8, device=DEV)
    assert ws.numel() > gq.gq_workspace_bytes(n, d)  # room for the span bounds
    mean = torch.empty(d, dtype=torch.float32, device=DEV)
    norm = torch.empty(1, dtype=torch.float32, device=DEV)
    mean2 = torch.empty_like(mean)
    norm2 = torch.empty_like(norm)

    def step(st):
        gq.gq_compress_mean(xd, s, INF, INF, "L", 9, mean=mean, norm=norm, workspace=ws, stream=st)
        gq.gq_compress_mean_noalloc(xd, s, INF, INF, "L", 9, mean=mean2, norm=norm2, stream=st)

    N, sums, omean = oracle.compress_mean(x, s, INF, INF, oracle.SCHEME_L, 9)
    assert np.abs(sums).max() > 127  # escapes beside plain bytes
    cur = torch.cuda.current_stream()
    step(cur)
    assert np.float32(host(norm)[0]) == N
    assert np.array_equal(host(mean), omean) and np.array_equal(host(mean2), omean)
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        step(side)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(side)
    other = torch.from_numpy(wl.random_rows(n, d, seed=78, scale=0.3)).to(DEV)
    for rep in range(3):
        # eager work between replays, leaving another input's bounds behind
        gq.gq_compress_mean(other, s, INF, INF, "L", 10, workspace=ws)
        mean.zero_()
        mean2.zero_()
        torch.cuda.synchronize()
        graph.replay()
        assert np.array_equal(host(mean), omean), rep
        assert np.array_equal(host(mean2), omean), rep
    del graph

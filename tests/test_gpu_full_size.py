"""GPU parity at full size: every coordinate of all five workloads.

Each workload is generated once, and each result of the HIP library is
compared with the CPU oracle at every coordinate, bit-exact. The results
come from the launch configuration the benchmark times.

- **Fused path.** The norm, the code sums at the container width and the
  dequantized mean (`gq_compress_mean`, with and without code sums, which
  skips provably zero codes), the same pass reading every coordinate
  (`gq_compress_mean_from_norm`), the span bounds behind the skip
  (`gq_global_norm_bounds`), and the staged step's 1-byte sums and mean
  (`gq_compress_sums8`, `gq_dequantize_sums8`).
- **Unfused path.** Every worker's packed codes (`gq_quantize`) at the
  minimal and at the container width, their integer sum
  (`gq_reduce_codes`), and the mean from it (`gq_dequantize`).
- **Word layout.** Every worker's words (`gq_quantize_words`), their
  word-wise sum (`gq_sum_words`), the one-pass row reading every
  coordinate (`gq_compress_words_from_norm`) and with the zero-code skip
  (`gq_norm_term_bounds`, `gq_compress_words_skip`), and the mean from it
  (`gq_dequantize_words`), all at the minimal width.
- **The pages' 8-bit format.** Every worker's code bytes
  (`gq_e8_quantize`); the root of the re-rounding tree, unfused and fused
  (`gq_e8_tree`, `gq_e8_compress_mean`); and the mean.
- **Local-norm QSGD ablation** (workload 5). The per-worker norms and the
  mean.

Expected values come only from the oracle, run in host threads over blocks
of columns (or rows). Each block is one oracle call, so the threads only
split the work. GPU outputs are compared byte for byte with the oracle's
own packed rows, and never fed back into it.
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
SCH = {"L": oracle.SCHEME_L, "E": oracle.SCHEME_E}
DEV = "cuda:0"
THREADS = oracle._threads(None)


def log(msg):
    print(f"[gpu-full {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gq.lib()


def to_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(x).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same_bytes(a: np.ndarray, b: np.ndarray) -> bool:
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.nbytes == b.nbytes and np.array_equal(a.view(np.uint8).reshape(-1),
                                                   b.view(np.uint8).reshape(-1))


def first_diff(a: np.ndarray, b: np.ndarray) -> str:
    a, b = a.reshape(-1), b.reshape(-1)
    bad = np.flatnonzero(a != b)
    return f"{bad.size} differ, first at {bad[0]}: {a[bad[0]]!r} vs {b[bad[0]]!r}" if bad.size else ""


@pytest.mark.timeout(1800)
@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_every_coordinate(key):
    w = wl.WORKLOADS[key]
    n, d, s, seed, sch = w.n, w.d, w.s, w.seed, SCH[w.scheme]
    M = oracle.top_code(s, sch)
    Wc = w.code_bits
    Wmin = gq.gq_min_code_bits(n, s, w.scheme)
    log(f"workload {key} {w.name}: generating {w.input_bytes / 1e9:.2f} GB ({THREADS} threads)")
    x = wl.generate(w, threads=THREADS)
    xd = to_dev(x)
    compared = 0

    # ---- norm
    N, _ = oracle.global_norm_rows(x, w.q, w.p, threads=THREADS)
    mean_b, norm, _ = gq.gq_compress_mean(xd, s, w.q, w.p, w.scheme, seed)  # benchmarked call
    gN = np.float32(host(norm)[0])
    assert abs(float(gN) - float(N)) <= 1e-6 * float(N), (gN, N)
    assert gN == N, f"norm differs in the last bit: {gN!r} vs {N!r}"

    # ---- fused path at every coordinate
    log("oracle: code sums and mean at every coordinate")
    osums, omean = oracle.compress_mean_all(x, N, s, sch, seed, threads=THREADS)
    assert np.abs(osums).max() <= n * M
    gmean = host(mean_b)
    assert same_bytes(gmean, omean), first_diff(gmean.view(np.uint32), omean.view(np.uint32))
    compared += d
    # the same pass reading every coordinate (the benchmarked call above
    # skips the groups whose codes are provably zero)
    dmean, _ = gq.gq_compress_mean_from_norm(xd, s, w.scheme, seed, norm)
    assert same_bytes(host(dmean), omean), "the pass without the zero-code skip differs"
    del dmean
    compared += d
    # the span bounds pass 1 wrote with the norm: the bf16 rounding-up of each
    # 512-coordinate span's largest |x|, every entry
    nb, bounds = gq.gq_global_norm_bounds(xd, w.q, w.p)
    assert np.float32(host(nb)[0]) == N
    spans, stride = -(-d // 512), -(-d // 8192) * 16
    gb = host(bounds)[: 2 * n * stride].view(np.uint16).reshape(n, stride)[:, :spans]
    bad_b = []

    def bound_rows(i0, i1):
        step = 1 << 24  # coordinates per slice (a multiple of 512)
        for i in range(i0, i1):
            for j in range(0, d, step):
                je = min(d, j + step)
                seg = x[i, j:je]
                bits = (seg.astype(np.uint32) << np.uint32(16)) if x.dtype == np.uint16 else seg.view(np.uint32)
                k = -(-(je - j) // 512)
                row = np.zeros(k * 512, dtype=np.uint32)
                row[:je - j] = bits & np.uint32(0x7FFFFFFF)
                m = row.reshape(k, 512).max(axis=1).astype(np.uint64)
                if not np.array_equal(gb[i, j // 512:j // 512 + k], ((m + 0xFFFF) >> 16).astype(np.uint16)):
                    bad_b.append((i, j))

    oracle.run_blocks(bound_rows, [(i, i + 1) for i in range(n)], THREADS)
    assert not bad_b, f"span bounds differ in rows {bad_b[:8]}"
    del bounds, gb
    mean_c, _, csum = gq.gq_compress_mean(xd, s, w.q, w.p, w.scheme, seed, code_bits=Wc,
                                          want_code_sum=True)
    assert same_bytes(host(mean_c), omean)
    exp_c = oracle.pack_row(osums, Wc, threads=THREADS)
    assert same_bytes(host(csum), exp_c), "fused code sums differ"
    del mean_c, csum
    # the staged compress step's two kernels: the group mask and the 1-byte
    # sums of the marked groups (escape -128), then the mean
    b8 = gq.gq_compress_sums8(xd, s, w.scheme, seed, norm)
    groups = -(-d // 8)
    words = -(-d // 512)
    mb = (words * 8 + 15) // 16 * 16
    hb8 = host(b8)
    bits = np.unpackbits(hb8[:words * 8], bitorder="little")
    padded = np.zeros(groups * 8, np.int64)
    padded[:d] = osums
    nzg = (padded.reshape(groups, 8) != 0).any(axis=1)
    del padded
    assert np.array_equal(bits[:groups].astype(bool), nzg) and not bits[groups:].any()
    cols = np.flatnonzero(np.repeat(nzg, 8)[:d])
    want8 = np.where(np.abs(osums[cols]) <= 127, osums[cols], -128).astype(np.int8)
    assert np.array_equal(hb8[mb:mb + d].view(np.int8)[cols], want8), "staged 1-byte sums differ"
    log(f"staged sums: {nzg.mean():.4f} of the 8-coordinate groups are non-zero")
    assert same_bytes(host(gq.gq_dequantize_sums8(xd, s, w.scheme, seed, norm, b8)), omean)
    compared += 2 * d
    del b8, hb8, want8, cols, bits, nzg

    # ---- unfused path and word layout: every worker's row
    widths = sorted({Wmin, Wc})
    gcodes = {W: host(gq.gq_quantize(xd, s, w.scheme, norm, seed, W)) for W in widths}
    gwords = host(gq.gq_quantize_words(xd, s, w.scheme, norm, seed, Wmin)).view(np.uint32)
    e8n = n & (n - 1) == 0
    if e8n:
        ge8 = host(gq.gq_e8_quantize(xd, norm, seed))
    owords = np.zeros(gwords.shape, dtype=np.uint32)
    bad_rows = []

    def row(i, _):
        c = oracle.quantize(x[i:i + 1], N, s, sch, seed, worker_base=i)
        for W in widths:
            if not same_bytes(gcodes[W][i], oracle.pack(c, W)[0]):
                bad_rows.append(("codes", W, i))
        owords[i] = oracle.pack_words(c, Wmin, M)[0]
        if not np.array_equal(gwords[i], owords[i]):
            bad_rows.append(("words", Wmin, i))
        if e8n:
            e = oracle.e8_quantize(x[i:i + 1], N, seed, worker_base=i)[0]
            if not np.array_equal(ge8[i, :d], e):
                bad_rows.append(("e8 codes", 8, i))

    log(f"oracle: {n} rows of codes at W = {widths}, words at W = {Wmin}"
        + (", 8-bit codes" if e8n else ""))
    oracle.run_blocks(row, [(i, i + 1) for i in range(n)], THREADS)
    assert not bad_rows, bad_rows[:8]
    compared += n * d * (len(widths) + 1 + (1 if e8n else 0))

    # the integer sum of the codes and the mean from it, at both widths
    for W in widths:
        codes_dev = torch.from_numpy(gcodes[W]).to(DEV)
        rsum = gq.gq_reduce_codes(codes_dev, n, d, W)
        exp = exp_c if W == Wc else oracle.pack_row(osums, W, threads=THREADS)
        assert same_bytes(host(rsum), exp), f"reduced code sums differ at W = {W}"
        dmean = gq.gq_dequantize(rsum, n, d, s, w.scheme, W, norm)
        assert same_bytes(host(dmean), omean), f"dequantized mean differs at W = {W}"
        del codes_dev, rsum, dmean
    compared += 2 * d * len(widths)
    del gcodes

    # the word-wise sum, the one-pass row and the mean from the words
    log("oracle: word-wise sum of the rows")
    owsum = oracle.sum_words_all(owords, threads=THREADS)
    wsum = gq.gq_sum_words(torch.from_numpy(gwords.view(np.int32)).to(DEV), n, d, Wmin)
    assert np.array_equal(host(wsum).view(np.uint32), owsum), "summed words differ"
    one = gq.gq_compress_words_from_norm(xd, s, w.scheme, norm, seed, Wmin)
    assert np.array_equal(host(one).view(np.uint32), owsum), "one-pass word row differs"
    _, tb = gq.gq_norm_term_bounds(xd, w.q, w.p)
    skip = gq.gq_compress_words_skip(xd, s, w.scheme, norm, tb, seed, Wmin)
    assert np.array_equal(host(skip).view(np.uint32), owsum), "skipped word row differs"
    wmean = gq.gq_dequantize_words(one, n, d, s, w.scheme, Wmin, norm)
    assert same_bytes(host(wmean), omean), "mean from the words differs"
    compared += 4 * d
    del gwords, owords, wsum, one, wmean, skip, tb

    # ---- the pages' 8-bit format: root of the re-rounding tree and the mean
    if e8n:
        log("oracle: 8-bit tree root and mean at every coordinate")
        oroot, oemean = oracle.e8_compress_all(x, N, seed, threads=THREADS)
        root = gq.gq_e8_tree(torch.from_numpy(ge8).to(DEV), n, d, seed)
        assert np.array_equal(host(root)[:d], oroot), "8-bit tree root differs"
        fmean, fnorm, froot = gq.gq_e8_compress_mean(xd, w.q, w.p, seed, want_root=True)
        assert np.float32(host(fnorm)[0]) == N
        assert np.array_equal(host(froot)[:d], oroot), "fused 8-bit root differs"
        assert same_bytes(host(fmean), oemean), "8-bit mean differs"
        compared += 3 * d
        del ge8, root, fmean, froot

    # ---- the local-norm ablation
    if key == 5:
        log("oracle: local norms and the ablation's mean at every coordinate")
        onorms = oracle.local_norms(x, threads=THREADS)
        lmean, lnorms, _ = gq.gq_qsgd_local_mean(xd, s, seed)
        assert same_bytes(host(lnorms), onorms), "local norms differ"
        olmean = oracle.qsgd_local_all(x, onorms, s, seed, threads=THREADS)
        assert same_bytes(host(lmean), olmean), "ablation mean differs"
        compared += d

    log(f"workload {key} ok: {compared} values compared bit for bit "
        f"(n d = {n * d}; every coordinate of every result)")
    del xd, x
    torch.cuda.empty_cache()

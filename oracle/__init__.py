"""CPU oracle for the Global-QSGD compression operator -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``allreduce_compatible_gradient_amd``) never does, and shares no code with
it: the arithmetic lives in ``gq_oracle.c`` (plain scalar C), and this module
only marshals numpy arrays into it.

Method: "Global-QSGD: Practical Floatless Quantization for Distributed
Learning with Theoretical Guarantees" -- Sec. 2 for the (q,p)-norm, Sec. 3 for
Global-Q and its two level families (standard dithering Global-L_s,
exponential dithering Global-E_s), Sec. 6 for the quantize / integer
Allreduce / dequantize pipeline.  The exact rules each function follows are
written next to the C function it calls.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gq_oracle.c")
_LIB_PATH = os.environ.get("GQ_ORACLE_LIB") or os.path.join(_HERE, "libgq_oracle.so")

SCHEME_L = 0
SCHEME_E = 1
F32 = 0
BF16 = 1

_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_int = ctypes.c_int
_f32 = ctypes.c_float
_vp = ctypes.c_void_p


def build() -> str:
    """Compile gq_oracle.c with gcc into libgq_oracle.so (plain C11, no FP contraction)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", _SRC, "-o", _LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_philox4x32_10.argtypes = [_vp, _vp, _vp]
        L.oracle_uniform32.argtypes = [_u64, _u64, _u64]
        L.oracle_uniform32.restype = ctypes.c_uint32
        L.oracle_global_norm.argtypes = [_vp, _int, _i64, _i64, _f32, _f32, _vp]
        L.oracle_global_norm.restype = _f32
        L.oracle_norm_from_partials.argtypes = [_vp, _i64, _f32, _f32]
        L.oracle_norm_from_partials.restype = _f32
        L.oracle_top_code.argtypes = [_int, _int]
        L.oracle_top_code.restype = _i64
        L.oracle_scale_params.argtypes = [_f32, _i64, _int, _int, _vp, _vp, _vp]
        L.oracle_bracket.argtypes = [_f32, _f32, _f32, _int, _int, _int, _vp, _vp, _vp]
        L.oracle_code.argtypes = [_f32, _f32, _f32, _int, _int, _int, ctypes.c_uint32]
        L.oracle_code.restype = ctypes.c_int32
        L.oracle_quantize.argtypes = [_vp, _int, _i64, _i64, _f32, _int, _int, _u64, _i64, _vp]
        L.oracle_min_code_bits.argtypes = [_i64, _int, _int]
        L.oracle_min_code_bits.restype = _int
        L.oracle_row_bytes.argtypes = [_i64, _int]
        L.oracle_row_bytes.restype = _i64
        L.oracle_pack.argtypes = [_vp, _i64, _i64, _int, _vp]
        L.oracle_unpack.argtypes = [_vp, _i64, _i64, _int, _vp]
        L.oracle_sum_codes.argtypes = [_vp, _i64, _i64, _vp]
        L.oracle_word_fields.argtypes = [_int]
        L.oracle_word_row_bytes.argtypes = [_i64, _int]
        L.oracle_word_row_bytes.restype = _i64
        L.oracle_pack_words.argtypes = [_vp, _i64, _i64, _int, _i64, _vp]
        L.oracle_sum_words.argtypes = [_vp, _i64, _i64, _vp]
        L.oracle_unpack_word_sums.argtypes = [_vp, _i64, _i64, _int, _i64, _vp]
        L.oracle_dequantize.argtypes = [_vp, _i64, _i64, _f32, _int, _int, _vp]
        L.oracle_compress_mean_cols.argtypes = [_vp, _int, _i64, _i64, _f32, _int, _int, _u64,
                                                _vp, _i64, _vp, _vp]
        L.oracle_compress_mean.argtypes = [_vp, _int, _i64, _i64, _int, _f32, _f32, _int, _u64,
                                           _vp, _vp]
        L.oracle_compress_mean.restype = _f32
        L.oracle_uniform32_ctr.argtypes = [_u64, ctypes.c_uint32, ctypes.c_uint32, _u64]
        L.oracle_uniform32_ctr.restype = ctypes.c_uint32
        L.oracle_e8_value.argtypes = [ctypes.c_uint8]
        L.oracle_e8_value.restype = ctypes.c_double
        L.oracle_e8_round.argtypes = [ctypes.c_double, ctypes.c_uint32]
        L.oracle_e8_round.restype = ctypes.c_uint8
        L.oracle_e8_quantize.argtypes = [_vp, _int, _i64, _i64, _f32, _u64, _i64, _vp]
        L.oracle_e8_reduce_pair.argtypes = [_vp, _vp, _i64, _u64, ctypes.c_uint32, ctypes.c_uint32,
                                            _vp]
        L.oracle_e8_tree.argtypes = [_vp, _i64, _i64, _u64, _vp, _vp]
        L.oracle_e8_tree.restype = _int
        L.oracle_e8_dequantize.argtypes = [_vp, _i64, _f32, _vp]
        L.oracle_e8_compress_cols.argtypes = [_vp, _int, _i64, _i64, _f32, _u64, _vp, _i64, _vp,
                                              _vp]
        L.oracle_local_norms.argtypes = [_vp, _int, _i64, _i64, _vp]
        L.oracle_qsgd_local_cols.argtypes = [_vp, _int, _i64, _i64, _int, _u64, _vp, _vp, _i64,
                                             _vp, _vp]
        L.oracle_qsgd_local_mean.argtypes = [_vp, _int, _i64, _i64, _int, _u64, _vp, _vp, _vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp)


def _x_dtype(x: np.ndarray) -> int:
    """fp32 arrays are fp32; uint16 arrays carry bf16 bit patterns."""
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs are float32 or bf16 bits in uint16, got {x.dtype}")


def _rows(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    if x.ndim != 2:
        raise ValueError("x must be [n, d]")
    return x


def _order(v) -> float:
    v = float(v)
    if v >= 1.0:  # a real >= 1 or +inf
        return v
    raise ValueError("q and p are reals >= 1 or inf")


# ---------------------------------------------------------------------------
# Random numbers


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform32(seed: int, worker: int, j: int) -> int:
    return int(lib().oracle_uniform32(seed, worker, j))


# ---------------------------------------------------------------------------
# Norm, scalars, bracketing


def global_norm(x: np.ndarray, q, p):
    """Returns (N as np.float32, per-worker partials: sum of squares or max |x|)."""
    x = _rows(x)
    n, d = x.shape
    pw = np.zeros(n, dtype=np.float64)
    N = lib().oracle_global_norm(_ptr(x), _x_dtype(x), n, d, _order(q), _order(p), _ptr(pw))
    return np.float32(N), pw


def global_norm_rows(x: np.ndarray, q, p, threads: int = 1):
    """global_norm computed one row at a time (rows in parallel threads), then combined.

    Same arithmetic as global_norm: each row's partial is its own oracle call."""
    from concurrent.futures import ThreadPoolExecutor
    x = _rows(x)
    n = x.shape[0]
    pw = np.zeros(n, dtype=np.float64)

    def one(i):
        pw[i] = global_norm(x[i:i + 1], q, p)[1][0]

    if threads > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    else:
        for i in range(n):
            one(i)
    N = lib().oracle_norm_from_partials(_ptr(pw), n, _order(q), _order(p))
    return np.float32(N), pw


def top_code(s: int, scheme: int) -> int:
    return int(lib().oracle_top_code(s, scheme))


def scale_params(N, n: int, s: int, scheme: int):
    """(pre, sigma, kappa) for a norm N: pre-scale, fp32 scale, fp64 dequant factor."""
    pre = np.zeros(1, np.float32)
    sig = np.zeros(1, np.float32)
    kap = np.zeros(1, np.float64)
    lib().oracle_scale_params(float(N), n, s, scheme, _ptr(pre), _ptr(sig), _ptr(kap))
    return pre[0], sig[0], kap[0]


def bracket(xv, N, n: int, s: int, scheme: int):
    """(m_lo, m_hi, F): the two candidate code magnitudes and the 32-bit threshold.

    The code magnitude is m_hi with probability F / 2^32, else m_lo."""
    pre, sig, _ = scale_params(N, n, s, scheme)
    lo = np.zeros(1, np.int32)
    hi = np.zeros(1, np.int32)
    F = np.zeros(1, np.uint32)
    lib().oracle_bracket(float(np.float32(xv)), float(pre), float(sig), int(np.float32(N) == 0),
                         s, scheme, _ptr(lo), _ptr(hi), _ptr(F))
    return int(lo[0]), int(hi[0]), int(F[0])


def code(xv, N, n: int, s: int, scheme: int, u: int) -> int:
    pre, sig, _ = scale_params(N, n, s, scheme)
    return int(lib().oracle_code(float(np.float32(xv)), float(pre), float(sig),
                                 int(np.float32(N) == 0), s, scheme, u))


# ---------------------------------------------------------------------------
# Pipeline pieces


def quantize(x: np.ndarray, N, s: int, scheme: int, seed: int, worker_base: int = 0) -> np.ndarray:
    x = _rows(x)
    n, d = x.shape
    codes = np.zeros((n, d), dtype=np.int32)
    lib().oracle_quantize(_ptr(x), _x_dtype(x), n, d, float(N), s, scheme, seed, worker_base,
                          _ptr(codes))
    return codes


def min_code_bits(n: int, s: int, scheme: int) -> int:
    return int(lib().oracle_min_code_bits(n, s, scheme))


def row_bytes(d: int, W: int) -> int:
    return int(lib().oracle_row_bytes(d, W))


def pack(codes: np.ndarray, W: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int32)
    if codes.ndim == 1:
        codes = codes.reshape(1, -1)
    n, d = codes.shape
    out = np.zeros((n, row_bytes(d, W)), dtype=np.uint8)
    lib().oracle_pack(_ptr(codes), n, d, W, _ptr(out))
    return out


def unpack(packed: np.ndarray, n: int, d: int, W: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    if packed.size != n * row_bytes(d, W):
        raise ValueError("packed buffer has the wrong size")
    codes = np.zeros((n, d), dtype=np.int32)
    lib().oracle_unpack(_ptr(packed), n, d, W, _ptr(codes))
    return codes


def sum_codes(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int32)
    n, d = codes.shape
    sums = np.zeros(d, dtype=np.int64)
    lib().oracle_sum_codes(_ptr(codes), n, d, _ptr(sums))
    return sums


def word_fields(W: int) -> int:
    """Fields per 32-bit word of the word layout: floor(32 / W)."""
    return int(lib().oracle_word_fields(W))


def word_row_bytes(d: int, W: int) -> int:
    return int(lib().oracle_word_row_bytes(d, W))


def pack_words(codes: np.ndarray, W: int, M: int) -> np.ndarray:
    """Codes [n][d] in the word layout (fields of code + M): uint32 [n][row words]."""
    codes = np.ascontiguousarray(codes, dtype=np.int32)
    if codes.ndim == 1:
        codes = codes.reshape(1, -1)
    n, d = codes.shape
    out = np.zeros((n, word_row_bytes(d, W) // 4), dtype=np.uint32)
    lib().oracle_pack_words(_ptr(codes), n, d, W, M, _ptr(out))
    return out


def sum_words(rows: np.ndarray) -> np.ndarray:
    """Word-wise uint32 sum of the rows (modulo 2^32), as a native SUM does it."""
    rows = np.ascontiguousarray(rows, dtype=np.uint32)
    n, nw = rows.shape
    out = np.zeros(nw, dtype=np.uint32)
    lib().oracle_sum_words(_ptr(rows), n, nw, _ptr(out))
    return out


def unpack_word_sums(word_sum: np.ndarray, n: int, d: int, W: int, M: int) -> np.ndarray:
    """Exact code sums [d] (int64) from a summed row of n rows in the word layout."""
    word_sum = np.ascontiguousarray(word_sum, dtype=np.uint32)
    if word_sum.size * 4 != word_row_bytes(d, W):
        raise ValueError("summed row has the wrong size")
    sums = np.zeros(d, dtype=np.int64)
    lib().oracle_unpack_word_sums(_ptr(word_sum), n, d, W, M, _ptr(sums))
    return sums


def dequantize(sums: np.ndarray, n: int, N, s: int, scheme: int) -> np.ndarray:
    sums = np.ascontiguousarray(sums, dtype=np.int64)
    mean = np.zeros(sums.shape[0], dtype=np.float32)
    lib().oracle_dequantize(_ptr(sums), n, sums.shape[0], float(N), s, scheme, _ptr(mean))
    return mean


def compress_mean(x: np.ndarray, s: int, q, p, scheme: int, seed: int):
    """Whole pipeline. Returns (N, sums int64 [d], mean float32 [d])."""
    x = _rows(x)
    n, d = x.shape
    sums = np.zeros(d, dtype=np.int64)
    mean = np.zeros(d, dtype=np.float32)
    N = lib().oracle_compress_mean(_ptr(x), _x_dtype(x), n, d, s, _order(q), _order(p), scheme,
                                   seed, _ptr(sums), _ptr(mean))
    return np.float32(N), sums, mean


def compress_mean_cols(x: np.ndarray, N, s: int, scheme: int, seed: int, cols) -> tuple:
    """Selected coordinates of the pipeline given the norm: (sums int64, mean float32)."""
    x = _rows(x)
    n, d = x.shape
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if cols.size and (cols.min() < 0 or cols.max() >= d):
        raise IndexError("column out of range")
    sums = np.zeros(cols.size, dtype=np.int64)
    mean = np.zeros(cols.size, dtype=np.float32)
    lib().oracle_compress_mean_cols(_ptr(x), _x_dtype(x), n, d, float(N), s, scheme, seed,
                                    _ptr(cols), cols.size, _ptr(sums), _ptr(mean))
    return sums, mean


# ---------------------------------------------------------------------------
# Whole rows in parallel host threads: the same oracle calls over blocks of
# columns (or rows), gathered in place.  Threads only split the work; each
# block is one call of the function above it, so the results are those of a
# single call over every column.

def _threads(threads: int | None) -> int:
    if threads:
        return max(1, int(threads))
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


def col_blocks(d: int, threads: int | None = None, align: int = 128):
    """[a, b) column ranges covering [0, d): starts are multiples of align
    (so that W-bit packed rows split at whole bytes), about 4 per thread."""
    t = _threads(threads)
    want = max(1, 4 * t)
    step = max(align, -(-d // want))
    step = -(-step // align) * align
    return [(a, min(d, a + step)) for a in range(0, d, step)]


def run_blocks(fn, blocks, threads: int | None = None):
    """fn(a, b) over every block, in a pool of host threads (ctypes calls
    release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    t = _threads(threads)
    if t == 1 or len(blocks) <= 1:
        for a, b in blocks:
            fn(a, b)
        return
    with ThreadPoolExecutor(max_workers=t) as ex:
        for f in [ex.submit(fn, a, b) for a, b in blocks]:
            f.result()


def compress_mean_all(x: np.ndarray, N, s: int, scheme: int, seed: int,
                      threads: int | None = None, d_end: int | None = None):
    """compress_mean_cols over every column in [0, d_end) (default d), split
    into column blocks run in host threads: (sums int64, mean float32)."""
    x = _rows(x)
    n, d = x.shape
    d_end = d if d_end is None else d_end
    sums = np.zeros(d_end, dtype=np.int64)
    mean = np.zeros(d_end, dtype=np.float32)
    dt = _x_dtype(x)

    def one(a, b):
        cols = np.arange(a, b, dtype=np.int64)
        lib().oracle_compress_mean_cols(_ptr(x), dt, n, d, float(N), s, scheme, seed,
                                        _ptr(cols), b - a, _ptr(sums[a:b]), _ptr(mean[a:b]))

    run_blocks(one, col_blocks(d_end, threads), threads)
    return sums, mean


def e8_compress_all(x: np.ndarray, N, seed: int, threads: int | None = None):
    """e8_compress_cols over every column, in column blocks: (root, mean)."""
    x = _rows(x)
    n, d = x.shape
    if n & (n - 1):
        raise ValueError("the tree needs a power-of-two number of rows")
    root = np.zeros(d, dtype=np.uint8)
    mean = np.zeros(d, dtype=np.float32)
    dt = _x_dtype(x)

    def one(a, b):
        cols = np.arange(a, b, dtype=np.int64)
        lib().oracle_e8_compress_cols(_ptr(x), dt, n, d, float(N), seed, _ptr(cols), b - a,
                                      _ptr(root[a:b]), _ptr(mean[a:b]))

    run_blocks(one, col_blocks(d, threads), threads)
    return root, mean


def qsgd_local_all(x: np.ndarray, norms: np.ndarray, s: int, seed: int,
                   threads: int | None = None):
    """The ablation's mean at every column given the norms, in column blocks."""
    x = _rows(x)
    n, d = x.shape
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    mean = np.zeros(d, dtype=np.float32)
    dt = _x_dtype(x)

    def one(a, b):
        cols = np.arange(a, b, dtype=np.int64)
        lib().oracle_qsgd_local_cols(_ptr(x), dt, n, d, s, seed, _ptr(norms), _ptr(cols), b - a,
                                     None, _ptr(mean[a:b]))

    run_blocks(one, col_blocks(d, threads), threads)
    return mean


def pack_row(values: np.ndarray, W: int, threads: int | None = None) -> np.ndarray:
    """pack of one row of d values, in 128-column blocks (each block's W-bit
    fields fill whole 16-byte units, so the blocks' bytes concatenate)."""
    values = np.ascontiguousarray(values, dtype=np.int32).reshape(-1)
    d = values.size
    out = np.zeros(row_bytes(d, W), dtype=np.uint8)

    def one(a, b):
        part = pack(values[a:b], W)[0]
        out[a * W // 8: a * W // 8 + part.size] = part

    run_blocks(one, col_blocks(d, threads), threads)
    return out


def sum_words_all(rows: np.ndarray, threads: int | None = None) -> np.ndarray:
    """sum_words over blocks of words, in host threads."""
    rows = np.ascontiguousarray(rows, dtype=np.uint32)
    n, nw = rows.shape
    out = np.zeros(nw, dtype=np.uint32)

    def one(a, b):
        out[a:b] = sum_words(np.ascontiguousarray(rows[:, a:b]))

    run_blocks(one, col_blocks(nw, threads, align=1), threads)
    return out


def qsgd_local_mean(x: np.ndarray, s: int, seed: int):
    """Local-norm QSGD ablation. Returns (norms float32 [n], codes int32 [n, d], mean [d])."""
    x = _rows(x)
    n, d = x.shape
    norms = np.zeros(n, dtype=np.float32)
    codes = np.zeros((n, d), dtype=np.int32)
    mean = np.zeros(d, dtype=np.float32)
    lib().oracle_qsgd_local_mean(_ptr(x), _x_dtype(x), n, d, s, seed, _ptr(norms), _ptr(codes),
                                 _ptr(mean))
    return norms, codes, mean


def local_norms(x: np.ndarray, threads: int = 1) -> np.ndarray:
    """Per-worker l2 norms of the ablation, fp32 [n] (rows in parallel threads)."""
    from concurrent.futures import ThreadPoolExecutor
    x = _rows(x)
    n, d = x.shape
    norms = np.zeros(n, dtype=np.float32)

    def one(i):
        r = np.ascontiguousarray(x[i:i + 1])
        out = np.zeros(1, dtype=np.float32)
        lib().oracle_local_norms(_ptr(r), _x_dtype(r), 1, d, _ptr(out))
        norms[i] = out[0]

    if threads > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(one, range(n)))
    else:
        for i in range(n):
            one(i)
    return norms


def qsgd_local_cols(x: np.ndarray, norms: np.ndarray, s: int, seed: int, cols):
    """Selected coordinates of the ablation given the norms: (codes int32 [n, k], mean [k])."""
    x = _rows(x)
    n, d = x.shape
    norms = np.ascontiguousarray(norms, dtype=np.float32)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if cols.size and (cols.min() < 0 or cols.max() >= d):
        raise IndexError("column out of range")
    codes = np.zeros((n, cols.size), dtype=np.int32)
    mean = np.zeros(cols.size, dtype=np.float32)
    lib().oracle_qsgd_local_cols(_ptr(x), _x_dtype(x), n, d, s, seed, _ptr(norms), _ptr(cols),
                                 cols.size, _ptr(codes), _ptr(mean))
    return codes, mean


# ---------------------------------------------------------------------------
# The pages' 8-bit exponential-dithering wire format and its tree reduction


def uniform32_ctr(seed: int, c2: int, c3pair: int, j: int) -> int:
    return int(lib().oracle_uniform32_ctr(seed, c2, c3pair, j))


def e8_value(c: int) -> float:
    return float(lib().oracle_e8_value(c))


def e8_round(v: float, u: int) -> int:
    return int(lib().oracle_e8_round(float(v), u))


def e8_quantize(x: np.ndarray, N, seed: int, worker_base: int = 0) -> np.ndarray:
    x = _rows(x)
    n, d = x.shape
    codes = np.zeros((n, d), dtype=np.uint8)
    lib().oracle_e8_quantize(_ptr(x), _x_dtype(x), n, d, float(N), seed, worker_base, _ptr(codes))
    return codes


def e8_reduce_pair(a: np.ndarray, b: np.ndarray, seed: int, level: int, node: int) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.zeros(a.size, dtype=np.uint8)
    lib().oracle_e8_reduce_pair(_ptr(a), _ptr(b), a.size, seed, level, node, _ptr(out))
    return out


def e8_tree(codes: np.ndarray, seed: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, d = codes.shape
    root = np.zeros(d, dtype=np.uint8)
    scratch = np.zeros(n * d, dtype=np.uint8)
    if lib().oracle_e8_tree(_ptr(codes), n, d, seed, _ptr(root), _ptr(scratch)) != 0:
        raise ValueError("the tree needs a power-of-two number of rows")
    return root


def e8_dequantize(root: np.ndarray, N) -> np.ndarray:
    root = np.ascontiguousarray(root, dtype=np.uint8)
    mean = np.zeros(root.size, dtype=np.float32)
    lib().oracle_e8_dequantize(_ptr(root), root.size, float(N), _ptr(mean))
    return mean


def e8_compress_mean(x: np.ndarray, q, p, seed: int):
    """Norm, 8-bit codes, tree reduction with re-rounding, dequantization: (N, root, mean)."""
    N, _ = global_norm(x, q, p)
    codes = e8_quantize(x, N, seed)
    root = e8_tree(codes, seed)
    return N, root, e8_dequantize(root, N)


def e8_compress_cols(x: np.ndarray, N, seed: int, cols):
    """Listed coordinates of the 8-bit pipeline given the norm (n a power of two): (root, mean)."""
    x = _rows(x)
    n, d = x.shape
    if n & (n - 1):
        raise ValueError("the tree needs a power-of-two number of rows")
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if cols.size and (cols.min() < 0 or cols.max() >= d):
        raise IndexError("column out of range")
    root = np.zeros(cols.size, dtype=np.uint8)
    mean = np.zeros(cols.size, dtype=np.float32)
    lib().oracle_e8_compress_cols(_ptr(x), _x_dtype(x), n, d, float(N), seed, _ptr(cols), cols.size,
                                  _ptr(root), _ptr(mean))
    return root, mean

"""The C ABI on the CPU: the library loads, exports what include/gq.h
declares, and rejects bad arguments before touching the device."""
import ctypes
import math
import os
import re

import pytest

import allreduce_compatible_gradient_amd as gq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gq_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = gq.lib()
    names = _declared()
    assert "gq_compress_mean" in names and len(names) >= 12
    for name in names:
        assert hasattr(L, name), name
        assert name in gq.SIGNATURES, name


def test_status_strings():
    L = gq.lib()
    for code, name in gq.STATUS.items():
        assert L.gq_status_str(code).decode() == name


def test_size_helpers_match_the_oracle():
    for n in (1, 2, 4, 8, 16, 64, 1000):
        for s in (1, 3, 7, 15, 127):
            assert gq.gq_min_code_bits(n, s, "L") == oracle.min_code_bits(n, s, oracle.SCHEME_L)
        for s in (1, 4, 8, 12):
            assert gq.gq_min_code_bits(n, s, "E") == oracle.min_code_bits(n, s, oracle.SCHEME_E)
    for d in (0, 1, 7, 8, 65536, 25_557_032):
        for W in (2, 6, 8, 9, 11, 13, 16, 31, 32):
            assert gq.gq_code_row_bytes(d, W) == oracle.row_bytes(d, W)
    assert gq.gq_min_code_bits(0, 3, "L") == -1
    assert gq.gq_min_code_bits(2, 0, "L") == -1
    assert gq.gq_min_code_bits(2, 32, "E") == -1
    assert gq.gq_code_row_bytes(10, 33) == -1
    assert gq.gq_workspace_bytes(8, 25_557_032) > 0
    assert gq.gq_workspace_bytes(0, 5) == -1


# Fake device pointers: every call below fails validation before any HIP call.
A = ctypes.c_void_p(0x10000)   # 16-byte aligned
U = ctypes.c_void_p(0x10004)   # misaligned
NUL = None
WS = gq.gq_workspace_bytes(4, 1000)


def _err(status):
    return gq.STATUS[status]


@pytest.mark.parametrize("args,expect", [
    ((NUL, 0, 4, 1000, 2.0, 2.0, A, A, WS, NUL), 1),      # x NULL
    ((A, 0, 4, 1000, 2.0, 2.0, NUL, A, WS, NUL), 1),      # norm NULL
    ((A, 5, 4, 1000, 2.0, 2.0, A, A, WS, NUL), 2),        # dtype
    ((A, 0, 0, 1000, 2.0, 2.0, A, A, WS, NUL), 2),        # n = 0
    ((A, 0, 4, -1, 2.0, 2.0, A, A, WS, NUL), 2),          # d < 0
    ((A, 0, 1 << 30, 1 << 40, 2.0, 2.0, A, A, WS, NUL), 2),  # n d overflow
    ((A, 0, 4, 1000, 0.5, 2.0, A, A, WS, NUL), 3),        # q < 1
    ((A, 0, 4, 1000, 2.0, 0.99, A, A, WS, NUL), 3),       # p < 1
    ((A, 0, 4, 1000, math.nan, 2.0, A, A, WS, NUL), 3),   # q NaN
    ((A, 0, 4, 1000, 2.0, -math.inf, A, A, WS, NUL), 3),  # p = -inf
    ((U, 0, 4, 1000, 2.0, 2.0, A, A, WS, NUL), 6),        # x misaligned
    ((A, 0, 4, 1000, 2.0, 2.0, A, A, WS - 1, NUL), 5),    # workspace too small
    ((A, 0, 4, 1000, 2.0, 2.0, A, NUL, WS, NUL), 1),      # workspace NULL
])
def test_global_norm_rejects(args, expect):
    assert gq.lib().gq_global_norm(*args) == expect
    assert gq.lib().gq_last_error().decode() != ""


@pytest.mark.parametrize("args,expect", [
    ((NUL, 0, 4, 1000, 2.0, 2.0, A, A, WS, NUL), 1),      # x NULL
    ((A, 0, 4, 1000, 2.0, 2.0, NUL, A, WS, NUL), 1),      # term NULL
    ((A, 5, 4, 1000, 2.0, 2.0, A, A, WS, NUL), 2),        # dtype
    ((A, 0, 0, 1000, 2.0, 2.0, A, A, WS, NUL), 2),        # n = 0
    ((A, 0, 4, 1000, 0.5, 2.0, A, A, WS, NUL), 3),        # q < 1
    ((A, 0, 4, 1000, 2.0, math.nan, A, A, WS, NUL), 3),   # p NaN
    ((U, 0, 4, 1000, 2.0, 2.0, A, A, WS, NUL), 6),        # x misaligned
    ((A, 0, 4, 1000, 2.0, 2.0, A, A, WS - 1, NUL), 5),    # workspace too small
])
def test_norm_term_rejects(args, expect):
    assert gq.lib().gq_norm_term(*args) == expect
    assert gq.lib().gq_last_error().decode() != ""


def test_norm_from_term_rejects():
    L = gq.lib()
    assert L.gq_norm_from_term(NUL, 2.0, 2.0, A, NUL) == 1
    assert L.gq_norm_from_term(A, 2.0, 2.0, NUL, NUL) == 1
    assert L.gq_norm_from_term(A, 0.5, 2.0, A, NUL) == 3
    assert L.gq_norm_from_term(A, 2.0, -math.inf, A, NUL) == 3


@pytest.mark.parametrize("args,expect", [
    ((A, 0, 4, 100, 0, 0, A, 1, 0, 8, A, NUL), 2),        # s = 0
    ((A, 0, 4, 100, 7, 2, A, 1, 0, 8, A, NUL), 2),        # scheme 2
    ((A, 0, 4, 100, 32, 1, A, 1, 0, 32, A, NUL), 2),      # E with s = 32
    ((A, 0, 4, 100, 7, 0, A, 1, 0, 5, A, NUL), 4),        # W below W_min = 6
    ((A, 0, 4, 100, 7, 0, A, 1, 0, 33, A, NUL), 4),       # W above 32
    ((A, 0, 1 << 28, 100, 127, 0, A, 1, 0, 32, A, NUL), 4),  # n s needs > 32 bits
    ((A, 0, 4, 100, 7, 0, NUL, 1, 0, 8, A, NUL), 1),      # norm NULL
    ((A, 0, 4, 100, 7, 0, A, 1, 0, 8, NUL, NUL), 1),      # codes NULL
    ((A, 0, 4, 100, 7, 0, A, 1, 0, 8, U, NUL), 6),        # codes misaligned
    ((A, 0, 4, 100, 7, 0, A, 1, -1, 8, A, NUL), 2),       # worker_base < 0
    ((A, 0, 4, 100, 7, 0, A, 1, (1 << 32) - 2, 8, A, NUL), 2),  # workers past 2^32
])
def test_quantize_rejects(args, expect):
    assert gq.lib().gq_quantize(*args) == expect


def test_other_entry_points_reject():
    L = gq.lib()
    assert L.gq_reduce_codes(NUL, 4, 100, 8, A, NUL) == 1
    assert L.gq_reduce_codes(A, 0, 100, 8, A, NUL) == 2
    assert L.gq_reduce_codes(A, 4, 100, 1, A, NUL) == 4
    assert L.gq_reduce_codes(U, 4, 100, 8, A, NUL) == 6
    assert L.gq_dequantize(A, 4, 100, 7, 0, 5, A, A, NUL) == 4
    assert L.gq_dequantize(A, 4, 100, 7, 0, 8, NUL, A, NUL) == 1
    assert L.gq_dequantize(A, 4, 100, 7, 0, 8, A, U, NUL) == 6
    assert L.gq_compress_mean_from_norm(A, 0, 4, 100, 7, 0, 1, A, 8, U, NUL, NUL) == 6
    assert L.gq_compress_mean_from_norm(A, 0, 4, 100, 7, 0, 1, A, 5, A, A, NUL) == 4
    assert L.gq_compress_mean_from_norm(A, 0, 4, 100, 7, 0, 1, NUL, 8, A, NUL, NUL) == 1
    ws = gq.gq_workspace_bytes(4, 100)
    assert L.gq_compress_mean(A, 0, 4, 100, 7, 2.0, 0.0, 0, 1, 8, A, A, NUL, A, ws, NUL) == 3
    assert L.gq_compress_mean(A, 0, 4, 100, 7, 2.0, 2.0, 0, 1, 8, A, A, NUL, A, ws - 1, NUL) == 5
    assert L.gq_compress_mean(A, 1, 4, 100, 0, 2.0, 2.0, 0, 1, 8, A, A, NUL, A, ws, NUL) == 2
    assert L.gq_qsgd_local_mean(A, 0, 4, 100, 3, 1, A, A, A, 2, A, ws, NUL) == 4
    assert L.gq_qsgd_local_mean(A, 0, 4, 100, 3, 1, NUL, A, NUL, 0, A, ws, NUL) == 1


def test_staged_sums_entry_points_reject():
    L = gq.lib()
    assert L.gq_compress_sums8(NUL, 0, 4, 100, 7, 0, 1, A, A, NUL) == 1
    assert L.gq_compress_sums8(A, 0, 4, 100, 7, 0, 1, NUL, A, NUL) == 1
    assert L.gq_compress_sums8(A, 0, 4, 100, 7, 0, 1, A, U, NUL) == 6
    assert L.gq_compress_sums8(A, 0, 4, 100, 0, 0, 1, A, A, NUL) == 2
    assert L.gq_compress_sums8(A, 2, 4, 100, 7, 0, 1, A, A, NUL) == 2
    assert L.gq_dequantize_sums8(A, 0, 4, 100, 7, 0, 1, A, NUL, A, NUL) == 1
    assert L.gq_dequantize_sums8(A, 0, 4, 100, 7, 0, 1, A, A, U, NUL) == 6
    # the staging buffer: a bit per 8-coordinate group in 64-bit words, then a
    # byte per coordinate, each part 16-byte aligned
    for d in (0, 1, 8, 511, 512, 513, 64_000_000):
        mask = (-(-d // 512) * 8 + 15) // 16 * 16
        assert gq.gq_sums8_bytes(d) == mask + -(-d // 16) * 16
    assert gq.gq_sums8_bytes(-1) == -1


def test_zero_code_skip_sizes_and_rejects():
    """The span bounds: one 16-bit entry per (row, 512 coordinates), rows
    padded to a multiple of 16 entries; the compress workspace is the
    norm's plus the bounds rounded up to 256."""
    L = gq.lib()
    for n, d in ((1, 0), (1, 1), (3, 511), (3, 512), (3, 513), (64, 64_000_000),
                 (8, 355_000_000)):
        assert gq.gq_span_bounds_bytes(n, d) == 2 * n * -(-d // 8192) * 16
        extra = gq.gq_compress_workspace_bytes(n, d) - gq.gq_workspace_bytes(n, d)
        assert extra == -(-gq.gq_span_bounds_bytes(n, d) // 256) * 256
    assert gq.gq_span_bounds_bytes(0, 5) == -1 and gq.gq_span_bounds_bytes(2, -1) == -1
    assert gq.gq_compress_workspace_bytes(0, 5) == -1
    ws = gq.gq_workspace_bytes(4, 100)
    B = ctypes.c_void_p(1 << 20)  # an aligned address (never dereferenced: rejected first)
    # gq_global_norm_bounds(x, dtype, n, d, q, p, norm, bounds, ws, ws_bytes, stream)
    assert L.gq_global_norm_bounds(NUL, 0, 4, 100, 2.0, 2.0, A, B, A, ws, NUL) == 1
    assert L.gq_global_norm_bounds(A, 0, 4, 100, 2.0, 2.0, A, NUL, A, ws, NUL) == 1
    assert L.gq_global_norm_bounds(A, 0, 4, 100, 2.0, 2.0, A, ctypes.c_void_p((1 << 20) + 2), A, ws,
                                   NUL) == 6
    assert L.gq_global_norm_bounds(A, 0, 4, 100, 2.0, 0.5, A, B, A, ws, NUL) == 3
    assert L.gq_global_norm_bounds(A, 0, 4, 100, 2.0, 2.0, A, B, A, ws - 1, NUL) == 5
    # gq_compress_mean_skip(x, dtype, n, d, s, scheme, seed, norm, bounds, W, mean, code_sum, stream)
    assert L.gq_compress_mean_skip(A, 0, 4, 100, 7, 0, 1, A, NUL, 0, A, NUL, NUL) == 1
    assert L.gq_compress_mean_skip(A, 0, 4, 100, 7, 0, 1, A, ctypes.c_void_p((1 << 20) + 8), 0, A,
                                   NUL, NUL) == 6
    assert L.gq_compress_mean_skip(A, 0, 4, 100, 7, 0, 1, A, B, 0, U, NUL, NUL) == 6
    assert L.gq_compress_mean_skip(A, 0, 4, 100, 7, 0, 1, A, B, 5, A, A, NUL) == 4
    assert L.gq_compress_mean_skip(A, 0, 4, 100, 0, 0, 1, A, B, 0, A, NUL, NUL) == 2
    # the sharded form: gq_norm_term_bounds(x, dtype, n, d, q, p, term, bounds, ws, ws_bytes,
    # stream) and gq_compress_words_skip(x, dtype, n, d, s, scheme, norm, bounds, seed,
    # worker_base, W, word_sum, stream)
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L.gq_norm_term_bounds(A, 0, 4, 100, 2.0, 2.0, NUL, B, A, ws, NUL) == 1
    assert L.gq_norm_term_bounds(A, 0, 4, 100, 2.0, 2.0, A, NUL, A, ws, NUL) == 1
    assert L.gq_norm_term_bounds(A, 0, 4, 100, 2.0, 2.0, A, odd, A, ws, NUL) == 6
    assert L.gq_norm_term_bounds(A, 0, 4, 100, 0.5, 2.0, A, B, A, ws, NUL) == 3
    assert L.gq_norm_term_bounds(A, 0, 4, 100, 2.0, 2.0, A, B, A, ws - 1, NUL) == 5
    assert L.gq_compress_words_skip(A, 0, 4, 100, 7, 0, A, NUL, 1, 0, 6, A, NUL) == 1
    assert L.gq_compress_words_skip(A, 0, 4, 100, 7, 0, NUL, B, 1, 0, 6, A, NUL) == 1
    assert L.gq_compress_words_skip(A, 0, 4, 100, 7, 0, A, odd, 1, 0, 6, A, NUL) == 6
    assert L.gq_compress_words_skip(A, 0, 4, 100, 7, 0, A, B, 1, 0, 6, U, NUL) == 6
    assert L.gq_compress_words_skip(A, 0, 4, 100, 7, 0, A, B, 1, 0, 5, A, NUL) == 4
    assert L.gq_compress_words_skip(A, 0, 4, 100, 7, 0, A, B, 1, (1 << 32) - 3, 6, A, NUL) == 2
    assert L.gq_compress_words_skip(A, 0, 4, 100, 7, 5, A, B, 1, 0, 6, A, NUL) == 2


def test_noalloc_entry_point_rejects():
    """The no-allocation entry point checks every argument, and the scratch
    it would need, before any HIP call (so these run without a GPU)."""
    L = gq.lib()
    cap = gq.NOALLOC_SCRATCH_BYTES
    assert L.gq_compress_mean_noalloc(NUL, 0, 4, 100, 7, 2.0, 2.0, 0, 1, 8, A, A, NUL, NUL) == 1
    assert L.gq_compress_mean_noalloc(A, 0, 4, 100, 7, 2.0, 0.0, 0, 1, 8, A, A, NUL, NUL) == 3
    assert L.gq_compress_mean_noalloc(A, 0, 4, 100, 7, 2.0, 2.0, 0, 1, 5, A, A, A, NUL) == 4
    assert L.gq_compress_mean_noalloc(A, 0, 4, 100, 7, 2.0, 2.0, 0, 1, 8, U, A, NUL, NUL) == 6
    assert L.gq_compress_mean_noalloc(A, 0, 4, 100, 7, 2.0, 2.0, 0, 1, 8, A, NUL, NUL, NUL) == 1
    # sizes whose norm-pass scratch exceeds the array: rejected, with the size named
    for n, d in ((1 << 22, 1), (2_500_000, 4096), (4, 40_000_000_000)):
        assert gq.gq_workspace_bytes(n, d) > cap
        assert L.gq_compress_mean_noalloc(A, 0, n, d, 7, 2.0, 2.0, 0, 1, 0, A, A, NUL, NUL) == 5
        assert str(cap) in L.gq_last_error().decode()
    # the largest workload's scratch fits (16 GB of fp32 input), with the
    # span bounds of the zero-code skip too
    assert gq.gq_compress_workspace_bytes(64, 64_000_000) <= cap


def test_binding_fails_loudly_without_a_gpu():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(ValueError):
        gq.gq_global_norm(torch.zeros(2, 8), 2, 2)


def test_word_layout_sizes_match_the_oracle():
    for d in (0, 1, 7, 8, 97, 65536, 25_557_032):
        for W in (2, 3, 5, 6, 8, 9, 11, 13, 16, 17, 32):
            assert gq.gq_word_row_bytes(d, W) == oracle.word_row_bytes(d, W)
    assert gq.gq_word_row_bytes(10, 1) == -1
    assert gq.gq_word_row_bytes(10, 33) == -1
    assert gq.gq_word_row_bytes(-1, 8) == -1


def test_word_layout_entry_points_reject():
    L = gq.lib()
    q = L.gq_quantize_words
    assert q(A, 0, 4, 100, 7, 0, A, 1, 0, 5, A, NUL) == 4      # W below W_min = 6
    assert q(A, 0, 4, 100, 7, 0, A, 1, 0, 33, A, NUL) == 4     # W above 32
    assert q(A, 0, 4, 100, 7, 0, NUL, 1, 0, 8, A, NUL) == 1    # norm NULL
    assert q(A, 0, 4, 100, 7, 0, A, 1, 0, 8, NUL, NUL) == 1    # words NULL
    assert q(A, 0, 4, 100, 7, 0, A, 1, 0, 8, U, NUL) == 6      # words misaligned
    assert q(U, 0, 4, 100, 7, 0, A, 1, 0, 8, A, NUL) == 6      # x misaligned
    assert q(A, 0, 4, 100, 7, 0, A, 1, -1, 8, A, NUL) == 2     # worker_base < 0
    assert q(A, 2, 4, 100, 7, 0, A, 1, 0, 8, A, NUL) == 2      # dtype
    c = L.gq_compress_words_from_norm
    assert c(A, 0, 4, 100, 7, 0, A, 1, 0, 5, A, NUL) == 4      # W below W_min = 6
    assert c(A, 0, 4, 100, 7, 0, NUL, 1, 0, 8, A, NUL) == 1    # norm NULL
    assert c(A, 0, 4, 100, 7, 0, A, 1, 0, 8, NUL, NUL) == 1    # word_sum NULL
    assert c(A, 0, 4, 100, 7, 0, A, 1, 0, 8, U, NUL) == 6      # word_sum misaligned
    assert c(A, 0, 4, 100, 7, 0, A, 1, -1, 8, A, NUL) == 2     # worker_base < 0
    assert L.gq_sum_words(NUL, 4, 100, 8, A, NUL) == 1
    assert L.gq_sum_words(A, 0, 100, 8, A, NUL) == 2
    assert L.gq_sum_words(A, 4, 100, 1, A, NUL) == 4
    assert L.gq_sum_words(A, 4, 100, 8, U, NUL) == 6
    dq = L.gq_dequantize_words
    assert dq(A, 4, 100, 7, 0, 5, A, A, NUL) == 4
    assert dq(A, 4, 100, 7, 0, 8, NUL, A, NUL) == 1
    assert dq(A, 4, 100, 7, 0, 8, A, U, NUL) == 6
    assert dq(A, 4, 100, 7, 3, 8, A, A, NUL) == 2


def test_e8_subtree_rejects():
    L = gq.lib()
    assert L.gq_e8_subtree(A, 4, 100, 1, 2, A, NUL) == 2      # worker_base not a multiple of n
    assert L.gq_e8_subtree(A, 4, 100, 1, -4, A, NUL) == 2     # negative worker_base
    assert L.gq_e8_subtree(A, 3, 100, 1, 0, A, NUL) == 3      # n not a power of two
    assert L.gq_e8_subtree(NUL, 4, 100, 1, 4, A, NUL) == 1
    assert L.gq_e8_subtree(A, 4, 100, 1, 4, U, NUL) == 6


def test_header_serves_a_plain_c_caller(tmp_path):
    """include/gq.h compiles as C99 and C++11, and a C program linked against
    libgq.so gets sizes, status names and argument errors without a GPU."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    src = tmp_path / "caller.c"
    src.write_text(r"""
#include <stdio.h>
#include <string.h>
#include "gq.h"
int main(void)
{
    if (gq_min_code_bits(8, 127, GQ_SCHEME_L) != 11) return 1;
    if (gq_code_row_bytes(25557032, 11) != 35140928) return 2; /* 16 ceil(d 11 / 128) */
    if (gq_word_row_bytes(64, 9) != 96) return 3;
    if (strcmp(gq_status_str(GQ_ERR_ALIGN), "GQ_ERR_ALIGN") != 0) return 4;
    float norm;
    if (gq_global_norm(NULL, GQ_IN_F32, 4, 100, 2.0f, 2.0f, &norm, NULL, 0, NULL) != GQ_ERR_NULL)
        return 5;
    if (gq_last_error()[0] == '\0') return 6;
    puts("ok");
    return 0;
}
""")
    lib_dir = os.path.join(ROOT, "allreduce_compatible_gradient_amd")
    exe = tmp_path / "caller"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-L", lib_dir, "-lgq",
                    f"-Wl,-rpath,{lib_dir}", "-o", str(exe)], check=True, timeout=120)
    subprocess.run(["g++", "-std=c++11", "-Wall", "-Werror", "-fsyntax-only", "-x", "c++",
                    "-I", os.path.join(ROOT, "include"), str(src)], check=True, timeout=120)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)

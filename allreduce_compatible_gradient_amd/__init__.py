"""Python binding of libgq.so -- Global-QSGD compression on AMD MI355X.

Argument marshalling only: every step of the operator runs in the HIP
kernels of ``csrc/gq.hip`` behind the C ABI of ``include/gq.h``.  PyTorch
supplies device memory and the stream.  There is no fallback: without the
built library, or without a GPU, the compute entry points raise.

The functions keep the C names.  Each takes CUDA (HIP) tensors, allocates
the outputs it is not given, launches on ``stream`` (default: torch's
current stream) and returns without synchronizing.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgq.so")

GQ_SCHEME_L = 0
GQ_SCHEME_E = 1
GQ_IN_F32 = 0
GQ_IN_BF16 = 1

STATUS = {0: "GQ_OK", 1: "GQ_ERR_NULL", 2: "GQ_ERR_ARG", 3: "GQ_ERR_UNSUPPORTED",
          4: "GQ_ERR_CODE_WIDTH", 5: "GQ_ERR_WORKSPACE", 6: "GQ_ERR_ALIGN", 7: "GQ_ERR_DEVICE"}

# exported symbols with their C signatures
_i32, _i64, _u64, _f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p
SIGNATURES = {
    "gq_min_code_bits": (_i32, [_i64, _i32, _i32]),
    "gq_code_row_bytes": (_i64, [_i64, _i32]),
    "gq_workspace_bytes": (_i64, [_i64, _i64]),
    "gq_compress_workspace_bytes": (_i64, [_i64, _i64]),
    "gq_global_norm": (_i32, [_vp, _i32, _i64, _i64, _f32, _f32, _vp, _vp, _i64, _vp]),
    "gq_norm_term": (_i32, [_vp, _i32, _i64, _i64, _f32, _f32, _vp, _vp, _i64, _vp]),
    "gq_norm_from_term": (_i32, [_vp, _f32, _f32, _vp, _vp]),
    "gq_quantize": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _vp, _u64, _i64, _i32, _vp, _vp]),
    "gq_reduce_codes": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "gq_dequantize": (_i32, [_vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
    "gq_word_row_bytes": (_i64, [_i64, _i32]),
    "gq_quantize_words": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _vp, _u64, _i64, _i32, _vp,
                                 _vp]),
    "gq_compress_words_from_norm": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _vp, _u64, _i64,
                                           _i32, _vp, _vp]),
    "gq_sum_words": (_i32, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "gq_dequantize_words": (_i32, [_vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
    "gq_compress_mean_from_norm": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _u64, _vp, _i32,
                                          _vp, _vp, _vp]),
    "gq_compress_mean": (_i32, [_vp, _i32, _i64, _i64, _i32, _f32, _f32, _i32, _u64, _i32, _vp,
                                _vp, _vp, _vp, _i64, _vp]),
    "gq_span_bounds_bytes": (_i64, [_i64, _i64]),
    "gq_global_norm_bounds": (_i32, [_vp, _i32, _i64, _i64, _f32, _f32, _vp, _vp, _vp, _i64,
                                     _vp]),
    "gq_compress_mean_skip": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _u64, _vp, _vp, _i32,
                                     _vp, _vp, _vp]),
    "gq_norm_term_bounds": (_i32, [_vp, _i32, _i64, _i64, _f32, _f32, _vp, _vp, _vp, _i64, _vp]),
    "gq_compress_words_skip": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _vp, _vp, _u64, _i64,
                                      _i32, _vp, _vp]),
    "gq_sums8_bytes": (_i64, [_i64]),
    "gq_compress_sums8": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _u64, _vp, _vp, _vp]),
    "gq_dequantize_sums8": (_i32, [_vp, _i32, _i64, _i64, _i32, _i32, _u64, _vp, _vp, _vp, _vp]),
    "gq_compress_mean_noalloc": (_i32, [_vp, _i32, _i64, _i64, _i32, _f32, _f32, _i32, _u64,
                                        _i32, _vp, _vp, _vp, _vp]),
    "gq_qsgd_local_mean": (_i32, [_vp, _i32, _i64, _i64, _i32, _u64, _vp, _vp, _vp, _i32, _vp,
                                  _i64, _vp]),
    "gq_e8_row_bytes": (_i64, [_i64]),
    "gq_e8_quantize": (_i32, [_vp, _i32, _i64, _i64, _vp, _u64, _i64, _vp, _vp]),
    "gq_e8_reduce_pair": (_i32, [_vp, _vp, _i64, _u64, _i32, _i64, _vp, _vp]),
    "gq_e8_tree": (_i32, [_vp, _i64, _i64, _u64, _vp, _vp]),
    "gq_e8_subtree": (_i32, [_vp, _i64, _i64, _u64, _i64, _vp, _vp]),
    "gq_e8_dequantize": (_i32, [_vp, _i64, _vp, _vp, _vp]),
    "gq_e8_compress_mean": (_i32, [_vp, _i32, _i64, _i64, _f32, _f32, _u64, _vp, _vp, _vp, _vp,
                                   _i64, _vp]),
    "gq_status_str": (ctypes.c_char_p, [_i32]),
    "gq_last_error": (ctypes.c_char_p, []),
}


class GQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise GQError(status, lib().gq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _input(x: torch.Tensor):
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [n, d] tensor")
    if x.dtype == torch.float32:
        return GQ_IN_F32
    if x.dtype == torch.bfloat16:
        return GQ_IN_BF16
    raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")


def _scheme(scheme) -> int:
    if scheme in ("L", GQ_SCHEME_L):
        return GQ_SCHEME_L
    if scheme in ("E", GQ_SCHEME_E):
        return GQ_SCHEME_E
    raise ValueError(f"unknown scheme {scheme!r}")


def _order(v) -> float:
    return math.inf if (isinstance(v, str) and v == "inf") else float(v)


# ---------------------------------------------------------------------------
# sizes

def gq_min_code_bits(n: int, s: int, scheme) -> int:
    return int(lib().gq_min_code_bits(n, s, _scheme(scheme)))


def gq_code_row_bytes(d: int, code_bits: int) -> int:
    return int(lib().gq_code_row_bytes(d, code_bits))


def gq_workspace_bytes(n: int, d: int) -> int:
    return int(lib().gq_workspace_bytes(n, d))


def gq_compress_workspace_bytes(n: int, d: int) -> int:
    """Workspace with which gq_compress_mean runs fastest (>= gq_workspace_bytes)."""
    return int(lib().gq_compress_workspace_bytes(n, d))


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _buf(t, nbytes: int, name: str, device, dtype=None):
    """A caller-given device buffer: on the input's device, contiguous, of the
    given dtype (raw byte buffers: any), and at least nbytes long.  The C ABI
    takes plain pointers and cannot check sizes, so the binding does."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, the input on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, {nbytes} are needed")
    return t


def _norm_in(norm, device):
    if norm is None:
        raise ValueError("norm is required (a 1-element float32 device tensor)")
    return _buf(norm, 4, "norm", device, torch.float32)


def _workspace(ws, n, d, device, alloc=None):
    """The caller's workspace (at least gq_workspace_bytes), or a new one of
    `alloc` bytes (default: gq_workspace_bytes)."""
    need = gq_workspace_bytes(n, d)
    if ws is None:
        ws = torch.empty(max(need if alloc is None else alloc, 16), dtype=torch.uint8,
                         device=device)
    return _buf(ws, need, "workspace", device)


# ---------------------------------------------------------------------------
# the path

def gq_global_norm(x: torch.Tensor, q=2.0, p=2.0, *, norm=None, workspace=None, stream=None):
    """Global (q,p)-norm of the rows of x; returns a 1-element float32 device tensor."""
    dt = _input(x)
    n, d = x.shape
    norm = (torch.empty(1, dtype=torch.float32, device=x.device) if norm is None
            else _buf(norm, 4, "norm", x.device, torch.float32))
    ws = _workspace(workspace, n, d, x.device)
    _check(lib().gq_global_norm(_ptr(x), dt, n, d, _order(q), _order(p), _ptr(norm), _ptr(ws),
                                _nbytes(ws), _stream(stream)))
    return norm


def gq_norm_term(x: torch.Tensor, q=2.0, p=2.0, *, term=None, workspace=None, stream=None):
    """fp64 term of the (q,p)-norm over the rows of x (a shard of the workers);
    returns a 1-element float64 device tensor.  Terms of disjoint shards combine
    by sum (finite p) or max (p = inf)."""
    dt = _input(x)
    n, d = x.shape
    term = (torch.empty(1, dtype=torch.float64, device=x.device) if term is None
            else _buf(term, 8, "term", x.device, torch.float64))
    ws = _workspace(workspace, n, d, x.device)
    _check(lib().gq_norm_term(_ptr(x), dt, n, d, _order(q), _order(p), _ptr(term), _ptr(ws),
                              _nbytes(ws), _stream(stream)))
    return term


def gq_norm_from_term(term: torch.Tensor, q=2.0, p=2.0, *, norm=None, stream=None):
    """The norm N from a term combined over shards; 1-element float32 device tensor."""
    if term.dtype != torch.float64 or term.numel() < 1 or not term.is_cuda:
        raise ValueError("term must be a float64 device tensor")
    norm = (torch.empty(1, dtype=torch.float32, device=term.device) if norm is None
            else _buf(norm, 4, "norm", term.device, torch.float32))
    _check(lib().gq_norm_from_term(_ptr(term), _order(q), _order(p), _ptr(norm), _stream(stream)))
    return norm


def gq_quantize(x: torch.Tensor, s: int, scheme, norm: torch.Tensor, seed: int, code_bits: int, *,
                worker_base: int = 0, codes=None, stream=None):
    """Packed W-bit codes, uint8 [n, gq_code_row_bytes(d, W)]."""
    dt = _input(x)
    n, d = x.shape
    rb = gq_code_row_bytes(d, code_bits)
    _norm_in(norm, x.device)
    if codes is None:
        codes = torch.empty((n, max(rb, 0)), dtype=torch.uint8, device=x.device)
    _buf(codes, n * max(rb, 0), "codes", x.device)
    _check(lib().gq_quantize(_ptr(x), dt, n, d, s, _scheme(scheme), _ptr(norm), seed, worker_base,
                             code_bits, _ptr(codes), _stream(stream)))
    return codes


def gq_reduce_codes(codes: torch.Tensor, n: int, d: int, code_bits: int, *, code_sum=None,
                    stream=None):
    """Exact sum over the n packed rows; one packed row, uint8 [row_bytes]."""
    rb = max(gq_code_row_bytes(d, code_bits), 0)
    _buf(codes, n * rb, "codes", None)
    if code_sum is None:
        code_sum = torch.empty(rb, dtype=torch.uint8, device=codes.device)
    _buf(code_sum, rb, "code_sum", codes.device)
    _check(lib().gq_reduce_codes(_ptr(codes), n, d, code_bits, _ptr(code_sum), _stream(stream)))
    return code_sum


def gq_dequantize(code_sum: torch.Tensor, n: int, d: int, s: int, scheme, code_bits: int,
                  norm: torch.Tensor, *, mean=None, stream=None):
    """Mean over the n workers from the packed code sums, float32 [d]."""
    _buf(code_sum, max(gq_code_row_bytes(d, code_bits), 0), "code_sum", None)
    _norm_in(norm, code_sum.device)
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=code_sum.device)
    _buf(mean, 4 * d, "mean", code_sum.device, torch.float32)
    _check(lib().gq_dequantize(_ptr(code_sum), n, d, s, _scheme(scheme), code_bits, _ptr(norm),
                               _ptr(mean), _stream(stream)))
    return mean


def gq_word_row_bytes(d: int, code_bits: int) -> int:
    return int(lib().gq_word_row_bytes(d, code_bits))


def gq_quantize_words(x: torch.Tensor, s: int, scheme, norm: torch.Tensor, seed: int,
                      code_bits: int, *, worker_base: int = 0, words=None, stream=None):
    """Codes in the word layout (floor(32/W) fields of code + M per word):
    the uint32 words held in an int32 tensor [n, gq_word_row_bytes(d, W) / 4]."""
    dt = _input(x)
    n, d = x.shape
    rb = max(gq_word_row_bytes(d, code_bits), 0)
    _norm_in(norm, x.device)
    if words is None:
        words = torch.empty((n, rb // 4), dtype=torch.int32, device=x.device)
    _buf(words, n * rb, "words", x.device)
    _check(lib().gq_quantize_words(_ptr(x), dt, n, d, s, _scheme(scheme), _ptr(norm), seed,
                                   worker_base, code_bits, _ptr(words), _stream(stream)))
    return words


def gq_compress_words_from_norm(x: torch.Tensor, s: int, scheme, norm: torch.Tensor, seed: int,
                                code_bits: int, *, worker_base: int = 0, word_sum=None,
                                stream=None):
    """The n rows' codes summed into one word row (fields of sum_i (code + M)),
    in an int32 tensor of the uint32 bits [gq_word_row_bytes(d, W) / 4]."""
    dt = _input(x)
    n, d = x.shape
    rb = max(gq_word_row_bytes(d, code_bits), 0)
    _norm_in(norm, x.device)
    if word_sum is None:
        word_sum = torch.empty(rb // 4, dtype=torch.int32, device=x.device)
    _buf(word_sum, rb, "word_sum", x.device)
    _check(lib().gq_compress_words_from_norm(_ptr(x), dt, n, d, s, _scheme(scheme), _ptr(norm),
                                             seed, worker_base, code_bits, _ptr(word_sum),
                                             _stream(stream)))
    return word_sum


def gq_sum_words(words: torch.Tensor, n: int, d: int, code_bits: int, *, word_sum=None,
                 stream=None):
    """Word-wise uint32 sum of the n rows (what a native SUM all-reduce computes),
    in an int32 tensor of the same bits."""
    rb = max(gq_word_row_bytes(d, code_bits), 0)
    _buf(words, n * rb, "words", None)
    if word_sum is None:
        word_sum = torch.empty(rb // 4, dtype=torch.int32, device=words.device)
    _buf(word_sum, rb, "word_sum", words.device)
    _check(lib().gq_sum_words(_ptr(words), n, d, code_bits, _ptr(word_sum), _stream(stream)))
    return word_sum


def gq_dequantize_words(word_sum: torch.Tensor, n: int, d: int, s: int, scheme, code_bits: int,
                        norm: torch.Tensor, *, mean=None, stream=None):
    """Mean over the n workers from a summed row in the word layout, float32 [d]."""
    _buf(word_sum, max(gq_word_row_bytes(d, code_bits), 0), "word_sum", None)
    _norm_in(norm, word_sum.device)
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=word_sum.device)
    _buf(mean, 4 * d, "mean", word_sum.device, torch.float32)
    _check(lib().gq_dequantize_words(_ptr(word_sum), n, d, s, _scheme(scheme), code_bits,
                                     _ptr(norm), _ptr(mean), _stream(stream)))
    return mean


def gq_compress_mean_from_norm(x: torch.Tensor, s: int, scheme, seed: int, norm: torch.Tensor, *,
                               code_bits: int = 0, want_code_sum: bool = False, mean=None,
                               code_sum=None, stream=None):
    """Fused quantize + integer sum + dequantize given the norm: (mean, code_sum or None)."""
    dt = _input(x)
    n, d = x.shape
    _norm_in(norm, x.device)
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=x.device)
    _buf(mean, 4 * d, "mean", x.device, torch.float32)
    if want_code_sum and code_sum is None:
        code_sum = torch.empty(max(gq_code_row_bytes(d, code_bits), 0), dtype=torch.uint8,
                               device=x.device)
    _buf(code_sum, max(gq_code_row_bytes(d, code_bits), 0), "code_sum", x.device)
    _check(lib().gq_compress_mean_from_norm(_ptr(x), dt, n, d, s, _scheme(scheme), seed,
                                            _ptr(norm), code_bits, _ptr(mean), _ptr(code_sum),
                                            _stream(stream)))
    return mean, code_sum


def gq_span_bounds_bytes(n: int, d: int) -> int:
    """Bytes of the span bounds of the zero-code skip: 2 n stride, with
    stride = 16 ceil(d / 8192) entries per row (one per 512 coordinates,
    padded)."""
    return int(lib().gq_span_bounds_bytes(n, d))


def gq_global_norm_bounds(x: torch.Tensor, q=2.0, p=2.0, *, norm=None, bounds=None,
                          workspace=None, stream=None):
    """The global norm and, in the same pass, the span bounds of the
    zero-code skip: (norm, bounds), bounds a uint8 device tensor of
    gq_span_bounds_bytes(n, d) bytes holding the 16-bit bounds."""
    dt = _input(x)
    n, d = x.shape
    norm = (torch.empty(1, dtype=torch.float32, device=x.device) if norm is None
            else _buf(norm, 4, "norm", x.device, torch.float32))
    nb = max(gq_span_bounds_bytes(n, d), 0)
    if bounds is None:
        bounds = torch.empty(max(nb, 2), dtype=torch.uint8, device=x.device)
    _buf(bounds, nb, "bounds", x.device)
    ws = _workspace(workspace, n, d, x.device)
    _check(lib().gq_global_norm_bounds(_ptr(x), dt, n, d, _order(q), _order(p), _ptr(norm),
                                       _ptr(bounds), _ptr(ws), _nbytes(ws), _stream(stream)))
    return norm, bounds


def gq_compress_mean_skip(x: torch.Tensor, s: int, scheme, seed: int, norm: torch.Tensor,
                          bounds: torch.Tensor, *, code_bits: int = 0,
                          want_code_sum: bool = False, mean=None, code_sum=None, stream=None):
    """gq_compress_mean_from_norm with the zero-code skip, given the bounds
    gq_global_norm_bounds wrote for this x: (mean, code_sum or None)."""
    dt = _input(x)
    n, d = x.shape
    _norm_in(norm, x.device)
    _buf(bounds, max(gq_span_bounds_bytes(n, d), 0), "bounds", x.device)
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=x.device)
    _buf(mean, 4 * d, "mean", x.device, torch.float32)
    if want_code_sum and code_sum is None:
        code_sum = torch.empty(max(gq_code_row_bytes(d, code_bits), 0), dtype=torch.uint8,
                               device=x.device)
    _buf(code_sum, max(gq_code_row_bytes(d, code_bits), 0), "code_sum", x.device)
    _check(lib().gq_compress_mean_skip(_ptr(x), dt, n, d, s, _scheme(scheme), seed, _ptr(norm),
                                       _ptr(bounds), code_bits, _ptr(mean), _ptr(code_sum),
                                       _stream(stream)))
    return mean, code_sum


def gq_norm_term_bounds(x: torch.Tensor, q=2.0, p=2.0, *, term=None, bounds=None,
                        workspace=None, stream=None):
    """gq_norm_term and, in the same pass, the span bounds of this shard's
    rows: (term, bounds), as gq_global_norm_bounds lays them out."""
    dt = _input(x)
    n, d = x.shape
    term = (torch.empty(1, dtype=torch.float64, device=x.device) if term is None
            else _buf(term, 8, "term", x.device, torch.float64))
    nb = max(gq_span_bounds_bytes(n, d), 0)
    if bounds is None:
        bounds = torch.empty(max(nb, 2), dtype=torch.uint8, device=x.device)
    _buf(bounds, nb, "bounds", x.device)
    ws = _workspace(workspace, n, d, x.device)
    _check(lib().gq_norm_term_bounds(_ptr(x), dt, n, d, _order(q), _order(p), _ptr(term),
                                     _ptr(bounds), _ptr(ws), _nbytes(ws), _stream(stream)))
    return term, bounds


def gq_compress_words_skip(x: torch.Tensor, s: int, scheme, norm: torch.Tensor,
                           bounds: torch.Tensor, seed: int, code_bits: int, *,
                           worker_base: int = 0, word_sum=None, stream=None):
    """gq_compress_words_from_norm with the zero-code skip, given the bounds
    gq_norm_term_bounds wrote for this x: the same word row."""
    dt = _input(x)
    n, d = x.shape
    rb = max(gq_word_row_bytes(d, code_bits), 0)
    _norm_in(norm, x.device)
    _buf(bounds, max(gq_span_bounds_bytes(n, d), 0), "bounds", x.device)
    if word_sum is None:
        word_sum = torch.empty(rb // 4, dtype=torch.int32, device=x.device)
    _buf(word_sum, rb, "word_sum", x.device)
    _check(lib().gq_compress_words_skip(_ptr(x), dt, n, d, s, _scheme(scheme), _ptr(norm),
                                        _ptr(bounds), seed, worker_base, code_bits,
                                        _ptr(word_sum), _stream(stream)))
    return word_sum


def gq_compress_mean(x: torch.Tensor, s: int, q, p, scheme, seed: int, *, code_bits: int = 0,
                     want_code_sum: bool = False, mean=None, norm=None, code_sum=None,
                     workspace=None, stream=None):
    """The whole path: (mean float32 [d], norm float32 [1], code_sum or None)."""
    dt = _input(x)
    n, d = x.shape
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=x.device)
    if norm is None:
        norm = torch.empty(1, dtype=torch.float32, device=x.device)
    if want_code_sum and code_sum is None:
        code_sum = torch.empty(max(gq_code_row_bytes(d, code_bits), 0), dtype=torch.uint8,
                               device=x.device)
    _buf(mean, 4 * d, "mean", x.device, torch.float32)
    _buf(norm, 4, "norm", x.device, torch.float32)
    _buf(code_sum, max(gq_code_row_bytes(d, code_bits), 0), "code_sum", x.device)
    ws = _workspace(workspace, n, d, x.device, alloc=gq_compress_workspace_bytes(n, d))
    _check(lib().gq_compress_mean(_ptr(x), dt, n, d, s, _order(q), _order(p), _scheme(scheme), seed,
                                  code_bits, _ptr(mean), _ptr(norm), _ptr(code_sum), _ptr(ws),
                                  _nbytes(ws), _stream(stream)))
    return mean, norm, code_sum


def gq_sums8_bytes(d: int) -> int:
    """Bytes of the staging buffer of gq_compress_sums8 / gq_dequantize_sums8."""
    return int(lib().gq_sums8_bytes(d))


def sums8_parts(staged: torch.Tensor, d: int):
    """Views of a staging buffer: (the group mask as int64 words, the d sum bytes as int8)."""
    mb = (((d + 511) // 512) * 8 + 15) // 16 * 16
    u8 = staged.view(torch.uint8)
    return u8[:mb].view(torch.int64)[: (d + 511) // 512], u8[mb:mb + d].view(torch.int8)


def gq_compress_sums8(x: torch.Tensor, s: int, scheme, seed: int, norm: torch.Tensor, *,
                      sums8=None, stream=None):
    """Staged exact code sums: a bit per 8-coordinate group (1: not all zero),
    then a byte per coordinate of the marked groups (-128: beyond one byte);
    uint8 [gq_sums8_bytes(d)] (see sums8_parts)."""
    dt = _input(x)
    n, d = x.shape
    _norm_in(norm, x.device)
    if sums8 is None:
        sums8 = torch.empty(max(gq_sums8_bytes(d), 16), dtype=torch.uint8, device=x.device)
    _buf(sums8, gq_sums8_bytes(d), "sums8", x.device)
    _check(lib().gq_compress_sums8(_ptr(x), dt, n, d, s, _scheme(scheme), seed, _ptr(norm),
                                   _ptr(sums8), _stream(stream)))
    return sums8


def gq_dequantize_sums8(x: torch.Tensor, s: int, scheme, seed: int, norm: torch.Tensor,
                        sums8: torch.Tensor, *, mean=None, stream=None):
    """The mean from gq_compress_sums8's bytes (escaped groups recomputed from x)."""
    dt = _input(x)
    n, d = x.shape
    _norm_in(norm, x.device)
    _buf(sums8, gq_sums8_bytes(d), "sums8", x.device)
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=x.device)
    _buf(mean, 4 * d, "mean", x.device, torch.float32)
    _check(lib().gq_dequantize_sums8(_ptr(x), dt, n, d, s, _scheme(scheme), seed, _ptr(norm),
                                     _ptr(sums8), _ptr(mean), _stream(stream)))
    return mean


# bytes of the device array behind gq_compress_mean_noalloc (GQ_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def gq_compress_mean_noalloc(x: torch.Tensor, s: int, q, p, scheme, seed: int, *, mean,
                             norm, code_bits: int = 0, code_sum=None, stream=None):
    """gq_compress_mean with the library's own scratch instead of a workspace:
    the caller passes every output (nothing is allocated on this path).
    Returns (mean, norm, code_sum)."""
    dt = _input(x)
    n, d = x.shape
    _buf(mean, 4 * d, "mean", x.device, torch.float32)
    _buf(norm, 4, "norm", x.device, torch.float32)
    _buf(code_sum, max(gq_code_row_bytes(d, code_bits), 0), "code_sum", x.device)
    _check(lib().gq_compress_mean_noalloc(_ptr(x), dt, n, d, s, _order(q), _order(p),
                                          _scheme(scheme), seed, code_bits, _ptr(mean),
                                          _ptr(norm), _ptr(code_sum), _stream(stream)))
    return mean, norm, code_sum


def gq_qsgd_local_mean(x: torch.Tensor, s: int, seed: int, *, code_bits: int = 0,
                       want_codes: bool = False, mean=None, norms=None, codes=None,
                       workspace=None, stream=None):
    """Local-norm QSGD ablation: (mean float32 [d], norms float32 [n], codes or None)."""
    dt = _input(x)
    n, d = x.shape
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=x.device)
    if norms is None:
        norms = torch.empty(n, dtype=torch.float32, device=x.device)
    if want_codes and codes is None:
        codes = torch.empty((n, max(gq_code_row_bytes(d, code_bits), 0)), dtype=torch.uint8,
                            device=x.device)
    _buf(mean, 4 * d, "mean", x.device, torch.float32)
    _buf(norms, 4 * n, "norms", x.device, torch.float32)
    _buf(codes, n * max(gq_code_row_bytes(d, code_bits), 0), "codes", x.device)
    ws = _workspace(workspace, n, d, x.device, alloc=gq_compress_workspace_bytes(n, d))
    _check(lib().gq_qsgd_local_mean(_ptr(x), dt, n, d, s, seed, _ptr(mean), _ptr(norms),
                                    _ptr(codes), code_bits, _ptr(ws), _nbytes(ws),
                                    _stream(stream)))
    return mean, norms, codes


# ---------------------------------------------------------------------------
# the pages' 8-bit exponential-dithering format and its re-rounding tree

def gq_e8_row_bytes(d: int) -> int:
    return int(lib().gq_e8_row_bytes(d))


def gq_e8_quantize(x: torch.Tensor, norm: torch.Tensor, seed: int, *, worker_base: int = 0,
                   codes=None, stream=None):
    """8-bit codes, uint8 [n, gq_e8_row_bytes(d)]."""
    dt = _input(x)
    n, d = x.shape
    _norm_in(norm, x.device)
    if codes is None:
        codes = torch.empty((n, gq_e8_row_bytes(d)), dtype=torch.uint8, device=x.device)
    _buf(codes, n * gq_e8_row_bytes(d), "codes", x.device)
    _check(lib().gq_e8_quantize(_ptr(x), dt, n, d, _ptr(norm), seed, worker_base, _ptr(codes),
                                _stream(stream)))
    return codes


def gq_e8_reduce_pair(a: torch.Tensor, b: torch.Tensor, d: int, seed: int, level: int, node: int,
                      *, out=None, stream=None):
    rb = max(gq_e8_row_bytes(d), 0)
    _buf(a, rb, "a", None)
    _buf(b, rb, "b", a.device)
    if out is None:
        out = torch.empty(rb, dtype=torch.uint8, device=a.device)
    _buf(out, rb, "out", a.device)
    _check(lib().gq_e8_reduce_pair(_ptr(a), _ptr(b), d, seed, level, node, _ptr(out),
                                   _stream(stream)))
    return out


def gq_e8_tree(codes: torch.Tensor, n: int, d: int, seed: int, *, root=None, stream=None):
    rb = max(gq_e8_row_bytes(d), 0)
    _buf(codes, n * rb, "codes", None)
    if root is None:
        root = torch.empty(rb, dtype=torch.uint8, device=codes.device)
    _buf(root, rb, "root", codes.device)
    _check(lib().gq_e8_tree(_ptr(codes), n, d, seed, _ptr(root), _stream(stream)))
    return root


def gq_e8_subtree(codes: torch.Tensor, n: int, d: int, seed: int, worker_base: int, *, root=None,
                  stream=None):
    """Root of the subtree over workers worker_base .. worker_base + n - 1, with
    the whole tree's node indices (worker_base a multiple of n)."""
    rb = max(gq_e8_row_bytes(d), 0)
    _buf(codes, n * rb, "codes", None)
    if root is None:
        root = torch.empty(rb, dtype=torch.uint8, device=codes.device)
    _buf(root, rb, "root", codes.device)
    _check(lib().gq_e8_subtree(_ptr(codes), n, d, seed, worker_base, _ptr(root), _stream(stream)))
    return root


def gq_e8_dequantize(root: torch.Tensor, d: int, norm: torch.Tensor, *, mean=None, stream=None):
    _buf(root, max(gq_e8_row_bytes(d), 0), "root", None)
    _norm_in(norm, root.device)
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=root.device)
    _buf(mean, 4 * d, "mean", root.device, torch.float32)
    _check(lib().gq_e8_dequantize(_ptr(root), d, _ptr(norm), _ptr(mean), _stream(stream)))
    return mean


def gq_e8_compress_mean(x: torch.Tensor, q, p, seed: int, *, want_root: bool = False, mean=None,
                        norm=None, root=None, workspace=None, stream=None):
    """Norm + 8-bit codes + re-rounding tree + dequantization: (mean, norm, root or None)."""
    dt = _input(x)
    n, d = x.shape
    if mean is None:
        mean = torch.empty(d, dtype=torch.float32, device=x.device)
    if norm is None:
        norm = torch.empty(1, dtype=torch.float32, device=x.device)
    if want_root and root is None:
        root = torch.empty(gq_e8_row_bytes(d), dtype=torch.uint8, device=x.device)
    _buf(mean, 4 * d, "mean", x.device, torch.float32)
    _buf(norm, 4, "norm", x.device, torch.float32)
    _buf(root, max(gq_e8_row_bytes(d), 0), "root", x.device)
    ws = _workspace(workspace, n, d, x.device)
    _check(lib().gq_e8_compress_mean(_ptr(x), dt, n, d, _order(q), _order(p), seed, _ptr(mean),
                                     _ptr(norm), _ptr(root), _ptr(ws), _nbytes(ws),
                                     _stream(stream)))
    return mean, norm, root

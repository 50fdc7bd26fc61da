"""Binding of libgq_probe.so: the measurement kernels behind the rooflines.

``read_ceiling`` times a plain stream read of a device buffer in several
launch shapes and returns the best rate: the HBM read ceiling the library's
bandwidth-bound passes are compared with.  ``valu_rates`` times long loops
of independent vector-ALU instructions of one kind and returns their issue
rate in wave64 instructions per second (and per CU per clock at the nominal
2.4 GHz).  Timing uses HIP events on the stream the kernels run on.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_PKG, "libgq_probe.so")
CUS = 256
NOMINAL_GHZ = 2.4
READ_SHAPES = {0: "512 threads x 2 loads (16 KB/block)", 1: "256 x 2 (8 KB)",
               2: "512 x 4 (32 KB)", 3: "256 x 8 (32 KB)", 4: "1024 x 1 (16 KB)"}
VALU_OPS = {0: "v_fma_f32", 1: "v_add_u32", 2: "v_bitop3_b32", 3: "v_mad_u64_u32",
            4: "v_add_f64", 5: "v_fma_f64"}

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.gqp_read_blocks.argtypes = [i64, i32]
        L.gqp_read_blocks.restype = i32
        L.gqp_read_out_words.argtypes = [i64, i32]
        L.gqp_read_out_words.restype = i32
        L.gqp_read.argtypes = [vp, i64, i32, vp, vp]
        L.gqp_read.restype = i32
        L.gqp_valu.argtypes = [i32, i32, i32, ctypes.c_uint32, vp, vp]
        L.gqp_valu.restype = i32
        _lib = L
    return _lib


def _time_ms(fn, stream, reps: int) -> float:
    for _ in range(2):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def read_ceiling(buf: torch.Tensor, reps: int = 10, stream=None) -> dict:
    """Best stream-read rate over the launch shapes, reading all of buf once
    per launch (buf: a contiguous device tensor, 16-byte aligned)."""
    stream = stream or torch.cuda.current_stream()
    nbytes = buf.numel() * buf.element_size()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = torch.empty(max(lib().gqp_read_out_words(nbytes, s) for s in READ_SHAPES),
                      dtype=torch.int32, device=buf.device)
    rates = {}
    for shape in READ_SHAPES:
        def run(shape=shape):
            rc = lib().gqp_read(ctypes.c_void_p(buf.data_ptr()), nbytes, shape,
                                ctypes.c_void_p(out.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"gqp_read failed ({rc})")
        rates[shape] = nbytes / (_time_ms(run, stream, reps) * 1e-3) / 1e9
    best = max(rates, key=rates.get)
    return {"GBs": round(rates[best], 1), "frac_of_8TBs": round(rates[best] / 8000.0, 4),
            "bytes": nbytes, "shape": READ_SHAPES[best],
            "all_GBs": {READ_SHAPES[k]: round(v, 1) for k, v in rates.items()}}


def valu_rates(blocks: int = 4096, iters: int = 4096, reps: int = 5, stream=None) -> dict:
    """Issue rate of each instruction kind: wave64 instructions per second over
    blocks x 4 waves x iters x 8, and per CU per clock at the nominal clock."""
    stream = stream or torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    res = {}
    for op, name in VALU_OPS.items():
        def run(op=op):
            rc = lib().gqp_valu(op, blocks, iters, 1, ctypes.c_void_p(out.data_ptr()), sp)
            if rc != 0:
                raise RuntimeError(f"gqp_valu failed ({rc})")
        ms = _time_ms(run, stream, reps)
        winst = blocks * 4.0 * iters * 8.0
        rate = winst / (ms * 1e-3)
        res[name] = {"ms": round(ms, 4), "G_wave_inst_s": round(rate / 1e9, 1),
                     "per_cu_per_clock": round(rate / (CUS * NOMINAL_GHZ * 1e9), 3)}
    return res

"""Seeded synthetic gradient shards for the Global-QSGD workloads.

This module only draws inputs.  It holds none of the operator's arithmetic,
and both the HIP library's tests/benchmark and the CPU oracle take their
inputs from it.  Every row (one simulated worker) comes from its own numpy
PCG64 streams, keyed by (data seed, worker, component), so any prefix of a
row can be regenerated alone and rows can be drawn in parallel threads.

The five workloads stand in for gradient buckets of models of the stated
sizes; only the parameter counts are taken from those models, the values
are synthetic draws with the stated distributions.  Quantizer settings
follow "Global-QSGD: Practical Floatless Quantization for Distributed
Learning with Theoretical Guarantees": standard dithering (Global-L_s) and
exponential dithering (Global-E_s) of Sec. 3, (q,p)-norms of Sec. 2.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

INF = math.inf


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    scheme: str          # "L" (standard dithering) or "E" (exponential dithering)
    q: float
    p: float
    s: int
    n: int               # simulated workers (rows)
    d: int               # coordinates per worker
    dtype: str           # "f32" or "bf16"
    code_bits: int       # width of the integer codes / code sums
    seed: int            # data seed == quantizer seed
    values: str

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def input_bytes(self) -> int:
        return self.n * self.d * self.elem_bytes


WORKLOADS = {
    1: Workload(1, "small_L_s7_q2p2_n4_d65536_f32", "L", 2.0, 2.0, 7, 4, 65_536, "f32", 8, 0,
                "worker i ~ N(0, (0.5 + 0.25 i)^2)"),
    2: Workload(2, "resnet50_grad_L_s127_q2pinf_n8_d25557032_f32", "L", 2.0, INF, 127, 8,
                25_557_032, "f32", 16, 1,
                "161 layer blocks of log-uniform size, block b ~ N(0, sigma_b^2), "
                "sigma_b log-uniform in [1e-4, 1e-1]"),
    3: Workload(3, "bert_base_grad_E_s8_q2p2_n16_d110000000_f32", "E", 2.0, 2.0, 8, 16,
                110_000_000, "f32", 32, 2,
                "Laplace(0, 1e-3), 0.1% of entries scaled by 100"),
    4: Workload(4, "gpt2_medium_grad_L_s15_q2p2_n8_d355000000_bf16", "L", 2.0, 2.0, 15, 8,
                355_000_000, "bf16", 8, 3,
                "per-worker scale c_i ~ U[0.5, 2] times N(0, 1e-2), rounded to bf16"),
    5: Workload(5, "t3_ablation_L_s3_q2p2_n64_d64000000_f32", "L", 2.0, 2.0, 3, 64,
                64_000_000, "f32", 9, 4,
                "1e-3 * Student-t(3); local-norm QSGD (s=3) timed beside it"),
}

# component ids of the per-row streams
_C_MAIN, _C_AUX, _C_MASK, _C_SCALE = 0, 1, 2, 3
_LAYOUT_ROW = 1_000_000  # stream id of the shared layer layout (workload 2)


def _rng(seed: int, row: int, comp: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, row, comp])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def layer_layout(seed: int, d: int, blocks: int = 161):
    """Block sizes (summing to d) and per-block std for the ResNet-50-sized workload.

    Sizes are drawn log-uniform in [2^6, 2^21], scaled to sum to d (the last
    block takes the rounding remainder); stds are log-uniform in [1e-4, 1e-1]."""
    rng = _rng(seed, _LAYOUT_ROW, _C_MAIN)
    raw = np.exp2(rng.uniform(6.0, 21.0, size=blocks))
    sizes = np.maximum(1, np.floor(raw * (d / raw.sum()))).astype(np.int64)
    sizes[-1] += d - sizes.sum()
    if sizes[-1] < 1:
        raise ValueError("layout does not fit d")
    stds = np.exp(rng.uniform(math.log(1e-4), math.log(1e-1), size=blocks)).astype(np.float32)
    return sizes, stds


def _row(w: Workload, i: int, dd: int, layout) -> np.ndarray:
    seed = w.seed
    if w.key == 1:
        z = _rng(seed, i, _C_MAIN).standard_normal(dd, dtype=np.float32)
        return z * np.float32(0.5 + 0.25 * i)
    if w.key == 2:
        sizes, stds = layout
        z = _rng(seed, i, _C_MAIN).standard_normal(dd, dtype=np.float32)
        std = np.repeat(stds, sizes)[:dd]
        return z * std
    if w.key == 3:
        e = _rng(seed, i, _C_MAIN).standard_exponential(dd, dtype=np.float32)
        bits = np.frombuffer(_rng(seed, i, _C_AUX).bytes((dd + 7) // 8), dtype=np.uint8)
        sign = np.unpackbits(bits, bitorder="little")[:dd]
        x = e * np.float32(1e-3)
        np.negative(x, out=x, where=sign.astype(bool))
        # Bernoulli(0.001) outliers as a Bernoulli process: geometric gaps
        g = _rng(seed, i, _C_MASK)
        pos, start = [], -1
        while True:
            gaps = g.geometric(0.001, size=max(1024, int(dd * 0.0012)))
            p = start + np.cumsum(gaps)
            pos.append(p[p < dd])
            if p[-1] >= dd:
                break
            start = int(p[-1])
        idx = np.concatenate(pos)
        x[idx] *= np.float32(100.0)
        return x
    if w.key == 4:
        c = np.float32(_rng(seed, i, _C_SCALE).uniform(0.5, 2.0))
        z = _rng(seed, i, _C_MAIN).standard_normal(dd, dtype=np.float32)
        return f32_to_bf16_bits(c * (np.float32(0.1) * z))
    if w.key == 5:
        z = _rng(seed, i, _C_MAIN).standard_normal(dd, dtype=np.float32)
        g = _rng(seed, i, _C_AUX).standard_gamma(1.5, dd, dtype=np.float32)
        chi2_over_nu = np.maximum(g, np.float32(1e-30)) * np.float32(2.0 / 3.0)
        return np.float32(1e-3) * (z / np.sqrt(chi2_over_nu))
    raise KeyError(w.key)


def generate(w: Workload | int, d: int | None = None, threads: int | None = None) -> np.ndarray:
    """Rows [n, d'] of workload w; d' = d (a prefix of every full row) or the full size.

    fp32 workloads return float32, bf16 workloads return the uint16 bit patterns."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    dd = w.d if d is None else int(d)
    if not 0 <= dd <= w.d:
        raise ValueError("prefix longer than the row")
    out = np.empty((w.n, dd), dtype=np.float32 if w.dtype == "f32" else np.uint16)
    layout = layer_layout(w.seed, w.d) if w.key == 2 else None

    def fill(i):
        out[i] = _row(w, i, dd, layout)

    nt = threads or min(16, os.cpu_count() or 1, w.n)
    if nt <= 1 or dd * w.n < 1 << 20:
        for i in range(w.n):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=nt) as ex:
            list(ex.map(fill, range(w.n)))
    return out


def random_rows(n: int, d: int, seed: int, dtype: str = "f32", scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) rows for small parity cases (uint16 bf16 bits when dtype == 'bf16')."""
    x = np.empty((n, d), dtype=np.float32)
    for i in range(n):
        x[i] = _rng(seed, i, _C_MAIN).standard_normal(d, dtype=np.float32) * np.float32(scale)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x

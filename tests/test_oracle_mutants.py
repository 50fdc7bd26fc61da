"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case below changes one line of arithmetic in a copy of
oracle/gq_oracle.c -- a sign, a comparison, a scale, an index, a constant
of the generator, a bias, a bit position -- builds the copy into its own
library and runs the oracle's pin tests against it (the oracle loads the
library named by GQ_ORACLE_LIB).  Every mutant must make at least one pin
fail; the unchanged source must pass.  The mistakes live only in the
temporary copies: nothing here touches the GPU or the library under test.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gq_oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in
        ("test_oracle_pins.py", "test_oracle_e8_pins.py", "test_oracle_word_pins.py")]

# (name, exact text in the source, its replacement)
MUTANTS = [
    ("philox multiplier", "0xD2511F53u * (uint64_t)c[0]", "0xD2511F55u * (uint64_t)c[0]"),
    ("philox key word", "uint32_t n0 = hi1 ^ c[1] ^ k0;", "uint32_t n0 = hi1 ^ c[1] ^ k1;"),
    ("philox key schedule", "k1 += 0xBB67AE85u;", "k1 += 0xBB67AE86u;"),
    ("uniform word index", "uint32_t hi16 = (A[e / 2] >> shift) & 0xFFFFu;",
     "uint32_t hi16 = (A[e % 4] >> shift) & 0xFFFFu;"),
    ("uniform halves swapped", "return (hi16 << 16) | lo16;", "return (lo16 << 16) | hi16;"),
    ("(2,inf) root dropped", "return q_inf ? (float)m : (float)sqrt(m);",
     "return q_inf ? (float)m : (float)m;"),
    ("(inf,2) square dropped", "nsum_add(&tot, q_inf ? per_worker[i] * per_worker[i] : per_worker[i]);",
     "nsum_add(&tot, q_inf ? per_worker[i] : per_worker[i]);"),
    ("q=2 square dropped", "nsum_add(&acc, q == 2.0f ? v * v : pow(fabs(v), (double)q));",
     "nsum_add(&acc, q == 2.0f ? fabs(v) : pow(fabs(v), (double)q));"),
    ("q=inf magnitude", "float a = fabsf(load_x(x, dtype, (uint64_t)(i * d + j)));",
     "float a = load_x(x, dtype, (uint64_t)(i * d + j));"),
    ("kappa without n", "*kappa = (double)N / ((double)n * (double)oracle_top_code(s, scheme));",
     "*kappa = (double)N / ((double)oracle_top_code(s, scheme));"),
    ("sigma numerator", "double num = (scheme == ORACLE_SCHEME_L) ? (double)s : 1.0;",
     "double num = (scheme == ORACLE_SCHEME_L) ? (double)(s + 1) : 1.0;"),
    ("pre-scale", "float pr = (N < 0x1p-64f) ? 0x1p64f : 1.0f;",
     "float pr = (N < 0x1p-64f) ? 0x1p63f : 1.0f;"),
    ("clamp level", "float top = (float)s;", "float top = (float)(s + 1);"),
    ("L threshold scale", "*F = (uint32_t)(f * 0x1p32f);\n        return;",
     "*F = (uint32_t)(f * 0x1p31f);\n        return;"),
    ("E level index", "int32_t lo = (int32_t)1 << (e + s - 1);",
     "int32_t lo = (int32_t)1 << (e + s - 2);"),
    ("E fraction threshold", "*F = mant << 9;", "*F = mant << 8;"),
    ("E small-value scale", "float f = t * ldexpf(1.0f, s - 1);", "float f = t * ldexpf(1.0f, s);"),
    ("rounding direction", "int32_t m = (u < F) ? m_hi : m_lo;", "int32_t m = (u > F) ? m_hi : m_lo;"),
    ("sign dropped", "return (float_bits(xv) >> 31) ? -m : m;", "return m;"),
    ("code width", "    return bits + 1;\n}", "    return bits;\n}"),
    ("packing bit order", "out[i * rb + k / 8] |= (uint8_t)(1u << (k % 8));",
     "out[i * rb + k / 8] |= (uint8_t)(1u << (7 - k % 8));"),
    ("unpack sign", "v -= (int64_t)1 << W;", "v -= (int64_t)1 << (W - 1);"),
    ("sum skips a worker", "for (int64_t i = 0; i < n; ++i)\n            acc += codes[i * d + j];",
     "for (int64_t i = 1; i < n; ++i)\n            acc += codes[i * d + j];"),
    ("local kappa without n", "kappa = (double)norms[i] / ((double)n * (double)s);",
     "kappa = (double)norms[i] / ((double)s);"),
    ("8-bit level value", "double v = ldexp(1.0, 1 - idx);", "double v = ldexp(1.0, -idx);"),
    ("8-bit step direction", "int idx = 1 - (e + up);", "int idx = 1 - (e - up);"),
    ("8-bit threshold scale", "uint32_t F = (uint32_t)(phi * 0x1p32);",
     "uint32_t F = (uint32_t)(phi * 0x1p31);"),
    ("8-bit smallest level", "return (uint8_t)(u < F ? (sign | 127) : 0);",
     "return (uint8_t)(u < F ? (sign | 126) : 0);"),
    ("8-bit pair is a sum", "double v = 0.5 * (oracle_e8_value(a[j]) + oracle_e8_value(b[j]));",
     "double v = (oracle_e8_value(a[j]) + oracle_e8_value(b[j]));"),
    ("8-bit tree node index", "(uint32_t)m, scratch + m * d);",
     "(uint32_t)(m + 1), scratch + m * d);"),
    ("word bias", "uint32_t biased = (uint32_t)((int64_t)codes[i * d + j] + M);",
     "uint32_t biased = (uint32_t)((int64_t)codes[i * d + j] + M + 1);"),
    ("word field position", "out[i * rw + j / f] |= biased << (W * (int)(j % f));",
     "out[i * rw + j / f] |= biased << (W * (int)(j % f) + 1);"),
    ("word sum bias", "sums[j] = (int64_t)field - n * M;", "sums[j] = (int64_t)field - M;"),
]


def _run(tmp, name, text):
    """Build `text` into a library in tmp and run the pins against it: the exit code."""
    tag = "".join(c if c.isalnum() else "_" for c in name)
    src = os.path.join(tmp, f"{tag}.c")
    lib = os.path.join(tmp, f"lib_{tag}.so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-ffp-contract=off", src,
                    "-o", lib, "-lm"], check=True, capture_output=True, timeout=300)
    env = dict(os.environ, GQ_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode


@pytest.mark.timeout(900)
def test_every_planted_mistake_fails_a_pin(tmp_path):
    base = open(SRC).read()
    for name, old, new in MUTANTS:
        assert base.count(old) == 1, f"{name}: the mutated text must occur exactly once"
    jobs = [("unchanged", base)] + [(name, base.replace(old, new)) for name, old, new in MUTANTS]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        codes = list(ex.map(lambda job: _run(str(tmp_path), *job), jobs))
    assert codes[0] == 0, "the unchanged oracle must pass its pins"
    survivors = [name for (name, _), rc in zip(jobs[1:], codes[1:]) if rc == 0]
    assert survivors == [], f"planted mistakes no pin caught: {survivors}"

"""The Eq. (8) reading of the Sec. 5 performance model ("Global-QSGD:
Practical Floatless Quantization ..."): pinned by the two consequences the
page prints -- with omega_S = 1 standard dithering always speeds up, and with
omega_E = 1/79 exponential dithering speeds up iff beta < 0.08 gamma (rho = 4)."""
import math

import pytest

from bench import eq8_threshold


def test_printed_consequences():
    assert eq8_threshold(4.0, 1.0) == math.inf
    assert eq8_threshold(4.0, 1.0 / 79.0) == pytest.approx(0.08, rel=1e-12)


def test_monotone_in_omega_and_rho():
    assert eq8_threshold(4.0, 1 / 50) > eq8_threshold(4.0, 1 / 79) > eq8_threshold(4.0, 1 / 200)
    assert eq8_threshold(8.0, 1 / 79) > eq8_threshold(4.0, 1 / 79)
    # rho omega = 1 is the boundary of "always"
    assert eq8_threshold(4.0, 0.25) == math.inf

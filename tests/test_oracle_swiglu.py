"""Pins of the oracle's SwiGLU with alpha, beta and clamp.

The pages name the three parameters and say they must survive the
quantization bridge (PR "Incubate DeepSeek V4 WNA16 runtime on SM86", "What
this branch adds" item 9) but print no formula.  Reading used here:
g' = min(g, c), u' = clamp(u, -c, c), act = g' * sigmoid(alpha g') * (u' + beta).
Each test checks a property that a plausible slip in that reading would break.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle import oracle as O

INF = float("inf")


def test_plain_swiglu_is_silu_times_up():
    """alpha = 1, beta = 0, no clamp: the textbook silu(g) * u."""
    for g in np.linspace(-12, 12, 49):
        for u in (-3.5, -1.0, 0.0, 0.25, 2.0, 40.0):
            ref = g * expit(g) * u
            assert O.swiglu(g, u) == pytest.approx(ref, rel=1e-14, abs=1e-300)


def test_closed_form_point():
    """sigmoid(ln 3) = 3/4, so act(ln 3, 2) = 1.5 ln 3."""
    assert O.swiglu(math.log(3.0), 2.0) == pytest.approx(1.5 * math.log(3.0), rel=1e-15)


def test_alpha_scales_the_gate_logit():
    """act(g, 1; alpha, beta=0)/g = sigmoid(alpha g), so its log-odds is alpha*g."""
    for alpha in (0.5, 1.702, 3.0):
        for g in (-2.0, -0.3, 0.7, 2.5):
            r = O.swiglu(g, 1.0, alpha, 0.0, INF) / g
            assert math.log(r / (1.0 - r)) == pytest.approx(alpha * g, rel=1e-12)


def test_beta_adds_to_up():
    """u = -beta zeroes the output for any gate; beta shifts u linearly."""
    for g in (-3.0, 0.5, 4.0):
        assert O.swiglu(g, -1.0, 1.702, 1.0, 7.0) == 0.0
        a0 = O.swiglu(g, 2.0, 1.702, 0.0, INF)
        a1 = O.swiglu(g, 2.0, 1.702, 1.0, INF)
        assert a1 == pytest.approx(a0 * 3.0 / 2.0, rel=1e-14)


def test_zero_gate_gives_zero():
    for u in (-9.0, 0.0, 9.0):
        assert O.swiglu(0.0, u, 1.702, 1.0, 7.0) == 0.0


def test_gate_clamped_from_above_only():
    c, a, b = 7.0, 1.702, 1.0
    top = O.swiglu(c, 2.0, a, b, c)
    assert top == pytest.approx(c * expit(a * c) * (2.0 + b), rel=1e-14)
    for g in (7.0 + 1e-9, 8.0, 50.0, 1e6):
        assert O.swiglu(g, 2.0, a, b, c) == top       # saturates at the clamp
    # far below -c the gate stays unclamped: the output is ~g e^{alpha g}, not
    # the value at g = -c
    low = O.swiglu(-30.0, 2.0, a, b, c)
    at_minus_c = O.swiglu(-c, 2.0, a, b, c)
    assert abs(low) < 1e-19 and abs(at_minus_c) > 1e-5
    assert low == pytest.approx(-30.0 * expit(-a * 30.0) * 3.0, rel=1e-12)


def test_up_clamped_on_both_sides_before_beta():
    c, a, b, g = 7.0, 1.702, 1.0, 1.5
    gate = g * expit(a * g)
    assert O.swiglu(g, 100.0, a, b, c) == pytest.approx(gate * (c + b), rel=1e-14)
    assert O.swiglu(g, -100.0, a, b, c) == pytest.approx(gate * (-c + b), rel=1e-14)
    assert O.swiglu(g, c, a, b, c) == O.swiglu(g, c + 5.0, a, b, c)
    assert O.swiglu(g, -c, a, b, c) == O.swiglu(g, -c - 5.0, a, b, c)
    # inside the clamp nothing changes
    assert O.swiglu(g, 6.5, a, b, c) == O.swiglu(g, 6.5, a, b, INF)


def test_large_negative_gate_underflows_to_zero_cleanly():
    assert O.swiglu(-1000.0, 3.0) == 0.0 or abs(O.swiglu(-1000.0, 3.0)) < 1e-300

"""Pins for the oracle's fused bounded gate (CPU only).

Sources: "Inside Kimi K3" (academa.ai lecture), sequence paragraph (the decay
curve is changed so that log alpha is bounded below at -5); "Kimi K3's
architecture" (orkas.ai), "A lower bound that deleted a GPU code path" (each
step forgets down to 0.67% and no further).  The curve itself is not printed;
the reading is log alpha = -5 * sigmoid(x).

Pins (closed forms of the curve, chosen so that a wrong scale, a wrong sign of
x, a missing bound or a swapped branch fails one of them):

* x = 0 gives exactly -2.5; the curve is odd about (0, -2.5):
  f(x) + f(-x) = -5;
* f(x) -> 0 as x -> -inf and -> -5 as x -> +inf, never leaving (-5, 0) for
  finite x that do not round to the limits, and monotone decreasing;
* f'(0) = -5/4 (central difference);
* the gated recurrence equals the recurrence fed log alpha = -5 / (1 + e^{-x})
  evaluated independently here, and one step with beta = 0 decays S0 by
  exactly alpha = exp(f(x)) >= e^-5.
"""
import numpy as np

import oracle


def test_curve_closed_forms():
    f = oracle.gate_log_alpha
    assert f(np.array([0.0]))[0] == -2.5
    x = np.linspace(-30, 30, 601)
    y = f(x)
    assert np.allclose(y + f(-x), -5.0, atol=1e-12)
    assert np.all(np.diff(y) < 0)
    assert np.all((y < 0) & (y > -5))
    assert abs(f(np.array([-800.0]))[0]) < 1e-300 and f(np.array([800.0]))[0] == -5.0
    h = 1e-5
    d = (f(np.array([h]))[0] - f(np.array([-h]))[0]) / (2 * h)
    assert abs(d + 1.25) < 1e-9


def test_gated_recurrence_matches_explicit_curve():
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 2, 9, 2, 6, 5
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = 3.0 * rng.standard_normal((B, T, H, dk))
    bt = rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    la = np.array([[[[-5.0 / (1.0 + np.exp(-x)) for x in row] for row in hh] for hh in tt] for tt in g])
    o1, s1 = oracle.prefill_gate(q, k, v, g, bt, S0)
    o2, s2 = oracle.prefill(q, k, v, la, bt, S0)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-13) and np.allclose(s1, s2, rtol=1e-13, atol=1e-13)


def test_one_step_pure_decay_is_bounded():
    rng = np.random.default_rng(12)
    dk, dv = 8, 4
    g = np.array([-40.0, -3.0, 0.0, 0.5, 2.0, 7.0, 40.0, 80.0])[None, None, None]
    S0 = rng.standard_normal((1, 1, dk, dv))
    z = np.zeros((1, 1, 1, dk))
    _, s1 = oracle.prefill_gate(z, z, np.zeros((1, 1, 1, dv)), g, np.zeros((1, 1, 1)), S0)
    alpha = np.exp(-5.0 / (1.0 + np.exp(-g[0, 0, 0])))
    assert np.allclose(s1[0, 0], alpha[:, None] * S0[0, 0], rtol=1e-14, atol=0)
    assert np.all(alpha >= np.exp(-5.0) * (1 - 1e-15))

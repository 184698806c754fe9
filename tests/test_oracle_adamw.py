"""Pins of the AdamW oracle against values and facts fixed outside of it.

* the decay experiment printed by the handbook (Adam + L2 vs AdamW, gradients
  a thousand times apart), which also pins bias correction;
* the closed form of the first step and of a constant gradient;
* pure decay under a zero gradient; special cases of cautious decay.
"""
import numpy as np
import pytest

from oracle import adamw_step


def _run_decay_experiment(decoupled, bias_correction_steps=None):
    lr, wd = 1e-2, 0.1
    scale = np.array([0.01, 10.0])
    w, m, v = np.ones(2), np.zeros(2), np.zeros(2)
    for t in range(1000):
        r = adamw_step(w, scale * (-1.0) ** t, m, v, step=t + 1, lr=lr, beta1=0.9, beta2=0.999,
                       eps=1e-8, weight_decay=wd, decoupled=decoupled)
        w, m, v = r.param, r.exp_avg, r.exp_avg_sq
    return w


def test_decay_experiment_matches_printed(golden):
    g = golden("adamw_decay_experiment.txt")
    coupled = _run_decay_experiment(False)
    decoupled = _run_decay_experiment(True)
    assert f"{coupled[0]:.3f}" == g["coupled_small"][0]
    assert f"{coupled[1]:.3f}" == g["coupled_large"][0]
    assert f"{decoupled[0]:.3f}" == g["decoupled_small"][0]
    assert f"{decoupled[1]:.3f}" == g["decoupled_large"][0]
    assert f"{(1 - 1e-2 * 0.1) ** 1000:.3f}" == g["decay_only_theory"][0]


def test_first_step_closed_form():
    rng = np.random.default_rng(0)
    p = rng.standard_normal(1000)
    g = 1e-3 * rng.standard_normal(1000)
    r = adamw_step(p, g, np.zeros(1000), np.zeros(1000), step=1, lr=3e-3, beta1=0.9, beta2=0.95,
                   eps=1e-8, weight_decay=0.1)
    # t = 1: mhat = g, vhat = g^2, so the update is lr * g / (|g| + eps)
    want = p * (1 - 3e-3 * 0.1) - 3e-3 * g / (np.abs(g) + 1e-8)
    assert np.max(np.abs(r.param - want)) < 1e-15
    assert np.allclose(r.exp_avg, 0.1 * g, rtol=1e-14, atol=0)
    assert np.allclose(r.exp_avg_sq, 0.05 * g * g, rtol=1e-14, atol=0)
    # nearly sign(g) once |g| >> eps
    zero = adamw_step(np.zeros(1000), g, np.zeros(1000), np.zeros(1000), step=1, lr=3e-3,
                      beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.0).param
    assert np.max(np.abs(zero + 3e-3 * np.sign(g))) < 3e-3 * 1e-8 / np.abs(g).min() * 1.01


def test_constant_gradient_bias_correction():
    # With the same gradient every step the bias-corrected moments equal g and
    # g^2 at every t, so each step moves by lr * g / (|g| + eps).
    g = np.array([1e-3, -2e-2, 5.0])
    w, m, v = np.zeros(3), np.zeros(3), np.zeros(3)
    for t in range(1, 40):
        r = adamw_step(w, g, m, v, step=t, lr=1e-2, beta1=0.9, beta2=0.95, eps=1e-8,
                       weight_decay=0.0)
        assert np.allclose(r.param - w, -1e-2 * g / (np.abs(g) + 1e-8), rtol=1e-12, atol=0)
        w, m, v = r.param, r.exp_avg, r.exp_avg_sq


def test_zero_gradient_is_pure_decay():
    p0 = np.linspace(-2, 2, 9)
    w, m, v = p0.copy(), np.zeros(9), np.zeros(9)
    for t in range(1, 101):
        r = adamw_step(w, np.zeros(9), m, v, step=t, lr=1e-2, weight_decay=0.1)
        w, m, v = r.param, r.exp_avg, r.exp_avg_sq
    assert np.allclose(w, p0 * (1 - 1e-3) ** 100, rtol=1e-13, atol=0)
    assert np.all(m == 0) and np.all(v == 0)


def test_coupled_and_decoupled_agree_without_decay():
    rng = np.random.default_rng(1)
    p, g = rng.standard_normal(50), rng.standard_normal(50)
    a = adamw_step(p, g, np.zeros(50), np.zeros(50), step=3, lr=1e-2, weight_decay=0.0, decoupled=True)
    b = adamw_step(p, g, np.zeros(50), np.zeros(50), step=3, lr=1e-2, weight_decay=0.0, decoupled=False)
    assert np.array_equal(a.param, b.param)


def test_cautious_special_cases():
    rng = np.random.default_rng(2)
    g = rng.standard_normal(64)
    kw = dict(step=1, lr=1e-2, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    same = np.abs(rng.standard_normal(64)) * np.sign(g)  # update has the sign of g at t = 1
    a = adamw_step(same, g, np.zeros(64), np.zeros(64), cautious_wd=True, **kw).param
    b = adamw_step(same, g, np.zeros(64), np.zeros(64), cautious_wd=False, **kw).param
    assert np.array_equal(a, b)
    opp = -same
    c = adamw_step(opp, g, np.zeros(64), np.zeros(64), cautious_wd=True, **kw).param
    d = adamw_step(opp, g, np.zeros(64), np.zeros(64), weight_decay=0.0,
                   **{k: v for k, v in kw.items() if k != "weight_decay"}).param
    assert np.array_equal(c, d)


def test_step_must_start_at_one():
    with pytest.raises(ValueError):
        adamw_step(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), step=0, lr=1e-3)

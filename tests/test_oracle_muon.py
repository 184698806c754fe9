"""Pins of the Muon oracle against values and facts fixed outside of it.

The oracle evaluates the Newton-Schulz result through the eigendecomposition of the
Gram matrix; it is pinned here against two other formulations of the same thing:

* the iteration as the handbook prints it, matrix products repeated in float64
  (normalise, transpose a tall matrix, X <- a X + (b R + c R R) X with R = X X^T,
  transpose back);
* the closed form through numpy's SVD (Newton-Schulz acts on the singular values
  only, through the scalar quintic p(x) = a x + b x^3 + c x^5);

and against
* the cubic (1.5, -0.5, 0) iteration, which converges to the exact polar factor
  U V^T that numpy's SVD gives;
* the spectra, energy and RMS printed by the handbook's orthogonalize.py run;
* the quintic's invariant band, transpose symmetry, steepest-descent sign;
* momentum and Nesterov closed forms over several steps, zero-gradient decay,
  and the special cases of cautious weight decay.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import QUINTIC, muon_step, newton_schulz, route, update_scale


def _rand(shape, seed, row_scale=0.0):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(shape)
    if row_scale:
        g *= np.exp(row_scale * rng.standard_normal((shape[0], 1)))
    return g


def _quintic_scalar(x, steps, coeffs=QUINTIC):
    a, b, c = coeffs
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def _svd_closed_form(G, steps, coeffs=QUINTIC, eps=1e-7):
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    f = _quintic_scalar(s / (np.linalg.norm(G) + eps), steps, coeffs)
    return (U * f) @ Vt


def _printed_iteration(G, steps, coeffs=QUINTIC, eps=1e-7):
    """The handbook's newton_schulz, as matrix products in float64."""
    table = [coeffs] * steps if np.ndim(coeffs) == 1 else [tuple(r) for r in coeffs]
    X = G / (np.linalg.norm(G) + eps)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    for a, b, c in table:
        R = X @ X.T
        X = a * X + (b * R + c * R @ R) @ X
    return X.T if tall else X


@pytest.mark.parametrize("shape,seed", [((64, 128), 0), ((128, 64), 1), ((96, 96), 2),
                                        ((40, 130), 3), ((1, 9), 4), ((9, 1), 5)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5, 7])
@pytest.mark.parametrize("coeffs", [QUINTIC, (2.0, -1.5, 0.5), (1.5, -0.5, 0.0),
                                    (0.0, 1.0, 0.0), (0.0, 0.0, 1.0), (1.0, 0.0, 0.0)])
def test_ns_matches_printed_iteration(shape, seed, steps, coeffs):
    """Term by term: (0, 1, 0) is the b R X term alone, (0, 0, 1) the c R^2 X term,
    (1, 0, 0) the a X term (normalisation only).  The repeated products carry their own
    float64 rounding, which each iteration amplifies at most by the polynomial's slope
    (a = 3.4445 near zero): the bound grows with it."""
    G = _rand(shape, seed, row_scale=1.0)
    got = newton_schulz(G, steps, coeffs)
    ref = _printed_iteration(G, steps, coeffs)
    tol = 1e-14 * 3.5 ** steps
    assert np.max(np.abs(got - ref)) <= tol * max(1.0, np.max(np.abs(ref)))


def test_ns_per_iteration_table_matches_printed_iteration():
    G = _rand((70, 45), 8, row_scale=1.0)
    table = np.array([[3.4445, -4.7750, 2.0315], [2.0, -1.5, 0.5], [1.5, -0.5, 0.0]])
    assert np.max(np.abs(newton_schulz(G, 3, table) - _printed_iteration(G, 3, table))) < 1e-12


def test_ns_zero_and_non_finite_inputs():
    assert np.array_equal(newton_schulz(np.zeros((6, 9))), np.zeros((6, 9)))
    for bad in (np.nan, np.inf):
        G = _rand((6, 9), 1)
        G[2, 3] = bad
        with np.errstate(invalid="ignore"):
            ref = _printed_iteration(G, 1)
            got = newton_schulz(G, 1)
        assert np.all(np.isnan(ref)) and np.all(np.isnan(got))


@pytest.mark.parametrize("shape,seed", [((64, 128), 0), ((128, 64), 1), ((96, 96), 2), ((40, 130), 3)])
@pytest.mark.parametrize("steps", [0, 1, 5, 7])
def test_ns_matches_svd_closed_form(shape, seed, steps):
    G = _rand(shape, seed, row_scale=1.0)
    got = newton_schulz(G, steps)
    ref = _svd_closed_form(G, steps)
    # the oracle decomposes X X^T, whose small eigenvalues carry absolute (not relative)
    # float64 errors; the polynomial's slope near zero (a per step) scales them
    assert np.max(np.abs(got - ref)) < 1e-14 * 3.5 ** steps


def test_ns_per_iteration_table_matches_closed_form():
    G = _rand((48, 80), 7)
    table = np.array([[3.4445, -4.7750, 2.0315], [2.0, -1.5, 0.5], [1.5, -0.5, 0.0]])
    got = newton_schulz(G, 3, table)
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    x = s / (np.linalg.norm(G) + 1e-7)
    for a, b, c in table:
        x = a * x + b * x ** 3 + c * x ** 5
    assert np.max(np.abs(got - (U * x) @ Vt)) < 1e-12


@pytest.mark.parametrize("shape", [(30, 50), (50, 30), (40, 40)])
def test_cubic_iteration_reaches_exact_polar_factor(shape):
    # Coefficients (1.5, -0.5, 0) turn the same iteration into the classical
    # cubic Newton-Schulz, which converges to U V^T for a full-rank input.
    rng = np.random.default_rng(11)
    U, _ = np.linalg.qr(rng.standard_normal((shape[0], min(shape))))
    V, _ = np.linalg.qr(rng.standard_normal((shape[1], min(shape))))
    s = np.linspace(1.0, 0.3, min(shape))
    G = (U * s) @ V.T
    got = newton_schulz(G, 60, (1.5, -0.5, 0.0))
    Ug, _, Vgt = np.linalg.svd(G, full_matrices=False)
    assert np.max(np.abs(got - Ug @ Vgt)) < 1e-10


def test_identity_coefficients_only_normalise():
    G = _rand((20, 33), 5)
    got = newton_schulz(G, 4, (1.0, 0.0, 0.0), eps=1e-7)
    assert np.allclose(got, G / (np.linalg.norm(G) + 1e-7), rtol=0, atol=1e-15)


def _printed_input(seed=0):
    rng = np.random.default_rng(seed)
    U, _ = np.linalg.qr(rng.standard_normal((256, 256)))
    V, _ = np.linalg.qr(rng.standard_normal((1024, 256)))
    S = np.logspace(0, -2, 256)
    return U, S, V, (U * S) @ V.T


@pytest.mark.parametrize("steps", [1, 3, 5])
def test_ns_printed_spectra(golden, steps):
    g = golden("ns_spectrum.txt")
    lo_band, hi_band = (float(v) for v in g["band_open"])
    *_, G = _printed_input()
    s = np.linalg.svd(newton_schulz(G, steps), compute_uv=False)
    lo, hi = (float(v) for v in g[f"steps{steps}_range"])
    assert f"{s.min():.2f}" == f"{lo:.2f}" and f"{s.max():.2f}" == f"{hi:.2f}"
    frac = np.mean((s > lo_band) & (s < hi_band))
    assert f"{frac:.0%}" == g[f"steps{steps}_in_band_pct"][0] + "%"


def test_ns_printed_energy_and_rms(golden):
    g = golden("ns_spectrum.txt")
    _, S, V, G = _printed_input()
    X = newton_schulz(G)
    before = (S[:8] ** 2).sum() / (S ** 2).sum()
    after = np.linalg.norm(X @ V[:, :8]) ** 2 / np.linalg.norm(X) ** 2
    assert f"{before:.0%}" == g["top8_energy_before_pct"][0] + "%"
    assert f"{after:.1%}" == g["top8_energy_after_pct"][0] + "%"
    assert f"{np.sqrt(np.mean(X ** 2)):.4f}" == g["rms_after"][0]
    assert f"{1024 ** -0.5:.4f}" == g["rms_reference"][0]
    scaled = X * update_scale(256, 1024)
    assert f"{np.sqrt(np.mean(scaled ** 2)):.2f}" == g["rms_scaled"][0]


def test_printed_spectra_do_not_depend_on_the_rotations(golden):
    g = golden("ns_spectrum.txt")
    *_, G = _printed_input(seed=123)
    s = np.linalg.svd(newton_schulz(G, 5), compute_uv=False)
    assert f"{s.min():.2f}" == g["steps5_range"][0] and f"{s.max():.2f}" == g["steps5_range"][1]


def test_quintic_band():
    # p(x) = a x + b x^3 + c x^5 peaks near 1.2024 and dips near 0.6818 on [0, 1.2]:
    # every normalised singular value above ~1.51e-3 lands in that band in 5 steps,
    # and the band maps into itself.
    xs = np.linspace(0.0, 1.3, 200001)
    p = _quintic_scalar(xs, 1)
    peak = p[xs <= 0.8].max()
    dip = p[(xs > 0.8) & (xs <= 1.2)].min()
    assert abs(peak - 1.2024) < 1e-3 and abs(dip - 0.6818) < 1e-3
    band = np.linspace(dip, peak, 10001)
    pb = _quintic_scalar(band, 1)
    assert pb.min() >= dip - 1e-12 and pb.max() <= peak + 1e-12
    # Matrices: condition number ~1e4 (row and column log-normal scales).
    rng = np.random.default_rng(3)
    G = np.exp(rng.standard_normal((60, 1))) * rng.standard_normal((60, 150)) * np.exp(rng.standard_normal((1, 150)))
    sg = np.linalg.svd(G, compute_uv=False) / (np.linalg.norm(G) + 1e-7)
    so = np.linalg.svd(newton_schulz(G, 5), compute_uv=False)  # same order (p monotone below the peak)
    big = sg >= 1.51e-3
    assert big.sum() > 10
    assert np.all(so[big] >= dip - 1e-9) and np.all(so[big] <= peak + 1e-9)


@pytest.mark.parametrize("shape", [(64, 128), (128, 64), (77, 77)])
def test_ns_transpose_symmetry(shape):
    G = _rand(shape, 9)
    if shape[0] != shape[1]:
        # rectangular: both orientations iterate on the same short-side X
        assert np.array_equal(newton_schulz(G.T), newton_schulz(G).T)
    else:
        assert np.max(np.abs(newton_schulz(G.T) - newton_schulz(G).T)) < 1e-13


def test_ns_shares_singular_vectors_and_descends():
    G = _rand((50, 90), 4, row_scale=1.0)
    O = newton_schulz(G)
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    core = U.T @ O @ Vt.T
    off = core - np.diag(np.diag(core))
    assert np.max(np.abs(off)) < 1e-12
    assert np.all(np.diag(core) > 0)
    # Exercise 1 of the handbook: U V^T minimises <G, dW> under a spectral-norm
    # bound; the orthogonalised update must be a descent direction.
    assert np.sum(G * O) > 0


def test_route():
    assert route(64, 128) == oracle.Route(False, 64, 128, 5)
    assert route(128, 64) == oracle.Route(True, 64, 128, 5)
    assert route(768, 768) == oracle.Route(False, 768, 768, 5)
    assert route(2048, 512, 3) == oracle.Route(True, 512, 2048, 3)


def test_update_scales():
    assert update_scale(256, 1024) == pytest.approx(0.2 * 32)
    assert update_scale(1024, 256) == pytest.approx(0.2 * 32)
    assert update_scale(1024, 256, 1) == pytest.approx(2.0)
    assert update_scale(256, 1024, 1) == pytest.approx(1.0)


HP = dict(lr=0.02, mu=0.95, weight_decay=0.1)


def test_muon_zero_gradient_is_pure_decay():
    P0 = _rand((24, 40), 1)
    P, M = P0.copy(), np.zeros_like(P0)
    for _ in range(7):
        r = muon_step(P, np.zeros_like(P0), M, **HP)
        P, M = r.param, r.momentum
        assert np.all(r.ortho == 0)
    assert np.allclose(P, P0 * (1 - 0.02 * 0.1) ** 7, rtol=1e-14, atol=0)


@pytest.mark.parametrize("nesterov", [True, False])
def test_muon_momentum_and_nesterov_closed_form(nesterov):
    mu = 0.95
    shape = (16, 28)
    grads = [_rand(shape, 100 + t) for t in range(4)]
    P, M = _rand(shape, 7), np.zeros(shape)
    for t, G in enumerate(grads):
        r = muon_step(P, G, M, lr=0.02, mu=mu, weight_decay=0.1, nesterov=nesterov)
        # M_t = sum_k mu^(t-k) G_k
        m_closed = sum(mu ** (t - k) * grads[k] for k in range(t + 1))
        assert np.allclose(r.momentum, m_closed, rtol=1e-13, atol=1e-13)
        # Nesterov input (1 + mu) G_t + sum_{k<t} mu^(t-k+1) G_k, else M_t itself
        if nesterov:
            u = (1 + mu) * grads[t] + sum(mu ** (t - k + 1) * grads[k] for k in range(t))
        else:
            u = m_closed
        assert np.allclose(r.ortho, _svd_closed_form(u, 5), rtol=0, atol=1e-11)
        s = 0.2 * math.sqrt(max(shape))
        assert np.allclose(r.param, P * (1 - 0.02 * 0.1) - 0.02 * s * r.ortho, rtol=0, atol=1e-14)
        P, M = r.param, r.momentum


def test_muon_cautious_special_cases():
    G = _rand((12, 20), 2)
    O = _svd_closed_form(1.95 * G, 5)  # first step: U = (1 + mu) G
    s = 0.2 * math.sqrt(20)
    # same sign everywhere: cautious decay equals plain decay
    P_same = np.abs(_rand((12, 20), 3)) * np.sign(O)
    a = muon_step(P_same, G, np.zeros_like(G), cautious_wd=True, **HP).param
    b = muon_step(P_same, G, np.zeros_like(G), cautious_wd=False, **HP).param
    assert np.array_equal(a, b)
    # opposite sign everywhere: no decay at all
    P_opp = -P_same
    c = muon_step(P_opp, G, np.zeros_like(G), cautious_wd=True, **HP).param
    assert np.allclose(c, P_opp - 0.02 * s * O, rtol=0, atol=1e-13)
    # mixed signs, entry by entry (brute force on a tiny matrix)
    P_mix = _rand((12, 20), 4)
    d = muon_step(P_mix, G, np.zeros_like(G), cautious_wd=True, **HP).param
    for i in range(12):
        for j in range(20):
            keep = 1.0 if O[i, j] * P_mix[i, j] > 0 else 0.0
            want = P_mix[i, j] - keep * 0.02 * 0.1 * P_mix[i, j] - 0.02 * s * O[i, j]
            assert abs(d[i, j] - want) < 1e-13


def test_muon_bucket_matches_per_matrix():
    K, A, B = 3, 10, 14
    P, G = _rand((K, A, B), 1), _rand((K, A, B), 2)
    p, m, o, r = oracle.muon_step_bucket(P, G, np.zeros_like(P), **HP)
    for k in range(K):
        one = muon_step(P[k], G[k], np.zeros((A, B)), **HP)
        assert np.array_equal(p[k], one.param) and np.array_equal(o[k], one.ortho)
    assert r == route(A, B)

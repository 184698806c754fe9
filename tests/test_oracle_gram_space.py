"""The Gram-space form of the Newton-Schulz iteration ("DMuon: Efficient Distributed Muon
Training with Near-Adam Overhead", section 2.2), restated here in float64, equals the
printed iteration (the oracle) up to float64 rounding: the opt-in GPU route computes the
same thing, and its larger errors come from bf16 alone."""
import numpy as np
import pytest

import oracle


def gram_space_fp64(G, steps, coeffs=oracle.muon.QUINTIC, eps=1e-7):
    X0 = np.array(G, dtype=np.float64)
    X0 = X0 / (np.linalg.norm(X0) + eps)
    t = X0.shape[0] > X0.shape[1]
    if t:
        X0 = X0.T
    m = X0.shape[0]
    R = X0 @ X0.T
    Q = np.eye(m)
    table = np.broadcast_to(np.asarray(coeffs, dtype=np.float64), (steps, 3))
    for a, b, c in table:
        P = a * np.eye(m) + b * R + c * (R @ R)   # X_{k+1} = P_k X_k
        Q = P @ Q                                  # X_N = Q_N X_0
        R = P @ R @ P                              # R_{k+1} = X_{k+1} X_{k+1}^T
    X = Q @ X0
    return X.T if t else X


@pytest.mark.parametrize("shape", [(40, 100), (100, 40), (64, 64), (1, 9), (30, 300)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_gram_space_equals_printed_iteration(shape, steps):
    G = np.random.default_rng(sum(shape) + steps).standard_normal(shape)
    ref = oracle.newton_schulz(G, steps)
    got = gram_space_fp64(G, steps)
    assert np.max(np.abs(got - ref)) < 1e-11 * max(1.0, np.max(np.abs(ref)))


def test_gram_space_per_iteration_table():
    table = np.array([(3.4445, -4.7750, 2.0315), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)])
    G = np.random.default_rng(3).standard_normal((50, 120))
    assert np.allclose(gram_space_fp64(G, 3, table), oracle.newton_schulz(G, 3, table),
                       rtol=0, atol=1e-11)


def test_gram_space_factors_commute():
    """Every factor is a polynomial in R_0, so P_k, Q_k and R_k commute and their products
    are symmetric (what lets the GPU route run them on lower-triangle tiles)."""
    G = np.random.default_rng(4).standard_normal((30, 80))
    X0 = G / np.linalg.norm(G)
    R = X0 @ X0.T
    Q = np.eye(30)
    a, b, c = oracle.muon.QUINTIC
    for _ in range(3):
        P = a * np.eye(30) + b * R + c * (R @ R)
        for A, B in ((P, Q), (R, P), (P, R @ P)):
            AB = A @ B
            assert np.max(np.abs(AB - AB.T)) < 1e-12 * np.max(np.abs(AB))
        Q = P @ Q
        R = P @ R @ P

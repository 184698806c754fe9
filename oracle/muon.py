"""fp64 CPU oracle of the Muon update.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.

Sources (page titles as published):

* [HB] "Optimizers: AdamW, Muon and the distributed optimizer" (AI infra
  handbook), section "Muon: orthogonalising the update": the three-step
  update (sum-form momentum, orthogonalised Nesterov momentum, 0.2*sqrt(max(A,B))
  scale), the newton_schulz and Muon listings, and the remark on Keller
  Jordan's sqrt(max(1, A/B)) scaling.
* [DM] "dtensor-muon" package description, sections "Features" and "Key
  options": Nesterov switch, cautious weight decay (decay only where the
  update and the parameter have the same sign).

Each function is the pages' definition written out in float64 with numpy; the
library primitives are the matrix product and the symmetric eigendecomposition.
Pins: tests/test_oracle_muon.py.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Sequence, Tuple

import numpy as np

# [HB] newton_schulz listing: the quintic's coefficients (a, b, c).
QUINTIC = (3.4445, -4.7750, 2.0315)


@dataclass(frozen=True)
class Route:
    """How one A x B matrix is orthogonalised.

    [HB] newton_schulz listing: the matrix is transposed when it has more rows
    than columns (strictly), so that X X^T is the smaller Gram matrix.  m is the
    Gram side, n the long side.
    """

    transposed: bool
    m: int
    n: int
    ns_steps: int


def route(A: int, B: int, ns_steps: int = 5) -> Route:
    t = A > B
    return Route(transposed=t, m=B if t else A, n=A if t else B, ns_steps=ns_steps)


def _coeff_table(coeffs, steps: int) -> Sequence[Tuple[float, float, float]]:
    c = np.asarray(coeffs, dtype=np.float64)
    if c.ndim == 1:
        return [tuple(c)] * steps
    if c.shape != (steps, 3):
        raise ValueError("coefficient table must be (ns_steps, 3)")
    return [tuple(r) for r in c]


def _spectral_factor(t: np.ndarray, table) -> np.ndarray:
    """h(t) = f(s) / s for the squared normalised singular values t = s^2, where f is the
    composition of the scalar polynomials p_k(s) = a_k s + b_k s^3 + c_k s^5.

    Each p_k(s) = s q_k(s^2) with q_k(t) = a_k + b_k t + c_k t^2, so along the orbit
    s_{k+1} = s_k q_k(t_k) of one singular value, t_{k+1} = t_k q_k(t_k)^2 and
    f(s) / s = q_1(t_1) q_2(t_2) ... : no division by s (zero singular values included).
    """
    h = np.ones_like(t)
    for a, b, c in table:
        q = a + b * t + c * t * t
        h = h * q
        t = t * q * q
    return h


def newton_schulz(G: np.ndarray, steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7) -> np.ndarray:
    """The matrix the quintic Newton-Schulz iteration produces from G, in float64.

    [HB] Muon section: G is divided by its Frobenius norm plus eps, then each of the
    ``steps`` iterations replaces X by a X + b (X X^T) X + c (X X^T)^2 X.  Every term is
    a polynomial in X X^T times X, so with the singular value decomposition
    X = U diag(s) V^T one iteration gives U diag(a s + b s^3 + c s^5) V^T: the singular
    vectors are kept and each singular value follows the scalar polynomial on its own
    (the section's point: all of them are pushed toward 1).  The oracle evaluates that
    result directly instead of repeating the matrix products: with the smaller Gram
    matrix X X^T = Q diag(t) Q^T (t = s^2; eigendecomposition in float64), U = Q and
    diag(s) V^T = Q^T X, so the result is Q diag(h(t)) Q^T X with h(t) = f(s) / s
    (_spectral_factor).  For a matrix with more rows than columns the Gram matrix of the
    transpose is the smaller one: the result is computed for G^T and transposed back
    (the value is the same either way; [HB] transposes for the same reason, cost).
    ``coeffs`` is one (a, b, c) triple or a per-iteration (steps, 3) table.
    """
    X = np.array(G, dtype=np.float64, copy=True)
    if X.ndim != 2:
        raise ValueError("newton_schulz takes one 2-D matrix")
    X = X / (np.linalg.norm(X) + eps)
    if not np.all(np.isfinite(X)):
        # a NaN or Inf anywhere reaches every entry through the products X X^T and
        # (X X^T)^2 of the first iteration
        return np.full(X.shape, np.nan)
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = np.ascontiguousarray(X.T)
    t, Q = np.linalg.eigh(X @ X.T)
    h = _spectral_factor(t, _coeff_table(coeffs, steps))
    O = (Q * h) @ (Q.T @ X)
    return O.T if transposed else O


def update_scale(A: int, B: int, scale_mode: int = 0) -> float:
    """Shape scale of the orthogonalised update.

    [HB] step 3 of the update: 0.2 * sqrt(max(A, B)) (update RMS near 0.2).
    [HB] remark on Keller Jordan's original scaling: sqrt(max(1, A/B)).
    """
    if scale_mode == 0:
        return 0.2 * math.sqrt(max(A, B))
    if scale_mode == 1:
        return math.sqrt(max(1.0, A / B))
    raise ValueError("scale_mode must be 0 or 1")


@dataclass
class MuonResult:
    param: np.ndarray
    momentum: np.ndarray
    ortho: np.ndarray  # NS output in the parameter's own orientation
    route: Route


def muon_step(param: np.ndarray, grad: np.ndarray, momentum: np.ndarray, *, lr: float,
              mu: float = 0.95, weight_decay: float = 0.0, nesterov: bool = True,
              ns_steps: int = 5, coeffs=QUINTIC, ns_eps: float = 1e-7,
              cautious_wd: bool = False, scale_mode: int = 0) -> MuonResult:
    """One Muon step on one A x B matrix, in float64.

    [HB] the update's three steps: the momentum is the running sum M <- mu M + G
    (M starts at zero); the matrix that is orthogonalised is the Nesterov look-ahead
    G + mu M with the new M (or M itself without Nesterov); the parameter takes the
    orthogonalised matrix O scaled by s = update_scale(A, B) and the learning rate,
    after the decoupled decay P (1 - lr wd) of the old parameter.
    [DM] cautious weight decay: the decay applies only where the update u = s O and
    the old parameter have the same sign (u * p > 0, strict).
    """
    P = np.asarray(param, dtype=np.float64)
    G = np.asarray(grad, dtype=np.float64)
    M = np.asarray(momentum, dtype=np.float64)
    A, B = P.shape
    M = mu * M + G
    U = G + mu * M if nesterov else M
    O = newton_schulz(U, ns_steps, coeffs, ns_eps)
    s = update_scale(A, B, scale_mode)
    if cautious_wd:
        decay = np.where((s * O) * P > 0, lr * weight_decay, 0.0)
    else:
        decay = lr * weight_decay
    P_new = P - decay * P - lr * s * O
    return MuonResult(param=P_new, momentum=M, ortho=O, route=route(A, B, ns_steps))


def muon_step_bucket(params: np.ndarray, grads: np.ndarray, momenta: np.ndarray, **hp):
    """muon_step on each matrix of a (K, A, B) stack; matrices are independent."""
    outs = [muon_step(params[k], grads[k], momenta[k], **hp) for k in range(params.shape[0])]
    return (np.stack([o.param for o in outs]), np.stack([o.momentum for o in outs]),
            np.stack([o.ortho for o in outs]), outs[0].route if outs else None)

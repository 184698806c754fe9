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

Each step below is the pages' definition written out in float64 with numpy.
The only library primitive is the matrix product.  Pins: tests/test_oracle_muon.py.
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


def newton_schulz(G: np.ndarray, steps: int = 5, coeffs=QUINTIC, eps: float = 1e-7) -> np.ndarray:
    """Approximate orthogonal polar factor of G by the quintic Newton-Schulz iteration.

    [HB] newton_schulz listing, in its order:
      1. X = G / (||G||_F + eps)            (spectral norm <= 1)
      2. transpose when rows > cols         (smaller Gram side)
      3. repeat: R = X X^T;  X = a X + (b R + c R R) X
      4. transpose back
    ``coeffs`` is one (a, b, c) triple or a per-iteration (steps, 3) table.
    """
    X = np.array(G, dtype=np.float64, copy=True)
    if X.ndim != 2:
        raise ValueError("newton_schulz takes one 2-D matrix")
    X = X / (np.linalg.norm(X) + eps)
    transposed = X.shape[0] > X.shape[1]
    if transposed:
        X = X.T
    for a, b, c in _coeff_table(coeffs, steps):
        R = X @ X.T
        X = a * X + (b * R + c * (R @ R)) @ X
    return X.T if transposed else X


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

    [HB] update steps and Muon listing:
      1. M <- mu M + G                              (sum-form momentum, M starts at 0)
      2. U <- G + mu M  (Nesterov, new M)   or  U <- M
      3. O <- newton_schulz(U)
      4. P <- P (1 - lr wd)                         (decoupled decay, old P)
      5. P <- P - lr * s * O,   s = update_scale(A, B)
    [DM] cautious weight decay: the decay of step 4 applies only where the
    update u = s O and the old parameter have the same sign (u * p > 0).
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

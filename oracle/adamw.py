"""fp64 CPU oracle of the AdamW step (and of Adam with coupled L2 decay).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.

Sources (page titles as published):

* [HB] "Optimizers: AdamW, Muon and the distributed optimizer" (AI infra
  handbook), section "AdamW: decoupled weight decay": first and second moments,
  update m / (sqrt(v) + eps); decoupled decay w <- w - lr*wd*w applied to the
  weights directly, versus L2 decay added to the gradient before the
  normalisation.  The section's decay experiment runs torch.optim.AdamW /
  torch.optim.Adam, i.e. bias-corrected moments; the experiment's printed
  values pin that reading (tests/golden/adamw_decay_experiment.txt).
* [DM] "dtensor-muon" package description, "Key options": is_adamw (decoupled
  vs coupled decay) and cautious weight decay (decay only where update and
  parameter share a sign).

Element by element, float64, in the order of the definition.  Pins:
tests/test_oracle_adamw.py.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class AdamWResult:
    param: np.ndarray
    exp_avg: np.ndarray
    exp_avg_sq: np.ndarray


def adamw_step(param, grad, exp_avg, exp_avg_sq, *, step: int, lr: float, beta1: float = 0.9,
               beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
               decoupled: bool = True, cautious_wd: bool = False) -> AdamWResult:
    """One Adam(W) step at step number ``step`` (t >= 1), float64.

      decoupled:  decay the weights directly, w <- w (1 - lr wd)        [HB]
      coupled:    add wd * w to the gradient first (Adam + L2)           [HB]
      m <- b1 m + (1 - b1) g
      v <- b2 v + (1 - b2) g^2
      w <- w - lr * mhat / (sqrt(vhat) + eps),  mhat = m / (1 - b1^t),  vhat = v / (1 - b2^t)
    Cautious decay [DM] (decoupled only): the decay applies only where the
    update mhat / (sqrt(vhat) + eps) and the old weight have the same sign.
    """
    if step < 1:
        raise ValueError("step counts from 1")
    w = np.asarray(param, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64)
    m = np.asarray(exp_avg, dtype=np.float64)
    v = np.asarray(exp_avg_sq, dtype=np.float64)
    if not decoupled:
        g = g + weight_decay * w
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    upd = mhat / (np.sqrt(vhat) + eps)
    if decoupled:
        if cautious_wd:
            w = w * (1.0 - np.where(upd * w > 0, lr * weight_decay, 0.0))
        else:
            w = w * (1.0 - lr * weight_decay)
    w = w - lr * upd
    return AdamWResult(param=w, exp_avg=m, exp_avg_sq=v)

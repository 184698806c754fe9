"""Shared helpers of the GPU parity tests: tolerances and error measures.

The GPU receives fp32 hyperparameters through the C ABI; the oracle is given those
same fp32 values (in float64) so both compute the same function.

AdamW ("within 1e-6 relative"): each updated state element is compared with the
oracle's step from the same previous state, relative to the magnitude of the terms
that form it (|p| + lr |update| for the weight, b1 |m| + (1 - b1) |g| for the first
moment, the second moment itself).  That is the componentwise bound fp32 arithmetic
can keep; a plain |ref| denominator is meaningless where terms cancel to ~0.

Muon ("bf16 updates within 2e-2 relative Frobenius"): per matrix, the update
P_{t-1}(1 - lr wd) - P_t against the oracle's.  Degenerate Gram sides (m < 16, e.g.
a single row) get the bound bf16 arithmetic can keep, since nothing averages out
over singular values when there are only a few: each iteration rounds X, R and P
(3 x 2^-9 relative), and along the orbit of a singular value that starts at 1
(1 -> 0.701 -> 1.114 -> 0.721 -> ...) the quintic's slope |p'| stays below 1.3, so
5 iterations stay below 3 * 2^-9 * (1 + 1.3 + ... + 1.3^4) ~ 5.3e-2, rounded up to
6e-2.
"""
import numpy as np

ADAMW_RTOL = 1e-6
MUON_RTOL = 2e-2
MUON_RTOL_DEGENERATE = 6e-2
DEGENERATE_M = 16
MOMENTUM_RTOL = 1e-6


def f32(x):
    return float(np.float32(x))


def muon_rtol(A, B):
    return MUON_RTOL if min(A, B) >= DEGENERATE_M else MUON_RTOL_DEGENERATE


def rel_err_floor(got, ref):
    """max |got - ref| / (|ref| + RMS(ref))."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + rms)))


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref))
    return float(np.linalg.norm(got - ref)) / den if den > 0 else float(np.linalg.norm(got))


def adamw_term_scales(p, g, m, v, *, step, lr, beta1, beta2, eps, weight_decay,
                      decoupled=True, cautious_wd=False):
    """Magnitudes of the terms forming the updated (param, exp_avg, exp_avg_sq) and of
    the update itself, element by element, in float64."""
    p, g, m, v = (np.asarray(x, dtype=np.float64) for x in (p, g, m, v))
    if decoupled:
        ge, gs = g, np.abs(g)
    else:
        ge, gs = g + weight_decay * p, np.abs(g) + weight_decay * np.abs(p)
    sm = beta1 * np.abs(m) + (1 - beta1) * gs
    sv = beta2 * v + (1 - beta2) * ge * ge
    vhat = sv / (1 - beta2 ** step)
    su = (sm / (1 - beta1 ** step)) / (np.sqrt(vhat) + eps)
    sp = np.abs(p) + lr * su
    return sp, sm, sv, su


def muon_recover(prev, got, lr, wd, scale):
    """Recover the GPU's cautious-decay mask and its orthogonalised matrix O from
    one step: got = prev (1 - lr wd [mask]) - lr s O with mask = (O prev > 0).
    With O_dec = (prev (1 - lr wd) - got) / (lr s) and O_plain = (prev - got) / (lr s),
    O_dec prev = O_plain prev - (wd / s) prev^2, so exactly one of "mask and
    O_dec prev > 0" or "no mask and O_plain prev <= 0" holds."""
    o_dec = (prev * (1 - lr * wd) - got) / (lr * scale)
    o_plain = (prev - got) / (lr * scale)
    mask = o_dec * prev > 0
    return mask, np.where(mask, o_dec, o_plain)

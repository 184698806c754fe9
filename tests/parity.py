"""Shared helpers of the GPU parity tests: tolerance checks and hyperparameter
rounding.  The GPU receives fp32 hyperparameters through the C ABI; the oracle is
given those same fp32 values (in float64) so both compute the same function."""
import numpy as np

# AdamW fp32 state: within 1e-6 relative, measured against |ref| + RMS(ref) so that
# entries that cancel to near zero are judged on the tensor's own scale.
ADAMW_RTOL = 1e-6
# Muon: bf16 Newton-Schulz updates within 2e-2 relative Frobenius error.
MUON_RTOL = 2e-2
# Muon momentum is fp32 elementwise work: same bar as the AdamW state.
MOMENTUM_RTOL = 1e-6


def f32(x):
    return float(np.float32(x))


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

"""Seeded synthetic inputs (parameters and gradients) for the workloads.

This module holds input generation only: none of the optimizer's arithmetic.
Every tensor is drawn from its own stream keyed by (seed, step, tensor index,
stream id), so any subset can be regenerated on its own:

* parameters at t = 0:   key (seed, 0, idx, 0), N(0, 1) fp32
* gradient of step t>=1: key (seed, t, idx, 1), recipe below, fp32

Tensor indices: Muon matrices are numbered first, bucket by bucket and matrix
by matrix inside a bucket; the AdamW tensors follow.

Two backends draw from the same recipes:

* ``numpy`` (``numpy.random.default_rng``): the inputs of every oracle
  comparison; generated on the host, uploaded for the GPU path.
* ``torch`` on a device (``torch.Generator``): the same distributions, other
  values; used where only timing matters or where the oracle reads back the
  generated inputs (large workloads).

Gradient recipes (sigma0: the workload's muon_sigma for Muon matrices, 0.02 unless the
workload states otherwise, and adamw_sigma, 1e-3, for AdamW tensors):

* ``gauss``:        sigma0 * z
* ``rowlognormal``: sigma0 * z * exp(xi_row), xi ~ N(0, 1) per row (1-D: gauss)
* ``lowrank``:      sigma0 * z plus a rank-8 product of Gaussians rescaled to
                    hold 30 % of the energy (1-D: gauss)
* ``conditioned``:  diag(exp(s*rho)) (sigma0 * z) diag(exp(s*gamma)),
                    rho, gamma ~ N(0, 1), s = 1.2: log-normal row and column
                    scales whose spread gives a condition number near 1e4
                    (calibrated on a 1024 x 3584 replica of the 8192 x 28672
                    shape; tests/test_workloads.py) (1-D: gauss)
"""
from __future__ import annotations

import hashlib
import math
from typing import Iterator, Tuple

import numpy as np

from .configs import Workload

MUON_SIGMA = 0.02
ADAMW_SIGMA = 1e-3
LOWRANK_RANK = 8
LOWRANK_ENERGY = 0.30
COND_SIGMA = 1.2

STREAM_PARAM = 0
STREAM_GRAD = 1


# --------------------------------------------------------------------------
# tensor bookkeeping
# --------------------------------------------------------------------------
def muon_index(wl: Workload, bucket: int, k: int) -> int:
    return sum(b.K for b in wl.muon[:bucket]) + k


def adamw_index(wl: Workload, j: int) -> int:
    return wl.n_matrices + j


def adamw_offsets(wl: Workload) -> Iterator[Tuple[int, int, int]]:
    """(tensor j, start, stop) of each AdamW tensor inside the flat buffer."""
    off = 0
    for j, t in enumerate(wl.adamw):
        yield j, off, off + t.numel
        off += t.numel


# --------------------------------------------------------------------------
# numpy backend
# --------------------------------------------------------------------------
def _np_rng(seed: int, step: int, idx: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, step, idx, stream])


def _np_recipe(g: np.random.Generator, recipe: str, shape, sigma0: float) -> np.ndarray:
    z = g.standard_normal(shape, dtype=np.float32)
    if recipe == "gauss" or len(shape) != 2:
        return (sigma0 * z).astype(np.float32)
    rows, cols = shape
    if recipe == "rowlognormal":
        xi = g.standard_normal((rows, 1), dtype=np.float32)
        return (sigma0 * z * np.exp(xi)).astype(np.float32)
    if recipe == "lowrank":
        noise = sigma0 * z.astype(np.float64)
        left = g.standard_normal((rows, LOWRANK_RANK))
        right = g.standard_normal((LOWRANK_RANK, cols))
        low = left @ right
        target = LOWRANK_ENERGY / (1.0 - LOWRANK_ENERGY) * float(np.sum(noise * noise))
        low *= math.sqrt(target / float(np.sum(low * low)))
        return (noise + low).astype(np.float32)
    if recipe == "conditioned":
        rho = g.standard_normal(rows)
        gam = g.standard_normal(cols)
        dr = np.exp(COND_SIGMA * rho).astype(np.float32)[:, None]
        dc = np.exp(COND_SIGMA * gam).astype(np.float32)[None, :]
        return (dr * (sigma0 * z) * dc).astype(np.float32)
    raise ValueError(f"unknown gradient recipe {recipe!r}")


def np_param(seed: int, idx: int, shape) -> np.ndarray:
    return _np_rng(seed, 0, idx, STREAM_PARAM).standard_normal(shape, dtype=np.float32)


def np_grad(seed: int, step: int, idx: int, shape, recipe: str, sigma0: float) -> np.ndarray:
    if step < 1:
        raise ValueError("gradients are drawn for steps t >= 1")
    return _np_recipe(_np_rng(seed, step, idx, STREAM_GRAD), recipe, shape, sigma0)


def np_muon_bucket_params(wl: Workload, bucket: int) -> np.ndarray:
    b = wl.muon[bucket]
    out = np.empty((b.K, b.A, b.B), dtype=np.float32)
    for k in range(b.K):
        out[k] = np_param(wl.seed, muon_index(wl, bucket, k), (b.A, b.B))
    return out


def np_muon_bucket_grads(wl: Workload, bucket: int, step: int) -> np.ndarray:
    b = wl.muon[bucket]
    out = np.empty((b.K, b.A, b.B), dtype=np.float32)
    for k in range(b.K):
        out[k] = np_grad(wl.seed, step, muon_index(wl, bucket, k), (b.A, b.B),
                         wl.muon_grad, wl.muon_sigma)
    return out


def np_adamw_flat_params(wl: Workload) -> np.ndarray:
    out = np.empty(wl.adamw_numel, dtype=np.float32)
    for j, lo, hi in adamw_offsets(wl):
        out[lo:hi] = np_param(wl.seed, adamw_index(wl, j), wl.adamw[j].shape).reshape(-1)
    return out


def np_adamw_flat_grads(wl: Workload, step: int) -> np.ndarray:
    out = np.empty(wl.adamw_numel, dtype=np.float32)
    for j, lo, hi in adamw_offsets(wl):
        out[lo:hi] = np_grad(wl.seed, step, adamw_index(wl, j), wl.adamw[j].shape,
                             wl.adamw_grad, wl.adamw_sigma).reshape(-1)
    return out


# --------------------------------------------------------------------------
# torch backend (device-side generation of the same distributions)
# --------------------------------------------------------------------------
def _torch_seed(seed: int, step: int, idx: int, stream: int) -> int:
    h = hashlib.blake2b(f"{seed}/{step}/{idx}/{stream}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _torch_recipe(torch, gen, recipe: str, shape, sigma0: float, out):
    """Fill ``out`` (fp32, ``shape``) in place from ``recipe``."""
    out.normal_(0.0, 1.0, generator=gen)
    out.mul_(sigma0)
    if recipe == "gauss" or len(shape) != 2:
        return out
    rows, cols = shape
    dev = out.device
    if recipe == "rowlognormal":
        xi = torch.randn((rows, 1), generator=gen, device=dev, dtype=torch.float32)
        out.mul_(xi.exp_())
        return out
    if recipe == "lowrank":
        left = torch.randn((rows, LOWRANK_RANK), generator=gen, device=dev, dtype=torch.float32)
        right = torch.randn((LOWRANK_RANK, cols), generator=gen, device=dev, dtype=torch.float32)
        low = left @ right
        noise_e = float(out.double().square().sum())
        low_e = float(low.double().square().sum())
        target = LOWRANK_ENERGY / (1.0 - LOWRANK_ENERGY) * noise_e
        out.add_(low, alpha=math.sqrt(target / low_e))
        return out
    if recipe == "conditioned":
        rho = torch.randn(rows, generator=gen, device=dev, dtype=torch.float32)
        gam = torch.randn(cols, generator=gen, device=dev, dtype=torch.float32)
        out.mul_(torch.exp(COND_SIGMA * rho)[:, None])
        out.mul_(torch.exp(COND_SIGMA * gam)[None, :])
        return out
    raise ValueError(f"unknown gradient recipe {recipe!r}")


def torch_fill_param(torch, out, seed: int, idx: int):
    gen = torch.Generator(device=out.device)
    gen.manual_seed(_torch_seed(seed, 0, idx, STREAM_PARAM))
    return out.normal_(0.0, 1.0, generator=gen)


def torch_fill_grad(torch, out, seed: int, step: int, idx: int, recipe: str, sigma0: float):
    if step < 1:
        raise ValueError("gradients are drawn for steps t >= 1")
    gen = torch.Generator(device=out.device)
    gen.manual_seed(_torch_seed(seed, step, idx, STREAM_GRAD))
    return _torch_recipe(torch, gen, recipe, tuple(out.shape), sigma0, out)


def torch_muon_bucket(torch, wl: Workload, bucket: int, step: int, out):
    """Fill a (K, A, B) tensor: parameters when step == 0, else gradients."""
    for k in range(out.shape[0]):
        idx = muon_index(wl, bucket, k)
        if step == 0:
            torch_fill_param(torch, out[k], wl.seed, idx)
        else:
            torch_fill_grad(torch, out[k], wl.seed, step, idx, wl.muon_grad, wl.muon_sigma)
    return out


def torch_adamw_flat(torch, wl: Workload, step: int, out):
    """Fill the flat AdamW buffer: parameters when step == 0, else gradients."""
    for j, lo, hi in adamw_offsets(wl):
        view = out[lo:hi].view(wl.adamw[j].shape)
        idx = adamw_index(wl, j)
        if step == 0:
            torch_fill_param(torch, view, wl.seed, idx)
        else:
            torch_fill_grad(torch, view, wl.seed, step, idx, wl.adamw_grad, wl.adamw_sigma)
    return out

"""The Gram-space Newton-Schulz iteration (ns_mode 1; "DMuon: Efficient Distributed Muon
Training with Near-Adam Overhead", section 2.2) through the C ABI against the fp64
oracle of the printed iteration, at the same tolerance.  It applies to buckets with
n >= 2 m; its bf16 error grows with the spread of the singular values, so it is checked
on Gaussian and low-rank gradients of both orientations and on row log-normal ones of
wide matrices; on tall row-scaled and on conditioned gradients it does not hold the
tolerance (measured band pinned below).  The kernel's Gram-space results match a CPU bf16
emulation of the same rounding scheme to three digits."""
import numpy as np
import pytest

import oracle
from parity import MUON_RTOL, muon_rtol, rel_fro
from test_gpu_muon import LR, MU, WD, _buckets, _check_muon, _grad, _muon_run

torch = pytest.importorskip("torch")
ma = pytest.importorskip("adamw_optimizer_step_muon_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


WIDE = [(64, 128), (100, 333), (256, 1024), (1, 7), (130, 1000)]
TALL = [(128, 64), (333, 100), (1024, 256)]


@pytest.mark.parametrize("shape,recipe", [(s, r) for s in WIDE + TALL for r in ("gauss", "lowrank")]
                         + [(s, "rowlognormal") for s in WIDE])
def test_gram_space_newton_schulz_parity(shape, recipe):
    K = 3
    G = np.stack([_grad(shape, 20 + k, recipe) for k in range(K)])
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5, ns_mode=1)
    torch.cuda.synchronize()
    out = go.cpu().numpy()
    for k in range(K):
        err = rel_fro(out[k], oracle.newton_schulz(G[k], 5))
        assert err <= muon_rtol(*shape), (shape, recipe, k, err)


@pytest.mark.parametrize("shape", TALL)
def test_gram_space_error_band_on_tall_row_scaled_gradients(shape):
    """Where the Gram-space route does not hold the tolerance: tall matrices with
    log-normal row scales (after the transpose, scales on the long side).  A CPU bf16
    emulation of the same rounding scheme gives 2.3e-2 to 4.4e-2 on these inputs, the
    printed iteration's bf16 path about 1e-2; the kernel must land in that band (not
    better by accident of a skipped step, not worse by a defect)."""
    G = _grad(shape, 20, "rowlognormal")[None]
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5, ns_mode=1)
    torch.cuda.synchronize()
    err = rel_fro(go.cpu().numpy()[0], oracle.newton_schulz(G[0], 5))
    assert 1.5e-2 < err < 6e-2, err


@pytest.mark.parametrize("steps,coeffs", [(1, None), (2, None), (3, [(3.4445, -4.7750, 2.0315),
                                                                       (2.0, -1.5, 0.5),
                                                                       (1.5, -0.5, 0.0)]),
                                          (4, (1.5, -0.5, 0.0)), (0, None)])
def test_gram_space_step_counts_and_tables(steps, coeffs):
    """One step (only the polynomial and the final product), two (one Q product),
    a per-iteration table, the cubic, and no step at all (normalisation only)."""
    G = _grad((200, 520), 5)[None]
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=steps, ns_coeffs=coeffs, ns_mode=1)
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(G[0], steps, oracle.muon.QUINTIC if coeffs is None
                               else np.array(coeffs, dtype=np.float64))
    assert rel_fro(go.cpu().numpy()[0], ref) <= MUON_RTOL


def test_gram_space_muon_steps_mixed_buckets():
    """A Muon step list where only the 2:1 buckets take the Gram-space route: routes
    report it, every matrix matches the oracle over two steps, and the square bucket is
    bitwise the same as without ns_mode."""
    shapes = [(4, 256, 768), (3, 600, 200), (5, 192, 192)]
    P0, grads = _buckets(shapes, 31, 2, recipe="lowrank")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [r.ns_mode_run for r in routes] == [1, 1, 0]
    _check_muon(P0, grads, hist, routes)
    hist0, routes0 = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    assert [r.ns_mode_run for r in routes0] == [0, 0, 0]
    assert np.array_equal(hist[-1][2][0], hist0[-1][2][0])


def test_gram_space_full_size_mlp_buckets():
    """The 12-layer GPT's MLP buckets (768 x 3072 and its transpose, 12 each) at full
    size through the Gram-space route: first and last matrix of each bucket against the
    oracle over two steps, on the workload's low-rank gradient recipe."""
    shapes = [(12, 768, 3072), (12, 3072, 768)]
    P0, grads = _buckets(shapes, 41, 2, recipe="lowrank")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [r.ns_mode_run for r in routes] == [1, 1]
    _check_muon(P0, grads, hist, routes, only=[[0, 11], [0, 11]])


def test_gram_space_bucket_that_keeps_xt():
    """Gram sides above 2048 on 256-tiles keep X^T, so the final product reads X_0^T:
    both orientations (6 x 2560 x 5120 and its transpose, one phase), first matrix of each
    against the oracle for one step on Gaussian gradients (at this Gram side the route's
    error on low-rank gradients is 3.8e-2, bit for bit what a CPU bf16 emulation of the
    same scheme gives: outside the tolerance, so not a parity case)."""
    shapes = [(6, 2560, 5120), (6, 5120, 2560)]
    assert ma.muon_phases(shapes, ns_mode=1) == (1, [0, 0])
    P0, grads = _buckets(shapes, 51, 1, recipe="gauss")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [(r.ns_mode_run, r.m_pad) for r in routes] == [(1, 2560), (1, 2560)]
    _check_muon(P0, grads, hist, routes, only=[[0], [0]])

"""The Gram-space Newton-Schulz iteration (ns_mode 1; "DMuon: Efficient Distributed Muon
Training with Near-Adam Overhead", section 2.2) through the C ABI against the fp64
oracle, at the Muon tolerance.  The library takes it for wide buckets (A < B) with
B >= 2 A and A <= 1024, where its bf16 error was measured inside the tolerance on
Gaussian, low-rank and row log-normal gradients; tall buckets (whose row-scaled
gradients left the tolerance at every Gram side: 2.3e-2 to 5e-2) and wider Gram sides
(low-rank gradients: 2.2e-2 at 1536, 3.0e-2 at 2048, 3.8e-2 at 2560) keep the printed
iteration, which the routing report states and the tests below check along with
parity.  Inside the domain the route still misses the tolerance on gradients with a
condition number near 1e4 (6.5e-2 to 1.5e-1 in a CPU bf16 emulation of the kernel's
rounding scheme, which matches the kernel to three digits): a strict expected failure
below records it.  The route is opt-in for well-conditioned gradients."""
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


@pytest.mark.parametrize("shape,recipe", [(s, r) for s in WIDE + TALL
                                           for r in ("gauss", "lowrank", "rowlognormal")])
def test_gram_space_newton_schulz_parity(shape, recipe):
    """Wide shapes run the Gram-space route, tall ones (row-scaled included, where the
    route would miss the tolerance) the printed iteration: all within the tolerance."""
    K = 3
    route = ma.muon_route_of(*shape, 5, ns_mode=1)
    assert route.ns_mode_run == (1 if shape[0] < shape[1] else 0)
    G = np.stack([_grad(shape, 20 + k, recipe) for k in range(K)])
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5, ns_mode=1)
    torch.cuda.synchronize()
    out = go.cpu().numpy()
    for k in range(K):
        err = rel_fro(out[k], oracle.newton_schulz(G[k], 5))
        assert err <= muon_rtol(*shape), (shape, recipe, k, err)


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
    """A Muon step list where only the wide 2:1 bucket takes the Gram-space route: routes
    report it, every matrix matches the oracle over two steps, and the square bucket is
    bitwise the same as without ns_mode."""
    shapes = [(4, 256, 768), (3, 600, 200), (5, 192, 192)]
    P0, grads = _buckets(shapes, 31, 2, recipe="lowrank")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [r.ns_mode_run for r in routes] == [1, 0, 0]
    _check_muon(P0, grads, hist, routes)
    hist0, routes0 = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    assert [r.ns_mode_run for r in routes0] == [0, 0, 0]
    assert np.array_equal(hist[-1][2][0], hist0[-1][2][0])


def test_gram_space_full_size_mlp_buckets():
    """The 12-layer GPT's MLP buckets (768 x 3072 and its transpose, 12 each) at full
    size under ns_mode 1 (the up projection through the Gram-space route, the down
    projection through the printed iteration): first and last matrix of each bucket
    against the oracle over two steps, on the workload's low-rank gradient recipe."""
    shapes = [(12, 768, 3072), (12, 3072, 768)]
    P0, grads = _buckets(shapes, 41, 2, recipe="lowrank")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [r.ns_mode_run for r in routes] == [1, 0]
    _check_muon(P0, grads, hist, routes, only=[[0, 11], [0, 11]])


@pytest.mark.parametrize("recipe", ["rowlognormal", "lowrank", "gauss"])
def test_gram_space_largest_gram_side(recipe):
    """The largest Gram side the route takes, 1024 (2 x 1024 x 2048), on row-scaled,
    low-rank and Gaussian gradients: first and last matrix over two steps."""
    shapes = [(2, 1024, 2048)]
    P0, grads = _buckets(shapes, 53, 2, recipe=recipe)
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [r.ns_mode_run for r in routes] == [1]
    _check_muon(P0, grads, hist, routes, only=[[0, 1]])


@pytest.mark.xfail(strict=True, reason="Gram-space route on gradients with condition number "
                   "~1e4: bf16 R loses the small squared singular values (emulated 6.5e-2 to "
                   "1.5e-1 against the 2e-2 tolerance); opt-in for well-conditioned inputs")
@pytest.mark.parametrize("shape", [(512, 1024), (1024, 2048)])
def test_gram_space_misses_tolerance_on_conditioned_gradients(shape):
    G = _grad(shape, 20, "conditioned")[None]
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5, ns_mode=1)
    torch.cuda.synchronize()
    assert rel_fro(go.cpu().numpy()[0], oracle.newton_schulz(G[0], 5)) <= MUON_RTOL


def test_gram_space_declined_outside_its_domain():
    """Gram sides above 1024 (6 x 2560 x 5120, which keeps X^T, and its transpose) are
    outside the route's domain: on the low-rank gradients where the route measured
    3.8e-2 they run the printed iteration and meet the tolerance (first and last
    matrix, two steps)."""
    shapes = [(6, 2560, 5120), (6, 5120, 2560)]
    assert ma.muon_phases(shapes, ns_mode=1) == (1, [0, 0])
    P0, grads = _buckets(shapes, 51, 2, recipe="lowrank")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [(r.ns_mode_run, r.m_pad) for r in routes] == [(0, 2560), (0, 2560)]
    _check_muon(P0, grads, hist, routes, only=[[0, 5], [0, 5]])

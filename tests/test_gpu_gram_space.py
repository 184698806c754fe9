"""The Gram-space Newton-Schulz iteration (ns_mode 1; "DMuon: Efficient Distributed Muon
Training with Near-Adam Overhead", section 2.2) through the C ABI against the fp64
oracle of the printed iteration, at the Muon tolerance.

The route runs on fp16 operands (X0, R, P, Q and R P scaled by powers of two into fp16's
range; fp32 accumulation; the result in bf16) and the library takes it for buckets whose
long side is at least 3.5 times the Gram side, in either orientation and at any Gram
side.  A CPU emulation of that rounding scheme (which reproduces the kernel's error to
two digits) put its error at 2-7e-3 on Gaussian, low-rank, row-scaled and conditioned
gradients at the workloads' sizes up to 8192 x 28672, below the printed iteration's bf16
error on the same inputs (7-10e-3), and at most 1.3e-2 on conditioned gradients with Gram
sides of 64 to 512 over many seeds; at 3:1 those reached 2.0-2.5e-2, so squarer buckets
keep the printed iteration, which the routing report states and the tests below
check."""
import numpy as np
import pytest

import oracle
from parity import MUON_RTOL, muon_rtol, rel_fro
from test_gpu_muon import LR, MU, WD, _buckets, _check_muon, _grad, _muon_run

torch = pytest.importorskip("torch")
ma = pytest.importorskip("adamw_optimizer_step_muon_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

RECIPES = ("gauss", "lowrank", "rowlognormal", "conditioned")
WIDE = [(64, 256), (100, 350), (256, 1024), (1, 7), (130, 1000), (286, 1001)]
TALL = [(256, 64), (350, 100), (1024, 256), (1000, 130)]


@pytest.mark.parametrize("shape,recipe", [(s, r) for s in WIDE + TALL for r in RECIPES])
def test_gram_space_newton_schulz_parity(shape, recipe):
    """Wide and tall shapes at 3.5:1 and beyond run the Gram-space route: every matrix
    within the tolerance of the oracle."""
    K = 3
    route = ma.muon_route_of(*shape, 5, ns_mode=1)
    assert route.ns_mode_run == 1
    G = np.stack([_grad(shape, 20 + k, recipe) for k in range(K)])
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5, ns_mode=1)
    torch.cuda.synchronize()
    out = go.cpu().numpy()
    for k in range(K):
        err = rel_fro(out[k], oracle.newton_schulz(G[k], 5))
        assert err <= muon_rtol(*shape), (shape, recipe, k, err)


@pytest.mark.parametrize("shape", [(512, 1024), (2048, 4096), (100, 250), (100, 349), (192, 64)])
def test_gram_space_declines_squarer_buckets(shape):
    """Below 3.5:1 the printed iteration runs, also under ns_mode 1."""
    assert ma.muon_route_of(*shape, 5, ns_mode=1).ns_mode_run == 0
    assert ma.muon_route_of(*shape[::-1], 5, ns_mode=1).ns_mode_run == 0


@pytest.mark.parametrize("steps,coeffs,route", [
    (1, None, 1), (2, None, 1),
    (3, [(3.4445, -4.7750, 2.0315), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)], 1),
    (4, (1.5, -0.5, 0.0), 1), (0, None, 0), (8, None, 1), (9, None, 0), (12, None, 0),
    (2, (40.0, -4.0, 0.1), 0)])
def test_gram_space_step_counts_and_tables(steps, coeffs, route):
    """One step (only the polynomial and the final product), two (one Q product), a
    per-iteration table, the cubic, no step at all (normalisation only), and the range
    bound: the quintic's Q grows as a^N on a zero singular value, which fp16 holds up to 8
    steps; from 9 steps, or with coefficients that leave fp16's range, the bucket runs
    the printed iteration (the routing report says which)."""
    assert ma.muon_route_of(200, 700, steps, ns_mode=1, ns_coeffs=coeffs).ns_mode_run == route
    G = _grad((200, 700), 5)[None]
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=steps, ns_coeffs=coeffs, ns_mode=1)
    torch.cuda.synchronize()
    out = go.cpu().numpy()[0]
    assert np.isfinite(out).all()
    if route == 0:
        # the printed iteration, bit for bit (whose own bf16 drift past 8 quintic steps is
        # the subject of the iteration-count tests, not of this one)
        g0 = torch.empty_like(gi)
        ma.newton_schulz(gi, g0, ns_steps=steps, ns_coeffs=coeffs, ns_mode=0)
        torch.cuda.synchronize()
        assert np.array_equal(out, g0.cpu().numpy()[0])
    if steps <= 8:
        ref = oracle.newton_schulz(G[0], steps, oracle.muon.QUINTIC if coeffs is None
                                   else np.array(coeffs, dtype=np.float64))
        assert rel_fro(out, ref) <= MUON_RTOL, rel_fro(out, ref)


def test_gram_space_muon_steps_mixed_buckets():
    """A Muon step list where the 4:1 buckets (wide and tall) take the Gram-space route
    and the square one the printed iteration: routes report it, every matrix matches the
    oracle over two steps, and the square bucket is bitwise the same as without
    ns_mode."""
    shapes = [(4, 256, 1024), (3, 800, 200), (5, 192, 192)]
    P0, grads = _buckets(shapes, 31, 2, recipe="lowrank")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [r.ns_mode_run for r in routes] == [1, 1, 0]
    _check_muon(P0, grads, hist, routes)
    hist0, routes0 = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    assert [r.ns_mode_run for r in routes0] == [0, 0, 0]
    assert np.array_equal(hist[-1][2][0], hist0[-1][2][0])


def test_gram_space_full_size_mlp_buckets():
    """The 12-layer GPT's MLP buckets (768 x 3072 and its transpose, 12 each) at full
    size under ns_mode 1, both through the Gram-space route (one shared phase): first and
    last matrix of each bucket against the oracle over two steps, on the workload's
    low-rank gradient recipe."""
    shapes = [(12, 768, 3072), (12, 3072, 768)]
    assert ma.muon_phases(shapes, ns_mode=1) == (1, [0, 0])
    P0, grads = _buckets(shapes, 41, 2, recipe="lowrank")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [r.ns_mode_run for r in routes] == [1, 1]
    _check_muon(P0, grads, hist, routes, only=[[0, 11], [0, 11]])


@pytest.mark.parametrize("recipe", ["conditioned", "rowlognormal", "lowrank"])
def test_gram_space_keeps_xt_buckets(recipe):
    """Gram sides above 2048 keep X^T (the last product reads the stored fp16 X0^T):
    2 x 2304 x 8064 and its transpose, first and last matrix over two steps."""
    shapes = [(2, 2304, 8064), (2, 8064, 2304)]
    P0, grads = _buckets(shapes, 53, 2, recipe=recipe)
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [(r.ns_mode_run, r.m_pad) for r in routes] == [(1, 2304), (1, 2304)]
    _check_muon(P0, grads, hist, routes, only=[[0, 1], [0, 1]])


def test_gram_space_declined_outside_its_domain():
    """2:1 buckets (6 x 2560 x 5120, which keeps X^T, and its transpose) run the printed
    iteration under ns_mode 1 and meet the tolerance (first and last matrix, two
    steps)."""
    shapes = [(6, 2560, 5120), (6, 5120, 2560)]
    assert ma.muon_phases(shapes, ns_mode=1) == (1, [0, 0])
    P0, grads = _buckets(shapes, 51, 2, recipe="lowrank")
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_mode=1)
    assert [(r.ns_mode_run, r.m_pad) for r in routes] == [(0, 2560), (0, 2560)]
    _check_muon(P0, grads, hist, routes, only=[[0, 5], [0, 5]])


@pytest.mark.parametrize("scale,eps", [(1e-20, 0.0), (1e-6, 0.0), (1.0, 0.0), (1e6, 0.0),
                                       (1e18, 0.0), (1e18, 1e-7), (1e-8, 1e-7), (1e-9, 1e-7),
                                       (1e-12, 1e-7), (1e-20, 1e-7)])
def test_gram_space_input_range(scale, eps):
    """Gradients far from unit scale.  With ns_eps = 0 the normalisation is exact at every
    scale; with 1e-7 and norms near or below eps, X0 = U / (||U|| + eps) is itself small
    (down to ~1e-13 here) and the fp16 copy is scaled up per matrix by the power of two
    that brings ||X0|| back to [1/2, 1), so it neither flushes to zero nor loses digits;
    the products then see the true, small X0 (the quintic acts as a^5 on it).  Each case
    against the oracle at the same scale and eps."""
    G = (_grad((96, 384), 9, "rowlognormal").astype(np.float64) * scale).astype(np.float32)[None]
    assert np.all(np.isfinite(G))
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5, ns_eps=eps, ns_mode=1)
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(G[0], 5, eps=eps)
    err = rel_fro(go.cpu().numpy()[0], ref)
    assert err <= MUON_RTOL, (scale, eps, err)


def test_optimizer_group_takes_the_gram_space_route():
    """MuonAdamW with ns_mode 1 in its group, over a model's separate MLP matrices
    (768 x 3072 and 3072 x 768, 4:1) and attention matrices (768 x 768): the MLP buckets
    run the Gram-space route in one phase, the square one the printed iteration; two
    steps bit for bit the stacked ma_muon_step with ns_mode 1."""
    shapes = [(768, 768), (768, 3072), (3072, 768)]
    gen_ = torch.Generator(device=DEV).manual_seed(5)
    params = [torch.nn.Parameter(torch.randn(s, generator=gen_, device=DEV))
              for _ in range(4) for s in shapes]
    grads = [[0.02 * torch.randn(p.shape, generator=gen_, device=DEV) for p in params]
             for _ in range(2)]
    stacks = [torch.stack([p.detach().clone() for p in params if tuple(p.shape) == s])
              for s in shapes]
    opt = ma.MuonAdamW([{"params": params, "kind": "muon", "lr": LR, "momentum": MU,
                         "weight_decay": WD, "ns_mode": 1}])
    assert opt.muon_buckets() == [(4, 768, 768), (4, 768, 3072), (4, 3072, 768)]
    assert ma.muon_phases(opt.muon_buckets(), ns_mode=1) == (2, [0, 1, 1])
    moms = [torch.zeros_like(s) for s in stacks]
    for t in range(2):
        for p, g in zip(params, grads[t]):
            p.grad = g.clone()
        opt.step()
        gst = [torch.stack([g for p, g in zip(params, grads[t]) if tuple(p.shape) == s])
               for s in shapes]
        routes = ma.muon_step(list(zip(stacks, gst, moms)), lr=LR, momentum=MU,
                              weight_decay=WD, ns_mode=1)
        assert [r.ns_mode_run for r in routes] == [0, 1, 1]
        torch.cuda.synchronize()
        for s, st in zip(shapes, stacks):
            mine = [p.detach() for p in params if tuple(p.shape) == s]
            assert all(torch.equal(a, b) for a, b in zip(mine, st)), (t, s)
        opt.zero_grad()


@pytest.mark.parametrize("index", [1, 2, 3])
def test_gram_space_full_size_workloads(index, capsys):
    """Each GPT workload at full size under ns_mode 1, in one ma_muon_step over all its
    buckets, for three steps: its 4:1 buckets (MLP up and down projections; the 24-layer
    model's 2048 x 512 key/value projections too) take the fp16 Gram-space route, the
    square ones the printed iteration; the first and last matrix of every Gram-space
    bucket against the oracle at every step, stepped from the GPU's previous parameters
    and the oracle's own momentum."""
    import workloads
    from test_gpu_muon import _oracle_check_step
    from workloads import gen

    wl = workloads.workload(index)
    hp = wl.muon_hp
    ps, gs, ms = [], [], []
    for bi, b in enumerate(wl.muon):
        p = torch.empty((b.K, b.A, b.B), dtype=torch.float32, device=DEV)
        gen.torch_muon_bucket(torch, wl, bi, 0, p)
        ps.append(p)
        gs.append(torch.empty_like(p))
        ms.append(torch.zeros_like(p))
    on_route = [2 * max(b.A, b.B) >= 7 * min(b.A, b.B) for b in wl.muon]
    picks = [(bi, k) for bi, b in enumerate(wl.muon) if on_route[bi] for k in sorted({0, b.K - 1})]
    prev = {pk: ps[pk[0]][pk[1]].cpu().numpy().astype(np.float64) for pk in picks}
    mom = {pk: np.zeros((wl.muon[pk[0]].A, wl.muon[pk[0]].B)) for pk in picks}
    worst = 0.0
    for t in range(1, 4):
        for bi in range(len(wl.muon)):
            gen.torch_muon_bucket(torch, wl, bi, t, gs[bi])
        grads = {pk: gs[pk[0]][pk[1]].cpu().numpy() for pk in picks}
        routes = ma.muon_step(list(zip(ps, gs, ms)), lr=hp.lr, momentum=hp.momentum,
                              weight_decay=hp.weight_decay, cautious_wd=hp.cautious_wd,
                              ns_mode=1)
        torch.cuda.synchronize()
        assert [r.ns_mode_run for r in routes] == [int(x) for x in on_route]
        for bi, k in picks:
            b = wl.muon[bi]
            got_p = ps[bi][k].cpu().numpy()
            mom[(bi, k)], err = _oracle_check_step(prev[(bi, k)], grads[(bi, k)], mom[(bi, k)],
                                                   got_p, ms[bi][k].cpu().numpy(), b.A, b.B, hp)
            prev[(bi, k)] = got_p.astype(np.float64)
            worst = max(worst, err)
        with capsys.disabled():
            print(f"gram-space workload {index} step {t}: worst update error {worst:.3e}",
                  flush=True)

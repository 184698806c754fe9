"""Muon and Newton-Schulz through the C ABI on the GPU against the fp64 oracle.

The Muon update of a step depends only on the gradients (through the momentum), not
on the parameters, except for the cautious mask; so each step's update is compared
on its own: update = P_{t-1} (1 - lr wd) - P_t (non-cautious), and for cautious
decay the oracle steps from the GPU's own P_{t-1}.
"""
import os

import numpy as np
import pytest

import oracle
import workloads
from parity import MOMENTUM_RTOL, MUON_RTOL, f32, muon_recover, muon_rtol, rel_err_floor, rel_fro
from workloads import gen

torch = pytest.importorskip("torch")
ma = pytest.importorskip("adamw_optimizer_step_muon_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MU, LR, WD = 0.95, 0.02, 0.1


def _grad(shape, seed, recipe="rowlognormal"):
    return gen.np_grad(seed, 1, 0, shape, recipe, gen.MUON_SIGMA)


# --------------------------------------------------------------------------
# Newton-Schulz alone
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shape", [(64, 128), (128, 64), (300, 520), (520, 300), (257, 257),
                                   (1, 5), (5, 1), (130, 1000), (768, 768)])
@pytest.mark.parametrize("recipe", ["gauss", "rowlognormal", "lowrank"])
def test_newton_schulz_parity(shape, recipe):
    K = 3
    G = np.stack([_grad(shape, 10 + k, recipe) for k in range(K)])
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5)
    torch.cuda.synchronize()
    out = go.cpu().numpy()
    for k in range(K):
        ref = oracle.newton_schulz(G[k], 5)
        err = rel_fro(out[k], ref)
        assert err <= muon_rtol(*shape), (shape, recipe, k, err)


@pytest.mark.parametrize("coeffs,steps", [((0.0, 1.0, 0.0), 1), ((0.0, 0.0, 1.0), 1),
                                          ((1.0, 0.0, 0.0), 3), ((3.4445, -4.7750, 2.0315), 0),
                                          ((1.5, -0.5, 0.0), 4)])
@pytest.mark.parametrize("shape", [(200, 330), (330, 200)])
def test_newton_schulz_term_probes(coeffs, steps, shape):
    """Isolate the Gram product (b), the polynomial's square (c), the a X term, the
    normalisation (0 steps) and a convergent cubic, each against the oracle."""
    G = _grad(shape, 3)[None]
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=steps, ns_coeffs=coeffs)
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(G[0], steps, coeffs)
    assert rel_fro(go.cpu().numpy()[0], ref) <= muon_rtol(*shape)


def test_newton_schulz_per_iteration_table():
    table = [(3.4445, -4.7750, 2.0315), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)]
    G = _grad((256, 384), 4)[None]
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=3, ns_coeffs=table)
    torch.cuda.synchronize()
    assert rel_fro(go.cpu().numpy()[0], oracle.newton_schulz(G[0], 3, np.array(table))) <= MUON_RTOL


def test_newton_schulz_printed_spectrum(golden):
    """The handbook's 256 x 1024 input with S = logspace(0, -2, 256): the bf16 kernel
    reproduces the printed singular-value range and in-band share after 5 steps."""
    g = golden("ns_spectrum.txt")
    rng = np.random.default_rng(0)
    U, _ = np.linalg.qr(rng.standard_normal((256, 256)))
    V, _ = np.linalg.qr(rng.standard_normal((1024, 256)))
    G = ((U * np.logspace(0, -2, 256)) @ V.T).astype(np.float32)[None]
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5)
    torch.cuda.synchronize()
    s = np.linalg.svd(go.cpu().numpy()[0].astype(np.float64), compute_uv=False)
    lo, hi = (float(v) for v in g["steps5_range"])
    assert abs(s.min() - lo) < 0.02 and abs(s.max() - hi) < 0.02
    frac = np.mean((s > 0.7) & (s < 1.2))
    assert abs(frac - float(g["steps5_in_band_pct"][0]) / 100) < 0.05


@pytest.mark.parametrize("scale", [1e-30, 1e-20, 1e-12, 1e12, 1e18, 1e30])
@pytest.mark.parametrize("shape", [(96, 200), (300, 130)])
def test_newton_schulz_input_range(scale, shape):
    """Gradients far from unit scale: the Frobenius norm is summed in float64 and a matrix
    whose norm lies outside [2^-32, 2^32] is rescaled by a power of two before its first
    product, so the fp32 Gram accumulation neither overflows (entries above ~1e17 would
    overflow an fp32 tile sum of squares, ~1e19 the Gram itself) nor drops its small
    terms (below ~1e-19 the squares leave fp32's normal range).  ns_eps = 0, so the
    normalisation is exactly U / ||U|| at every scale, as in the oracle."""
    G = (_grad(shape, 31).astype(np.float64) * scale).astype(np.float32)[None]
    assert np.all(np.isfinite(G))
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=5, ns_eps=0.0)
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(G[0], 5, eps=0.0)
    err = rel_fro(go.cpu().numpy()[0], ref)
    assert err <= MUON_RTOL, (scale, shape, err)


@pytest.mark.parametrize("scale,eps", [(1e18, 1e-7), (1e30, 1e-7), (1e-20, 0.0), (1e-30, 0.0)])
def test_muon_step_input_range(scale, eps):
    """The whole Muon step (momentum, norm, Newton-Schulz, update) on gradients 1e-30 to
    1e30: each step's update against the oracle over two steps (tiny gradients with
    ns_eps = 0: with 1e-7 the eps would dominate the norm and the update would vanish
    below fp32's resolution of the parameters, in the oracle as here)."""
    shapes = [(2, 96, 200), (2, 300, 130)]
    rng = np.random.default_rng(77)
    P0 = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    grads = [[np.stack([(gen.np_grad(77, t, 10 * i + k, s[1:], "rowlognormal", gen.MUON_SIGMA)
                         .astype(np.float64) * scale).astype(np.float32) for k in range(s[0])])
              for i, s in enumerate(shapes)] for t in (1, 2)]
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD, ns_eps=eps)
    ohp = dict(lr=f32(LR), mu=f32(MU), weight_decay=f32(WD), ns_eps=eps)
    for bi, p0 in enumerate(P0):
        for k in range(p0.shape[0]):
            prev, mom = p0[k].astype(np.float64), np.zeros(p0.shape[1:])
            for t in range(2):
                gp, gm = hist[t][bi][0][k], hist[t][bi][1][k]
                ref = oracle.muon_step(prev, grads[t][bi][k], mom, **ohp)
                assert rel_err_floor(gm, ref.momentum) <= MOMENTUM_RTOL, (scale, bi, k, t)
                keep = 1.0 - ohp["lr"] * ohp["weight_decay"]
                err = rel_fro(prev * keep - gp, prev * keep - ref.param)
                assert err <= MUON_RTOL, (scale, bi, k, t, err)
                prev, mom = gp.astype(np.float64), ref.momentum


# --------------------------------------------------------------------------
# Muon step
# --------------------------------------------------------------------------
def _muon_run(P0, grads, **hp):
    """GPU steps over a list of buckets; returns per step [(param, momentum)] and routes."""
    ps = [torch.from_numpy(p).to(DEV) for p in P0]
    ms = [torch.zeros_like(p) for p in ps]
    gs = [torch.empty_like(p) for p in ps]
    hist, routes = [], None
    for step_grads in grads:
        for g, gr in zip(gs, step_grads):
            g.copy_(torch.from_numpy(gr))
        routes = ma.muon_step(list(zip(ps, gs, ms)), **hp)
        torch.cuda.synchronize()
        hist.append([(p.cpu().numpy().copy(), m.cpu().numpy().copy()) for p, m in zip(ps, ms)])
    return hist, routes


AMBIGUOUS = 4 * 2.0 ** -8  # |O_ref| below this share of max|O_ref|: sign not decided in bf16


def cautious_check(prev, got, ref_ortho, lr, wd, scale, tol):
    """Cautious-decay step: recover the GPU's mask and orthogonalised matrix exactly
    from its result, then (1) its O against the oracle's within ``tol`` relative
    Frobenius, (2) its mask against the oracle's wherever |O_ref| is above
    AMBIGUOUS * max|O_ref| (below it the bf16 sign is not decided).  Returns
    (O error, share of decided entries whose mask differs)."""
    mask, o_gpu = muon_recover(prev, got, lr, wd, scale)
    err = rel_fro(o_gpu, ref_ortho)
    decided = np.abs(ref_ortho) > AMBIGUOUS * np.max(np.abs(ref_ortho))
    mask_ref = ref_ortho * prev > 0
    flips = float(np.mean((mask != mask_ref)[decided])) if np.any(decided) else 0.0
    return err, flips


def _check_muon(P0, grads, hist, routes, *, lr=LR, momentum=MU, weight_decay=WD,
                cautious_wd=False, nesterov=True, scale_mode=0, ns_steps=5, only=None):
    """Every matrix of every bucket against the oracle, step by step (``only``: a
    list of matrix indices per bucket to check instead of all)."""
    ohp = dict(lr=f32(lr), mu=f32(momentum), weight_decay=f32(weight_decay),
               cautious_wd=cautious_wd, nesterov=nesterov, scale_mode=scale_mode,
               ns_steps=ns_steps)
    worst = 0.0
    for bi, p0 in enumerate(P0):
        K, A, B = p0.shape
        r = routes[bi]
        o = oracle.route(A, B, ns_steps)
        assert (r.transposed, r.m, r.n, r.ns_steps_run) == (o.transposed, o.m, o.n, o.ns_steps)
        for k in (range(K) if only is None else only[bi]):
            prev = p0[k].astype(np.float64)
            mom = np.zeros((A, B))
            for t, step_grads in enumerate(grads):
                gp, gm = hist[t][bi][0][k], hist[t][bi][1][k]
                ref = oracle.muon_step(prev, step_grads[bi][k], mom, **ohp)
                assert rel_err_floor(gm, ref.momentum) <= MOMENTUM_RTOL, (bi, k, t)
                tol = muon_rtol(A, B)
                if cautious_wd:
                    err, flips = cautious_check(prev, gp.astype(np.float64), ref.ortho, ohp["lr"],
                                                ohp["weight_decay"],
                                                oracle.update_scale(A, B, scale_mode), tol)
                    assert flips == 0.0, (bi, k, t, flips)
                else:
                    keep = 1.0 - ohp["lr"] * ohp["weight_decay"]
                    err = rel_fro(prev * keep - gp, prev * keep - ref.param)
                worst = max(worst, err)
                assert err <= tol, (bi, k, t, err)
                prev, mom = gp.astype(np.float64), ref.momentum
    return worst


def _buckets(shapes, seed, steps, recipe="rowlognormal"):
    rng = np.random.default_rng(seed)
    P0 = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    grads = [[np.stack([gen.np_grad(seed, t, 1000 * i + k, s[1:], recipe, gen.MUON_SIGMA)
                        for k in range(s[0])]) for i, s in enumerate(shapes)]
             for t in range(1, steps + 1)]
    return P0, grads


def test_muon_tiny_workload_all_steps():
    wl = workloads.workload(0)
    P0 = [gen.np_muon_bucket_params(wl, i) for i in range(len(wl.muon))]
    grads = [[gen.np_muon_bucket_grads(wl, i, t) for i in range(len(wl.muon))]
             for t in range(1, wl.steps + 1)]
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    _check_muon(P0, grads, hist, routes)


SHAPES = [(3, 300, 520), (2, 520, 300), (1, 257, 129), (4, 96, 96), (2, 1, 7)]


def test_muon_ragged_buckets():
    P0, grads = _buckets(SHAPES, 21, 3)
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    _check_muon(P0, grads, hist, routes)


@pytest.mark.parametrize("variant", [dict(cautious_wd=True), dict(nesterov=False),
                                     dict(scale_mode=1), dict(ns_steps=3), dict(ns_steps=0),
                                     dict(weight_decay=0.0)])
def test_muon_variants(variant):
    P0, grads = _buckets(SHAPES[:3], 22, 2)
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=variant.get("weight_decay", WD),
                             **{k: v for k, v in variant.items() if k != "weight_decay"})
    _check_muon(P0, grads, hist, routes, **variant)


def test_muon_mixed_configurations():
    """One call whose buckets need three GEMM configurations, so they run as three
    phases over the same workspace: 128-tiles, a 256-tile bucket with a short Gram side
    (combine reads X), and a transposed 128-tile bucket; first and last matrix of each
    checked against the oracle over two steps."""
    shapes = [(3, 200, 330), (43, 768, 1024), (2, 390, 130)]
    count, _ = ma.muon_phases(shapes)
    if "MA_NS_TILE" not in os.environ:  # a forced tile makes them one phase
        assert count == 3
    P0, grads = _buckets(shapes, 24, 2)
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    _check_muon(P0, grads, hist, routes, only=[[0, 2], [0, 42], [0, 1]])


def test_muon_promoted_phase():
    """Buckets that each run on 128-tiles alone but fill the chip together share a phase
    planned on 256-tiles (640-wide Gram sides padded to 768: ragged 256-tile edges, one
    bucket transposed); first and last matrix of each checked against the oracle over
    two steps."""
    shapes = [(24, 640, 640), (12, 640, 2560), (12, 2560, 640)]
    assert ma.muon_phases(shapes) == (1, [0, 0, 0])
    P0, grads = _buckets(shapes, 25, 2)
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    if os.environ.get("MA_NS_TILE") != "128":
        assert [r.m_pad for r in routes] == [768, 768, 768]
    _check_muon(P0, grads, hist, routes, only=[[0, 23], [0, 11], [0, 11]])


def test_muon_zero_gradient_is_pure_decay():
    P0 = [np.random.default_rng(1).standard_normal((2, 130, 70)).astype(np.float32)]
    grads = [[np.zeros((2, 130, 70), np.float32)]] * 2
    hist, _ = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    keep = np.float32(1) - np.float32(LR) * np.float32(WD)
    want = P0[0].astype(np.float64) * (1 - f32(LR) * f32(WD)) ** 2
    assert rel_err_floor(hist[-1][0][0], want) < 1e-6
    assert np.all(hist[-1][0][1] == 0)
    del keep


def test_muon_batch_invariance_and_determinism():
    """A matrix's result is bitwise the same alone (K = 1) or inside a K = 5 bucket,
    and repeated runs give identical bits (owner-based splitting is exact)."""
    P0, grads = _buckets([(5, 200, 330)], 23, 2)
    hist5, _ = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    again, _ = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    for t in range(2):
        assert np.array_equal(hist5[t][0][0], again[t][0][0])
        assert np.array_equal(hist5[t][0][1], again[t][0][1])
    k = 3
    hist1, _ = _muon_run([P0[0][k:k + 1].copy()], [[g[0][k:k + 1].copy()] for g in grads],
                         lr=LR, momentum=MU, weight_decay=WD)
    for t in range(2):
        assert np.array_equal(hist1[t][0][0][0], hist5[t][0][0][k])
        assert np.array_equal(hist1[t][0][1][0], hist5[t][0][1][k])


def test_muon_resume_is_bitwise():
    """Two steps straight equal one step, a state save/restore, and one more step."""
    P0, grads = _buckets([(2, 128, 384)], 24, 2)
    straight, _ = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    p = torch.from_numpy(P0[0]).to(DEV)
    g = torch.from_numpy(grads[0][0]).to(DEV)
    m = torch.zeros_like(p)
    ma.muon_step([(p, g, m)], lr=LR, momentum=MU, weight_decay=WD)
    saved = (p.cpu().clone(), m.cpu().clone())
    p2, m2 = saved[0].to(DEV), saved[1].to(DEV)
    g2 = torch.from_numpy(grads[1][0]).to(DEV)
    ma.muon_step([(p2, g2, m2)], lr=LR, momentum=MU, weight_decay=WD)
    torch.cuda.synchronize()
    assert np.array_equal(p2.cpu().numpy(), straight[1][0][0])
    assert np.array_equal(m2.cpu().numpy(), straight[1][0][1])


def test_optimizer_wrapper_matches_direct_calls():
    P0, grads = _buckets([(2, 96, 160)], 25, 2)
    w = torch.from_numpy(P0[0]).to(DEV)
    vec = torch.from_numpy(np.random.default_rng(2).standard_normal(1000).astype(np.float32)).to(DEV)
    vg = [torch.from_numpy((1e-3 * np.random.default_rng(10 + t).standard_normal(1000)).astype(np.float32)).to(DEV)
          for t in range(2)]
    opt = ma.MuonAdamW([{"params": [w], "kind": "muon", "lr": LR, "momentum": MU, "weight_decay": WD},
                        {"params": [vec], "kind": "adamw", "lr": 3e-3, "betas": (0.9, 0.95),
                         "weight_decay": 0.1}])
    for t in range(2):
        w.grad = torch.from_numpy(grads[t][0]).to(DEV)
        vec.grad = vg[t]
        opt.step()
        opt.zero_grad()
    torch.cuda.synchronize()
    direct, _ = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    assert np.array_equal(w.cpu().numpy(), direct[-1][0][0])
    sd = opt.state_dict()
    assert sd["param_groups"][0]["step"] == 2


def _oracle_check_step(prev, g, mom, got_p, got_m, A, B, hp, tol=MUON_RTOL):
    """One step of one matrix against the oracle stepped from the GPU's previous
    parameters and the oracle's own momentum; returns the oracle's new momentum."""
    ref = oracle.muon_step(prev, g, mom, lr=f32(hp.lr), mu=f32(hp.momentum),
                           weight_decay=f32(hp.weight_decay), cautious_wd=hp.cautious_wd)
    assert rel_err_floor(got_m, ref.momentum) <= MOMENTUM_RTOL
    got = got_p.astype(np.float64)
    if hp.cautious_wd:
        err, flips = cautious_check(prev, got, ref.ortho, f32(hp.lr), f32(hp.weight_decay),
                                    oracle.update_scale(A, B), tol)
        assert flips == 0.0, flips
    else:
        keep = 1.0 - f32(hp.lr) * f32(hp.weight_decay)
        err = rel_fro(prev * keep - got, prev * keep - ref.param)
    assert err <= tol, err
    return ref.momentum, err


@pytest.mark.parametrize("index", [1, 2, 3])
def test_muon_full_size_all_steps(index, capsys):
    """Every bucket of the workload at full size, in the launch configuration the
    benchmark times (one ma_muon_step over all buckets), for the workload's whole step
    count (10, 10 and 5 steps): the first and last matrix of each bucket (the last only
    on the 24-layer workload) against the oracle at every step, stepped from the GPU's
    previous parameters and the oracle's own momentum."""
    wl = workloads.workload(index)
    hp = wl.muon_hp
    ps, gs, ms = [], [], []
    for bi, b in enumerate(wl.muon):
        p = torch.empty((b.K, b.A, b.B), dtype=torch.float32, device=DEV)
        gen.torch_muon_bucket(torch, wl, bi, 0, p)
        ps.append(p)
        gs.append(torch.empty_like(p))
        ms.append(torch.zeros_like(p))
    picks = [(bi, k) for bi, b in enumerate(wl.muon) for k in sorted({0, b.K - 1})]
    if index == 3:
        picks = [(bi, b.K - 1) for bi, b in enumerate(wl.muon)]
    prev = {pk: ps[pk[0]][pk[1]].cpu().numpy().astype(np.float64) for pk in picks}
    mom = {pk: np.zeros((wl.muon[pk[0]].A, wl.muon[pk[0]].B)) for pk in picks}
    worst = 0.0
    for t in range(1, wl.steps + 1):
        for bi in range(len(wl.muon)):
            gen.torch_muon_bucket(torch, wl, bi, t, gs[bi])
        grads = {pk: gs[pk[0]][pk[1]].cpu().numpy() for pk in picks}
        routes = ma.muon_step(list(zip(ps, gs, ms)), lr=hp.lr, momentum=hp.momentum,
                              weight_decay=hp.weight_decay, cautious_wd=hp.cautious_wd)
        torch.cuda.synchronize()
        for bi, b in enumerate(wl.muon):
            o = oracle.route(b.A, b.B)
            r = routes[bi]
            assert (r.transposed, r.m, r.n, r.ns_steps_run) == (o.transposed, o.m, o.n, o.ns_steps)
        for bi, k in picks:
            b = wl.muon[bi]
            got_p = ps[bi][k].cpu().numpy()
            mom[(bi, k)], err = _oracle_check_step(prev[(bi, k)], grads[(bi, k)], mom[(bi, k)],
                                                   got_p, ms[bi][k].cpu().numpy(), b.A, b.B, hp)
            prev[(bi, k)] = got_p.astype(np.float64)
            worst = max(worst, err)
        with capsys.disabled():  # progress on the terminal even under capture
            print(f"workload {index} step {t}: worst update error {worst:.3e}", flush=True)


@pytest.mark.parametrize("shapes", [[(6, 4096, 2304), (6, 2304, 4096)], [(6, 4096, 2304)]])
def test_muon_buckets_that_keep_xt(shapes):
    """Gram sides above 2048 on 256-tiles keep X^T: the combine reads the stored X^T and
    the last combine of a transposed bucket writes only X'^T, which the update reads.
    A transposed 4096 x 2304 bucket (alone, and in one phase with its wide twin) over two
    steps, first and last matrix of each against the oracle."""
    for A, B in [(4096, 2304), (2304, 4096)]:
        assert ma.muon_route_of(A, B).m_pad == 2304
    assert ma.muon_phases(shapes)[0] == 1
    P0, grads = _buckets(shapes, 61, 2)
    hist, routes = _muon_run(P0, grads, lr=LR, momentum=MU, weight_decay=WD)
    assert [r.m_pad for r in routes] == [2304] * len(shapes)
    _check_muon(P0, grads, hist, routes, only=[[0, 5]] * len(shapes))


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_muon_non_finite_gradient_propagates_to_its_matrix_only(bad):
    """Non-finite gradients are not scrubbed: one NaN or Inf entry in matrix 1's gradient
    makes its whole update non-finite (its Frobenius norm is, and the orthogonalisation
    mixes every entry, as in the oracle), its momentum only at that entry, and leaves the
    bucket's other matrices bitwise as in a clean run."""
    shape = (3, 96, 200)
    P0 = [np.random.default_rng(9).standard_normal(shape).astype(np.float32)]
    g = np.stack([_grad(shape[1:], 60 + k) for k in range(3)])
    g_bad = g.copy()
    g_bad[1, 5, 7] = bad
    hist, _ = _muon_run(P0, [[g_bad]], lr=LR, momentum=MU, weight_decay=WD)
    clean, _ = _muon_run(P0, [[g]], lr=LR, momentum=MU, weight_decay=WD)
    p, m = hist[0][0]
    pc, mc = clean[0][0]
    assert not np.isfinite(p[1]).any()
    with np.errstate(invalid="ignore"):  # Inf / Inf in the normalisation, as intended
        ref = oracle.muon_step(P0[0][1], g_bad[1], np.zeros(shape[1:]), lr=f32(LR), mu=f32(MU),
                               weight_decay=f32(WD))
    assert not np.isfinite(ref.param).any()
    bad_m = ~np.isfinite(m[1])
    assert bad_m.sum() == 1 and bad_m[5, 7]
    for k in (0, 2):
        assert np.array_equal(p[k], pc[k]) and np.array_equal(m[k], mc[k])


def test_ns_time_reads_gradients_only():
    """ma_muon_ns_time (the benchmark's Newton-Schulz timer): one positive time per phase,
    gradients unchanged, and no parameter or momentum touched (none is passed)."""
    shapes = [(4, 256, 512), (2, 600, 200), (3, 768, 768)]
    gs = [torch.randn(s, device=DEV) * 0.02 for s in shapes]
    before = [g.clone() for g in gs]
    ms = ma.muon_ns_time(gs, reps=2)
    assert len(ms) == ma.muon_phases(shapes)[0] and all(t > 0 for t in ms)
    assert all(torch.equal(a, b) for a, b in zip(gs, before))


def test_optimizer_buckets_a_models_matrices():
    """MuonAdamW over the 12-layer GPT's 72 separate hidden matrices (per layer Q, K, V, O
    768 x 768, MLP 768 x 3072 and 3072 x 768, interleaved as a model lists them): they
    become three (K, A, B) buckets that run as one phase, the parameters the caller
    holds see the updates, and two steps are bit for bit the stacked ma_muon_step's.
    A third step where one matrix has no gradient leaves that matrix alone."""
    wl = workloads.workload(1)
    shapes = [(768, 768)] * 4 + [(768, 3072), (3072, 768)]
    gen_ = torch.Generator(device=DEV).manual_seed(3)
    params = [torch.nn.Parameter(torch.randn(s, generator=gen_, device=DEV))
              for _ in range(12) for s in shapes]
    grads = [[0.02 * torch.randn(p.shape, generator=gen_, device=DEV) for p in params]
             for _ in range(3)]
    stacks = [torch.stack([p.detach().clone() for p in params if tuple(p.shape) == s])
              for s in [(768, 768), (768, 3072), (3072, 768)]]
    opt = ma.MuonAdamW([{"params": params, "kind": "muon", "lr": LR, "momentum": MU,
                         "weight_decay": WD}])
    assert opt.muon_buckets() == [(48, 768, 768), (12, 768, 3072), (12, 3072, 768)]
    assert ma.muon_phases(opt.muon_buckets()) == (1, [0, 0, 0])
    moms = [torch.zeros_like(s) for s in stacks]
    for t in range(2):
        for p, g in zip(params, grads[t]):
            p.grad = g.clone()
        opt.step()
        gst = [torch.stack([g for p, g in zip(params, grads[t]) if tuple(p.shape) == tuple(s.shape[1:])])
               for s in stacks]
        ma.muon_step(list(zip(stacks, gst, moms)), lr=LR, momentum=MU, weight_decay=WD)
        torch.cuda.synchronize()
        for s, st in zip([(768, 768), (768, 3072), (3072, 768)], stacks):
            mine = [p.detach() for p in params if tuple(p.shape) == s]
            assert all(torch.equal(a, b) for a, b in zip(mine, st)), (t, s)
        opt.zero_grad()
    keep = params[5].detach().clone()
    for k, (p, g) in enumerate(zip(params, grads[2])):
        p.grad = None if k == 5 else g.clone()
    opt.step()
    torch.cuda.synchronize()
    assert torch.equal(params[5].detach(), keep)
    assert not torch.equal(params[4].detach(), stacks[1][0])
    del wl


def test_newton_schulz_maximum_iteration_count():
    """MA_MAX_NS_STEPS (64) iterations of the cubic (1.5, -0.5, 0), which converges to the
    polar factor U V^T and is contractive there, so bf16 rounding does not accumulate:
    against the oracle and against numpy's U V^T."""
    G = _grad((96, 160), 71)[None]
    gi = torch.from_numpy(G).to(DEV)
    go = torch.empty_like(gi)
    ma.newton_schulz(gi, go, ns_steps=64, ns_coeffs=(1.5, -0.5, 0.0))
    torch.cuda.synchronize()
    ref = oracle.newton_schulz(G[0], 64, (1.5, -0.5, 0.0))
    assert rel_fro(go.cpu().numpy()[0], ref) <= MUON_RTOL
    U, _, Vt = np.linalg.svd(G[0].astype(np.float64), full_matrices=False)
    assert rel_fro(go.cpu().numpy()[0], U @ Vt) <= MUON_RTOL


def test_muon_largest_bucket_count():
    """A bucket of K = 65535 matrices (the largest the launch grids take; K = 65536 is
    rejected before launch): first, middle and last matrix against the oracle."""
    K, A, B = 65535, 16, 40
    gen_ = torch.Generator(device=DEV).manual_seed(12)
    p = torch.randn((K, A, B), generator=gen_, device=DEV)
    g = 0.02 * torch.randn((K, A, B), generator=gen_, device=DEV)
    m = torch.zeros_like(p)
    picks = [0, K // 2, K - 1]
    saved = {k: (p[k].cpu().numpy().copy(), g[k].cpu().numpy().copy()) for k in picks}
    ma.muon_step([(p, g, m)], lr=LR, momentum=MU, weight_decay=WD)
    torch.cuda.synchronize()
    keep = 1.0 - f32(LR) * f32(WD)
    for k in picks:
        p0, g0 = saved[k]
        ref = oracle.muon_step(p0, g0, np.zeros((A, B)), lr=f32(LR), mu=f32(MU), weight_decay=f32(WD))
        prev = p0.astype(np.float64)
        err = rel_fro(prev * keep - p[k].cpu().numpy(), prev * keep - ref.param)
        assert err <= MUON_RTOL, (k, err)
    with pytest.raises(ma.MuonAdamWError):
        big = torch.zeros((65536, 1, 2), device=DEV)
        ma.muon_step([(big, big.clone(), big.clone())], lr=LR)


def test_muon_step_with_empty_buckets():
    """Empty buckets (K = 0) between real ones are skipped: their route records stay
    zero and the real buckets match the oracle."""
    P0, grads = _buckets([(2, 64, 128), (3, 130, 70)], 81, 1)
    empty = torch.zeros((0, 50, 60), device=DEV)
    ps = [torch.from_numpy(x).to(DEV) for x in P0]
    ms = [torch.zeros_like(x) for x in ps]
    gs = [torch.from_numpy(x).to(DEV) for x in grads[0]]
    routes = ma.muon_step([(empty, empty.clone(), empty.clone()), (ps[0], gs[0], ms[0]),
                           (empty, empty.clone(), empty.clone()), (ps[1], gs[1], ms[1])],
                          lr=LR, momentum=MU, weight_decay=WD)
    torch.cuda.synchronize()
    assert routes[0].m == 0 and routes[2].m == 0 and routes[1].m == 64 and routes[3].m == 70
    hist = [[(ps[i].cpu().numpy(), ms[i].cpu().numpy()) for i in range(2)]]
    _check_muon(P0, grads, hist, [routes[1], routes[3]])

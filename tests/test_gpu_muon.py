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


@pytest.mark.parametrize("index", [1, 2, 3])
def test_muon_full_size_sampled(index):
    """Every bucket of the workload at full size, in the launch configuration the
    benchmark times (one ma_muon_step over all buckets); the first and last matrix
    of each bucket re-computed by the oracle."""
    wl = workloads.workload(index)
    hp = wl.muon_hp
    ps, gs, ms = [], [], []
    for bi, b in enumerate(wl.muon):
        p = torch.empty((b.K, b.A, b.B), dtype=torch.float32, device=DEV)
        gen.torch_muon_bucket(torch, wl, bi, 0, p)
        g = torch.empty_like(p)
        gen.torch_muon_bucket(torch, wl, bi, 1, g)
        ps.append(p)
        gs.append(g)
        ms.append(torch.zeros_like(p))
    picks = [(bi, k) for bi, b in enumerate(wl.muon) for k in sorted({0, b.K - 1})]
    if index == 3:
        picks = [(bi, b.K - 1) for bi, b in enumerate(wl.muon)]
    saved = {(bi, k): (ps[bi][k].cpu().numpy().copy(), gs[bi][k].cpu().numpy().copy())
             for bi, k in picks}
    routes = ma.muon_step(list(zip(ps, gs, ms)), lr=hp.lr, momentum=hp.momentum,
                          weight_decay=hp.weight_decay, cautious_wd=hp.cautious_wd)
    torch.cuda.synchronize()
    for bi, b in enumerate(wl.muon):
        o = oracle.route(b.A, b.B)
        r = routes[bi]
        assert (r.transposed, r.m, r.n, r.ns_steps_run) == (o.transposed, o.m, o.n, o.ns_steps)
    for bi, k in picks:
        b = wl.muon[bi]
        p0, g1 = saved[(bi, k)]
        ref = oracle.muon_step(p0, g1, np.zeros_like(p0, dtype=np.float64), lr=f32(hp.lr),
                               mu=f32(hp.momentum), weight_decay=f32(hp.weight_decay),
                               cautious_wd=hp.cautious_wd)
        got = ps[bi][k].cpu().numpy().astype(np.float64)
        prev = p0.astype(np.float64)
        if hp.cautious_wd:
            err, flips = cautious_check(prev, got, ref.ortho, f32(hp.lr), f32(hp.weight_decay),
                                        oracle.update_scale(b.A, b.B), MUON_RTOL)
            assert flips == 0.0, (bi, k, flips)
        else:
            keep = 1.0 - f32(hp.lr) * f32(hp.weight_decay)
            err = rel_fro(prev * keep - got, prev * keep - ref.param)
        assert err <= MUON_RTOL, (bi, k, err)
        assert rel_err_floor(ms[bi][k].cpu().numpy(), ref.momentum) <= MOMENTUM_RTOL


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

"""AdamW through the C ABI on the GPU against the fp64 oracle, element by element."""
import numpy as np
import pytest

import oracle
import workloads
from parity import ADAMW_RTOL, adamw_term_scales, f32, rel_err_floor
from workloads import gen

torch = pytest.importorskip("torch")
ma = pytest.importorskip("adamw_optimizer_step_muon_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _hp(**kw):
    base = dict(lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, decoupled=True,
                cautious_wd=False)
    base.update(kw)
    return base


def _oracle_hp(hp):
    return {k: (f32(v) if isinstance(v, float) else v) for k, v in hp.items()}


def _run(p0, grads, hp, offset=0):
    """Run len(grads) steps on the GPU; return (param, exp_avg, exp_avg_sq) per step."""
    n = p0.size
    buf = torch.zeros(4, n + offset, dtype=torch.float32, device=DEV)
    gbuf = torch.zeros(n + offset, dtype=torch.float32, device=DEV)
    p, m, v = buf[0, offset:], buf[1, offset:], buf[2, offset:]
    g = gbuf[offset:]
    p.copy_(torch.from_numpy(p0))
    out = []
    for t, gr in enumerate(grads, start=1):
        g.copy_(torch.from_numpy(gr))
        ma.adamw_step(p, g, m, v, step=t, **hp)
        torch.cuda.synchronize()
        out.append((p.cpu().numpy().copy(), m.cpu().numpy().copy(), v.cpu().numpy().copy()))
    return out


def _oracle(p0, grads, hp):
    p, m, v = p0.astype(np.float64), np.zeros(p0.size), np.zeros(p0.size)
    out = []
    for t, gr in enumerate(grads, start=1):
        r = oracle.adamw_step(p, gr, m, v, step=t, **_oracle_hp(hp))
        p, m, v = r.param, r.exp_avg, r.exp_avg_sq
        out.append((p, m, v))
    return out


def _check(got, p0, grads, hp, traj=None):
    """Each GPU step against the oracle's step from the GPU's own previous state,
    element by element within ADAMW_RTOL of the magnitude of the terms that form
    it; where cautious decay is on and the update is within that bound of zero,
    either decay decision is accepted.  ``traj`` (the oracle's own run from p0) is
    also compared for large tensors, relative to |ref| + RMS(ref)."""
    ohp = _oracle_hp(hp)
    prev = (p0.astype(np.float64), np.zeros(p0.size), np.zeros(p0.size))
    for t, (gr, cur) in enumerate(zip(grads, got), start=1):
        ref = oracle.adamw_step(*prev[:1], gr, *prev[1:], step=t, **ohp)
        sp, sm, sv, su = adamw_term_scales(prev[0], gr, prev[1], prev[2], step=t, **ohp)
        errs = {}
        for name, a, b, sc in (("param", cur[0], ref.param, sp), ("exp_avg", cur[1], ref.exp_avg, sm),
                               ("exp_avg_sq", cur[2], ref.exp_avg_sq, sv)):
            d = np.abs(a.astype(np.float64) - b)
            if name == "param" and ohp.get("cautious_wd"):
                # either decision where the update's sign is not decided in fp32
                upd = ref.exp_avg / (1 - ohp["beta1"] ** t) / (
                    np.sqrt(ref.exp_avg_sq / (1 - ohp["beta2"] ** t)) + ohp["eps"])
                amb = np.abs(upd) <= ADAMW_RTOL * su
                other = prev[0] * np.where(upd * prev[0] > 0, 1.0, 1 - ohp["lr"] * ohp["weight_decay"]) \
                    - ohp["lr"] * upd
                d = np.where(amb, np.minimum(d, np.abs(a - other)), d)
            with np.errstate(invalid="ignore", divide="ignore"):
                e = np.where(sc > 0, d / sc, d)
            errs[name] = float(np.max(e)) if e.size else 0.0
            assert errs[name] <= ADAMW_RTOL, f"step {t} {name}: {errs[name]:.3e}"
        prev = tuple(x.astype(np.float64) for x in cur)
    if traj is not None and p0.size >= 4096:
        for (gp, gm, gv), (rp, rm, rv) in zip(got, traj):
            for a, b in ((gp, rp), (gm, rm), (gv, rv)):
                assert rel_err_floor(a, b) <= 4 * ADAMW_RTOL


@pytest.mark.parametrize("n", [1, 3, 4, 5, 255, 1023, 4096, 262147])
@pytest.mark.parametrize("offset", [0, 1])
def test_adamw_ragged_and_misaligned(n, offset):
    rng = np.random.default_rng(n * 7 + offset)
    p0 = rng.standard_normal(n).astype(np.float32)
    grads = [(1e-3 * rng.standard_normal(n)).astype(np.float32) for _ in range(3)]
    hp = _hp()
    _check(_run(p0, grads, hp, offset), p0, grads, hp, _oracle(p0, grads, hp))


@pytest.mark.parametrize("variant", [dict(decoupled=False), dict(cautious_wd=True),
                                     dict(weight_decay=0.0), dict(beta2=0.999, lr=1e-2)])
def test_adamw_variants(variant):
    rng = np.random.default_rng(5)
    n = 100003
    p0 = rng.standard_normal(n).astype(np.float32)
    grads = [(1e-3 * rng.standard_normal(n)).astype(np.float32) for _ in range(4)]
    hp = _hp(**variant)
    _check(_run(p0, grads, hp), p0, grads, hp, _oracle(p0, grads, hp))


def test_adamw_decay_experiment_on_gpu(golden):
    # the handbook's decay experiment (gradients 1000x apart, 1000 steps) through the kernel
    g = golden("adamw_decay_experiment.txt")
    scale = np.array([0.01, 10.0], dtype=np.float32)
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1)
    out = {}
    for decoupled in (False, True):
        p = torch.ones(2, device=DEV)
        gr = torch.zeros(2, device=DEV)
        m, v = torch.zeros(2, device=DEV), torch.zeros(2, device=DEV)
        for t in range(1000):
            gr.copy_(torch.from_numpy(scale * (-1.0) ** t))
            ma.adamw_step(p, gr, m, v, step=t + 1, decoupled=decoupled, **hp)
        out[decoupled] = p.cpu().numpy()
    assert f"{out[False][0]:.3f}" == g["coupled_small"][0]
    assert f"{out[False][1]:.3f}" == g["coupled_large"][0]
    assert f"{out[True][0]:.3f}" == g["decoupled_small"][0]
    assert f"{out[True][1]:.3f}" == g["decoupled_large"][0]


def test_adamw_tiny_workload_all_steps():
    wl = workloads.workload(0)
    p0 = gen.np_adamw_flat_params(wl)
    grads = [gen.np_adamw_flat_grads(wl, t) for t in range(1, wl.steps + 1)]
    ah = wl.adamw_hp
    hp = _hp(lr=ah.lr, beta1=ah.beta1, beta2=ah.beta2, eps=ah.eps, weight_decay=ah.weight_decay)
    _check(_run(p0, grads, hp), p0, grads, hp, _oracle(p0, grads, hp))


def test_adamw_zero_length_and_determinism():
    rng = np.random.default_rng(9)
    n = 65537
    p0 = rng.standard_normal(n).astype(np.float32)
    grads = [(1e-3 * rng.standard_normal(n)).astype(np.float32) for _ in range(2)]
    a = _run(p0, grads, _hp())
    b = _run(p0, grads, _hp())
    for x, y in zip(a, b):
        for u, w in zip(x, y):
            assert np.array_equal(u, w)
    e = torch.empty(0, device=DEV)
    ma.adamw_step(e, e, e, e, step=1, lr=1e-3)


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_adamw_full_size_sampled(index):
    """Full flat AdamW buffer of the workload, in the launch configuration the
    benchmark times; 200k sampled elements re-computed by the oracle one by one."""
    wl = workloads.workload(index)
    n = wl.adamw_numel
    ah = wl.adamw_hp
    hp = _hp(lr=ah.lr, beta1=ah.beta1, beta2=ah.beta2, eps=ah.eps, weight_decay=ah.weight_decay)
    steps = 2
    p = torch.empty(n, dtype=torch.float32, device=DEV)
    gen.torch_adamw_flat(torch, wl, 0, p)
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    idx = np.sort(np.random.default_rng(index).choice(n, size=200_000, replace=False))
    tidx = torch.from_numpy(idx).to(DEV)
    g = torch.empty_like(p)
    got, gs = [], []
    p0 = p[tidx].cpu().numpy()
    for t in range(1, steps + 1):
        gen.torch_adamw_flat(torch, wl, t, g)
        gs.append(g[tidx].cpu().numpy())
        ma.adamw_step(p, g, m, v, step=t, **hp)
        torch.cuda.synchronize()
        got.append((p[tidx].cpu().numpy(), m[tidx].cpu().numpy(), v[tidx].cpu().numpy()))
    _check(got, p0, gs, hp, _oracle(p0, gs, hp))


@pytest.mark.parametrize("variant", [dict(), dict(decoupled=False), dict(cautious_wd=True)])
def test_adamw_multi_matches_per_tensor_bitwise(variant):
    """ma_adamw_step_multi over 130 tensors (three launches of at most 48): ragged sizes,
    starts misaligned for the vector path, a gradient shared by two tensors, an empty
    tensor; every element bitwise equal to ma_adamw_step on the same tensor."""
    rng = np.random.default_rng(11)
    sizes = [int(x) for x in rng.integers(1, 9000, size=126)] + [0, 4096, 4097, 100_003]
    store = torch.randn(sum(sizes) + 8, device="cuda")
    shared = torch.randn(4097, device="cuda") * 1e-3
    segs, segs_ref = [], []
    off = 0
    for i, n in enumerate(sizes):
        lo = off + (i % 3)                           # odd starts: scalar path
        p = store[lo:lo + n].clone() if i % 5 else store[lo:lo + n].clone()[0:n]
        g = shared[:n] if (n <= 4097 and i in (3, 7)) else torch.randn(n, device="cuda") * 1e-3
        m = torch.randn(n, device="cuda").abs() * 1e-4
        v = torch.randn(n, device="cuda").abs() * 1e-6
        if i % 3:                                     # misaligned views of fresh buffers
            big = torch.empty(n + 1, device="cuda"); big[1:].copy_(p); p = big[1:]
        segs.append((p, g, m, v))
        segs_ref.append((p.clone(), g, m.clone(), v.clone()))
        off += n
    hp = dict(step=3, lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, **variant)
    ma.adamw_step_multi(segs, **hp)
    for p, g, m, v in segs_ref:
        ma.adamw_step(p, g, m, v, **hp)
    torch.cuda.synchronize()
    for (a, _, am, av), (b, _, bm, bv) in zip(segs, segs_ref):
        assert torch.equal(a, b) and torch.equal(am, bm) and torch.equal(av, bv)


def test_adamw_non_finite_gradient_stays_in_its_element():
    """No scrubbing: a NaN gradient element makes that element's parameter and moments
    NaN; every other element is bitwise as in a clean step (vector and tail paths)."""
    n = 4099
    rng = np.random.default_rng(12)
    p0 = rng.standard_normal(n).astype(np.float32)
    g = (1e-3 * rng.standard_normal(n)).astype(np.float32)
    g_bad = g.copy()
    g_bad[[10, 4097]] = np.nan          # one in the float4 body, one in the scalar tail
    hp = _hp()
    got = _run(p0, [g_bad], hp)[0]
    clean = _run(p0, [g], hp)[0]
    mask = np.zeros(n, bool)
    mask[[10, 4097]] = True
    for a, b in zip(got, clean):
        assert np.isnan(a[mask]).all()
        assert np.array_equal(a[~mask], b[~mask])


def test_stream_probe_values():
    """The bandwidth probe computes what it states (so its loads and stores are real):
    out[j] = in[0] + ... + in[R-1] + j, also streamed in place."""
    n = 1 << 16
    gen_ = torch.Generator(device="cuda").manual_seed(4)
    a, b, c, d = (torch.randn(n, generator=gen_, device="cuda") for _ in range(4))
    o1, o2 = torch.empty_like(a), torch.empty_like(a)
    ma.stream_probe([a, b, c], [o1, o2])
    torch.cuda.synchronize()
    assert torch.equal(o1, ((a + b) + c)) and torch.equal(o2, ((a + b) + c) + 1.0)
    ref = ((a + b) + c) + d
    ma.stream_probe([a, b, c, d], [a, c, d])
    torch.cuda.synchronize()
    assert torch.equal(a, ref) and torch.equal(c, ref + 1.0) and torch.equal(d, ref + 2.0)

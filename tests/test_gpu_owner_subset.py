"""The owner-subset workload at full size (8 x 8192x28672, 8 x 28672x8192, 16 x 8192x8192;
58 GB of fp32 Muon state) through ma_muon_step, in the launch configuration the
benchmark times, for the workload's three steps.

Sampled against the fp64 oracle, each stepped from the GPU's previous parameters and
the oracle's own momentum:
* the last matrix of the transposed 28672 x 8192 bucket at every step: the printed
  iteration with X^T kept (Gram side 8192 > 2048), whose last combine writes only X'^T,
  which the update reads;
* the first 8192 x 28672 matrix and the last 8192 x 8192 matrix at the last step (their
  momentum at every step).
Routing reports exact.
"""
import numpy as np
import pytest

import oracle
import workloads
from parity import MOMENTUM_RTOL, rel_err_floor
from test_gpu_muon import _oracle_check_step
from workloads import gen

torch = pytest.importorskip("torch")
ma = pytest.importorskip("adamw_optimizer_step_muon_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_owner_subset_full_size_three_steps(capsys):
    wl = workloads.workload(4)

    def progress(msg):
        # straight to the terminal even when pytest captures output: the oracle calls
        # take tens of seconds each, and a silent run looks hung
        with capsys.disabled():
            print(msg, flush=True)

    hp = wl.muon_hp
    ps, gs, ms = [], [], []
    for bi, b in enumerate(wl.muon):
        p = torch.empty((b.K, b.A, b.B), dtype=torch.float32, device=DEV)
        gen.torch_muon_bucket(torch, wl, bi, 0, p)
        ps.append(p)
        gs.append(torch.empty_like(p))
        ms.append(torch.zeros_like(p))
    down = (1, wl.muon[1].K - 1)
    picks = [(0, 0), down, (2, wl.muon[2].K - 1)]
    prev = {pk: ps[pk[0]][pk[1]].cpu().numpy().astype(np.float64) for pk in picks}
    mom = {pk: np.zeros((wl.muon[pk[0]].A, wl.muon[pk[0]].B)) for pk in picks}
    mu = np.float64(np.float32(hp.momentum))
    for t in range(1, wl.steps + 1):
        for bi in range(len(wl.muon)):
            gen.torch_muon_bucket(torch, wl, bi, t, gs[bi])
        grads = {pk: gs[pk[0]][pk[1]].cpu().numpy() for pk in picks}
        routes = ma.muon_step(list(zip(ps, gs, ms)), lr=hp.lr, momentum=hp.momentum,
                              weight_decay=hp.weight_decay)
        torch.cuda.synchronize()
        for bi, b in enumerate(wl.muon):
            o = oracle.route(b.A, b.B)
            r = routes[bi]
            assert (r.transposed, r.m, r.n, r.ns_steps_run) == (o.transposed, o.m, o.n, o.ns_steps)
        for pk in picks:
            b = wl.muon[pk[0]]
            got_p = ps[pk[0]][pk[1]].cpu().numpy()
            got_m = ms[pk[0]][pk[1]].cpu().numpy()
            if pk == down or t == wl.steps:
                progress(f"step {t} bucket {pk[0]} matrix {pk[1]}: oracle running")
                mom[pk], err = _oracle_check_step(prev[pk], grads[pk], mom[pk], got_p, got_m,
                                                  b.A, b.B, hp)
                progress(f"step {t} bucket {pk[0]} matrix {pk[1]}: update error {err:.3e}")
            else:
                # momentum only (sum form, exact closed form per step)
                mom[pk] = mu * mom[pk] + grads[pk].astype(np.float64)
                assert rel_err_floor(got_m, mom[pk]) <= MOMENTUM_RTOL
            prev[pk] = got_p.astype(np.float64)


def test_owner_subset_gram_space_first_step(capsys):
    """The same workload under ns_mode 1: both 3.5:1 buckets take the fp16 Gram-space
    route (the transposed one keeping X0^T, whose last product writes X'^T), the square
    bucket the printed iteration, all in one ma_muon_step.  The first 8192 x 28672 and the
    last 28672 x 8192 matrix against the oracle after the first step; every routing
    report exact."""
    wl = workloads.workload(4)

    def progress(msg):
        with capsys.disabled():
            print(msg, flush=True)

    hp = wl.muon_hp
    ps, gs, ms = [], [], []
    for bi, b in enumerate(wl.muon):
        p = torch.empty((b.K, b.A, b.B), dtype=torch.float32, device=DEV)
        gen.torch_muon_bucket(torch, wl, bi, 0, p)
        ps.append(p)
        g = torch.empty_like(p)
        gen.torch_muon_bucket(torch, wl, bi, 1, g)
        gs.append(g)
        ms.append(torch.zeros_like(p))
    picks = [(0, 0), (1, wl.muon[1].K - 1)]
    prev = {pk: ps[pk[0]][pk[1]].cpu().numpy().astype(np.float64) for pk in picks}
    grads = {pk: gs[pk[0]][pk[1]].cpu().numpy() for pk in picks}
    routes = ma.muon_step(list(zip(ps, gs, ms)), lr=hp.lr, momentum=hp.momentum,
                          weight_decay=hp.weight_decay, ns_mode=1)
    torch.cuda.synchronize()
    assert [r.ns_mode_run for r in routes] == [1, 1, 0]
    for bi, b in enumerate(wl.muon):
        o = oracle.route(b.A, b.B)
        r = routes[bi]
        assert (r.transposed, r.m, r.n, r.ns_steps_run) == (o.transposed, o.m, o.n, o.ns_steps)
    for pk in picks:
        b = wl.muon[pk[0]]
        got_p = ps[pk[0]][pk[1]].cpu().numpy()
        got_m = ms[pk[0]][pk[1]].cpu().numpy()
        progress(f"gram-space step 1 bucket {pk[0]} matrix {pk[1]}: oracle running")
        _, err = _oracle_check_step(prev[pk], grads[pk], np.zeros((b.A, b.B)), got_p, got_m,
                                    b.A, b.B, hp)
        progress(f"gram-space step 1 bucket {pk[0]} matrix {pk[1]}: update error {err:.3e}")

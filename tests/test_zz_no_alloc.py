"""ma_muon_step_static: the Muon step on the library's static device workspace (for
callers that cannot allocate), against ma_muon_step with a caller workspace: bit for bit
the same parameters and momenta on two calls in a row, the second with smaller buckets
(the workspace keeps the first call's contents), and requests above the static
workspace's size rejected before anything is launched."""
import ctypes

import numpy as np
import pytest

import oracle
from parity import MUON_RTOL, f32, rel_fro

torch = pytest.importorskip("torch")
ma = pytest.importorskip("adamw_optimizer_step_muon_amd")
from adamw_optimizer_step_muon_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HP = dict(lr=0.02, momentum=0.95, weight_decay=0.1)


def _state(shapes, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return [(torch.randn(s, generator=g, device=DEV), 0.02 * torch.randn(s, generator=g, device=DEV),
             0.01 * torch.randn(s, generator=g, device=DEV)) for s in shapes]


def _clone(state):
    return [(p.clone(), g.clone(), m.clone()) for p, g, m in state]


@pytest.mark.parametrize("calls", [
    [[(3, 300, 520), (2, 520, 300), (8, 768, 768)], [(2, 96, 200)]],
    [[(4, 2048, 4096)], [(1, 257, 129), (1, 1, 7)]],
])
def test_static_step_matches_workspace_step(calls):
    for i, shapes in enumerate(calls):
        assert ma.muon_workspace_bytes(shapes) <= _lib.MA_STATIC_WORKSPACE_BYTES
        state = _state(shapes, 100 + i)
        ref, got = _clone(state), _clone(state)
        r_ref = ma.muon_step(ref, **HP)
        r_got = ma.muon_step_static(got, **HP)
        torch.cuda.synchronize()
        assert r_ref == r_got
        for (p0, g0, m0), (pr, _, mr), (pg, _, mg) in zip(state, ref, got):
            assert torch.equal(pr, pg) and torch.equal(mr, mg)
        # and the shared result meets the oracle (first matrix of the first bucket)
        p0, g0, m0 = (t[0].cpu().numpy() for t in state[0])
        o = oracle.muon_step(p0, g0, m0, lr=f32(0.02), mu=f32(0.95), weight_decay=f32(0.1))
        keep = 1.0 - f32(0.02) * f32(0.1)
        prev = p0.astype(np.float64)
        assert rel_fro(prev * keep - got[0][0][0].cpu().numpy(), prev * keep - o.param) <= MUON_RTOL


def test_static_step_rejects_buckets_above_its_workspace():
    shapes = [(16, 4096, 4096)]
    need = ma.muon_workspace_bytes(shapes)
    assert need > _lib.MA_STATIC_WORKSPACE_BYTES
    lib = _lib.load()
    arr = (_lib._MuonBucket * 1)()
    # disjoint placeholders: the call must fail on the size before touching them
    base = 1 << 44
    nbytes = 16 * 4096 * 4096 * 4
    arr[0] = _lib._MuonBucket(16, 4096, 4096, base, base + nbytes, base + 2 * nbytes)
    hp, _ = _lib._muon_hparams(0.02, 0.95, 0.1, True, 5, None, 1e-7, False, 0, 0)
    assert lib.ma_muon_step_static(arr, 1, ctypes.byref(hp), None, None) == _lib.MA_ERR_WORKSPACE
    assert b"static workspace" in lib.ma_last_error()

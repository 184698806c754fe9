"""The step enqueues kernels only (no allocation, memset or synchronisation inside the
library), so a caller can capture it in a HIP graph.  Replays, with eager work and
synchronisations between them, must match the same steps run eagerly, bit for bit
(the kernels are deterministic)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
ma = pytest.importorskip("adamw_optimizer_step_muon_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPES = [(3, 200, 330), (2, 455, 130), (2, 130, 455), (4, 256, 256)]


def _state(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    ps = [torch.randn(s, device=DEV, generator=g) for s in SHAPES]
    gs = [torch.randn(s, device=DEV, generator=g) * 0.02 for s in SHAPES]
    ms = [torch.zeros(s, device=DEV) for s in SHAPES]
    return ps, gs, ms


@pytest.mark.parametrize("ns_mode", [0, 1])
def test_muon_step_graph_replays_match_eager(ns_mode):
    """ns_mode 1 routes the 3.5:1 buckets (130 x 455 and its transpose) through the fp16
    Gram-space launches."""
    assert [ma.muon_route_of(A, B, 5, ns_mode=ns_mode).ns_mode_run for _, A, B in SHAPES] == \
        [0, ns_mode, ns_mode, 0]
    ps, gs, ms = _state(5)
    ps_e, ms_e = [p.clone() for p in ps], [m.clone() for m in ms]
    ws = torch.empty(ma.muon_workspace_bytes(SHAPES, ns_mode), dtype=torch.uint8, device=DEV)
    ws_e = torch.empty_like(ws)
    hp = dict(lr=0.02, momentum=0.95, weight_decay=0.1, cautious_wd=True, ns_mode=ns_mode)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ma.muon_step(list(zip(ps, gs, ms)), workspace=ws, **hp)
    for step in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = (torch.ones(1024, device=DEV) * step).sum().item()  # eager work between replays
        ma.muon_step(list(zip(ps_e, gs, ms_e)), workspace=ws_e, **hp)
        torch.cuda.synchronize()
        for a, b in zip(ps + ms, ps_e + ms_e):
            assert torch.equal(a, b), step


def test_static_workspace_step_graph_replays_match_eager():
    """ma_muon_step_static, the entry point for callers that cannot allocate, captured in
    a HIP graph (its workspace resolved once before the capture): replays with eager work
    between them match eager ma_muon_step calls on a caller workspace bit for bit."""
    ps, gs, ms = _state(8)
    ps_e, ms_e = [p.clone() for p in ps], [m.clone() for m in ms]
    ws_e = torch.empty(ma.muon_workspace_bytes(SHAPES), dtype=torch.uint8, device=DEV)
    hp = dict(lr=0.02, momentum=0.95, weight_decay=0.1)
    ma.muon_static_init()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ma.muon_step_static(list(zip(ps, gs, ms)), **hp)
    for step in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = (torch.ones(1024, device=DEV) * step).sum().item()  # eager work between replays
        ma.muon_step(list(zip(ps_e, gs, ms_e)), workspace=ws_e, **hp)
        torch.cuda.synchronize()
        for a, b in zip(ps + ms, ps_e + ms_e):
            assert torch.equal(a, b), step


def test_adamw_step_graph_replay_matches_eager():
    g = torch.Generator(device=DEV)
    g.manual_seed(6)
    n = 300_001
    p = torch.randn(n, device=DEV, generator=g)
    grad = torch.randn(n, device=DEV, generator=g) * 1e-3
    m, v = torch.zeros_like(p), torch.zeros_like(p)
    p_e, m_e, v_e = p.clone(), m.clone(), v.clone()
    hp = dict(step=1, lr=3e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ma.adamw_step(p, grad, m, v, **hp)
    graph.replay()
    torch.cuda.synchronize()
    ma.adamw_step(p_e, grad, m_e, v_e, **hp)
    torch.cuda.synchronize()
    for a, b in ((p, p_e), (m, m_e), (v, v_e)):
        assert torch.equal(a, b)
    assert not np.isnan(p.cpu().numpy()).any()

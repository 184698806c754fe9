"""The C ABI on the host: the library loads, exports every symbol the header
declares, routes shapes like the oracle, sizes workspaces, and rejects bad
arguments before launching anything (no GPU needed: nothing here reaches a kernel).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from conftest import ROOT

ma = pytest.importorskip("adamw_optimizer_step_muon_amd")
from adamw_optimizer_step_muon_amd import _lib  # noqa: E402

HEADER = os.path.join(ROOT, "include", "muon_adamw.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libmuonadamw.so not built")
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ma_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = _declared()
    assert set(declared) == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_matches_header(lib):
    m = re.search(r"#define MA_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.ma_abi_version() == int(m.group(1)) == _lib.ABI_VERSION
    assert lib.ma_status_string(0) == b"ok"
    assert lib.ma_status_string(-3).startswith(b"workspace")


@pytest.mark.parametrize("A,B", [(64, 128), (128, 64), (768, 768), (768, 3072), (3072, 768),
                                 (2048, 512), (512, 2048), (8192, 28672), (28672, 8192),
                                 (1, 1), (1, 5), (5, 1), (257, 129), (129, 257)])
@pytest.mark.parametrize("steps", [0, 5, 7])
def test_routing_matches_oracle(lib, A, B, steps):
    r = ma.muon_route_of(A, B, steps)
    o = oracle.route(A, B, steps)
    assert (r.transposed, r.m, r.n, r.ns_steps_run) == (o.transposed, o.m, o.n, o.ns_steps)
    assert r.m_pad % 128 == 0 and r.n_pad % 128 == 0
    assert r.m <= r.m_pad < r.m + 128 and r.n <= r.n_pad < r.n + 128


def test_workspace_bytes(lib):
    assert ma.muon_workspace_bytes([]) == 0
    one = ma.muon_workspace_bytes([(1, 768, 3072)])
    # X twice (bf16 ping-pong, m x n, one orientation) plus R and P (bf16, m x m), plus
    # a little norm scratch
    xr = 2 * 768 * 3072 * 2 + 2 * 768 * 768 * 2
    assert xr <= one < xr + 65536
    assert ma.muon_workspace_bytes([(2, 768, 3072)]) > one
    # small buckets with the same tile share a phase: their needs add up
    other = ma.muon_workspace_bytes([(1, 3072, 768)])
    assert ma.muon_workspace_bytes([(1, 768, 3072), (1, 3072, 768)]) == one + other
    # large buckets run in phases of their own: the maximum, not the sum
    big = [(8, 8192, 28672), (16, 8192, 8192)]
    assert ma.muon_workspace_bytes(big) == max(ma.muon_workspace_bytes([s]) for s in big)
    # at most four buckets per phase
    five = ma.muon_workspace_bytes([(1, 64, 64)] * 5)
    assert five == 4 * ma.muon_workspace_bytes([(1, 64, 64)])
    assert ma.muon_workspace_bytes([(0, 10, 10)]) == 0


def test_phase_tile_promotion(lib):
    """Buckets that each pick 128-tiles alone but whose 256-tiles fill the chip together
    are planned on 256-tiles as one phase: their 640-wide Gram sides pad to 768."""
    if os.environ.get("MA_NS_TILE"):
        pytest.skip("GEMM tile forced")

    def need(K, m_pad):  # X twice, R and P, all m_pad x m_pad bf16 (m == n)
        return 4 * K * m_pad * m_pad * 2

    one = ma.muon_workspace_bytes([(40, 640, 640)])  # 240 Gram tiles at 256: too few
    assert need(40, 640) <= one < need(40, 640) + 65536
    assert ma.muon_phases([(40, 640, 640)] * 2) == (1, [0, 0])
    two = ma.muon_workspace_bytes([(40, 640, 640)] * 2)  # 480 Gram, 720 combine tiles
    assert 2 * need(40, 768) <= two < 2 * need(40, 768) + 2 * 65536
    # together still too few (240 Gram tiles): both stay on 128-tiles
    assert ma.muon_workspace_bytes([(20, 640, 640)] * 2) == 2 * ma.muon_workspace_bytes(
        [(20, 640, 640)])
    # Gram sides under 512 stay on 128-tiles however many there are
    assert ma.muon_workspace_bytes([(64, 384, 384)] * 4) == 4 * ma.muon_workspace_bytes(
        [(64, 384, 384)])


def test_phases(lib):
    import workloads
    assert ma.muon_phases([]) == (0, [])
    # the 12-layer GPT's three 768-wide buckets share one phase (on 256-tiles: each
    # alone would take 128-tiles, together they fill the chip)
    shapes = [(b.K, b.A, b.B) for b in workloads.workload(1).muon]
    assert ma.muon_phases(shapes) == (1, [0, 0, 0])
    # owner subset: every bucket needs more than the 4 GiB a phase may hold
    shapes = [(b.K, b.A, b.B) for b in workloads.workload(4).muon]
    assert ma.muon_phases(shapes) == (3, [0, 1, 2])
    # at most four buckets per phase; empty buckets belong to none
    count, of = ma.muon_phases([(1, 64, 64)] * 5 + [(0, 64, 64)])
    assert (count, of) == (2, [0, 0, 0, 0, 1, -1])
    # a change of tile closes the phase: the workspace is the maximum over phases
    shapes = [(1, 64, 64), (16, 8192, 8192), (1, 64, 64)]
    assert ma.muon_phases(shapes)[0] == 3
    assert ma.muon_workspace_bytes(shapes) == ma.muon_workspace_bytes([shapes[1]])
    with pytest.raises(ma.MuonAdamWError):
        ma.muon_phases([(1, 0, 5)])


def _hp(**kw):
    base = dict(lr=0.02, momentum=0.95, weight_decay=0.1, ns_eps=1e-7, nesterov=1,
                cautious_wd=0, ns_steps=5, scale_mode=0)
    base.update(kw)
    return _lib._MuonHParams(**base)


FAKE = 0x10000000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("case,status", [
    ("null_hp", _lib.MA_ERR_INVALID_ARG),
    ("neg_steps", _lib.MA_ERR_INVALID_ARG),
    ("big_steps", _lib.MA_ERR_INVALID_ARG),
    ("bad_scale", _lib.MA_ERR_INVALID_ARG),
    ("bad_ns_mode", _lib.MA_ERR_INVALID_ARG),
    ("small_gram_space_workspace", _lib.MA_ERR_WORKSPACE),
    ("nan_lr", _lib.MA_ERR_INVALID_ARG),
    ("neg_K", _lib.MA_ERR_INVALID_ARG),
    ("zero_A", _lib.MA_ERR_INVALID_ARG),
    ("null_param", _lib.MA_ERR_INVALID_ARG),
    ("misaligned", _lib.MA_ERR_INVALID_ARG),
    ("overlap", _lib.MA_ERR_INVALID_ARG),
    ("no_workspace", _lib.MA_ERR_WORKSPACE),
    ("small_workspace", _lib.MA_ERR_WORKSPACE),
    ("unaligned_workspace", _lib.MA_ERR_WORKSPACE),
])
def test_muon_step_rejects_before_launch(lib, case, status):
    K, A, B = 2, 64, 96
    size = K * A * 256 * 4  # room for the wider bucket of the Gram-space case
    bucket = _lib._MuonBucket(K, A, B, FAKE, FAKE + 2 * size, FAKE + 4 * size)
    hp = _hp()
    hp_ptr = ctypes.byref(hp)
    need = lib.ma_muon_workspace_bytes(ctypes.byref(bucket), 1, hp_ptr)
    ws, ws_bytes = FAKE + 8 * size, need
    if case == "null_hp":
        hp_ptr = None
    elif case == "neg_steps":
        hp.ns_steps = -1
    elif case == "big_steps":
        hp.ns_steps = _lib.MA_MAX_NS_STEPS + 1
    elif case == "bad_scale":
        hp.scale_mode = 2
    elif case == "bad_ns_mode":
        hp.ns_mode = 2
    elif case == "small_gram_space_workspace":
        # 64 x 96 is not 3.5:1, so 64 x 224 is used: its Gram-space plan needs more
        bucket.B = 224
        hp.ns_mode = 1
        ws_bytes = lib.ma_muon_workspace_bytes(ctypes.byref(bucket), 1, None)
    elif case == "nan_lr":
        hp.lr = float("nan")
    elif case == "neg_K":
        bucket.K = -1
    elif case == "zero_A":
        bucket.A = 0
    elif case == "null_param":
        bucket.param = None
    elif case == "misaligned":
        bucket.grad = FAKE + 2 * size + 2
    elif case == "overlap":
        bucket.grad = FAKE + 256   # inside the parameters
    elif case == "no_workspace":
        ws = None
    elif case == "small_workspace":
        ws_bytes = need - 1
    elif case == "unaligned_workspace":
        ws = FAKE + 8 * size + 16
    got = lib.ma_muon_step(ctypes.byref(bucket), 1, hp_ptr, ws, ws_bytes, None, None)
    assert got == status, (case, lib.ma_last_error())
    assert lib.ma_last_error()


@pytest.mark.parametrize("case", ["null_hp", "step0", "neg_n", "null_ptr", "overlap",
                                  "misaligned", "beta_one", "inf_eps"])
def test_adamw_step_rejects_before_launch(lib, case):
    n = 1000
    p, g, m, v = FAKE, FAKE + 4 * n, FAKE + 8 * n, FAKE + 12 * n
    hp = _lib._AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1,
                            decoupled=1, cautious_wd=0)
    hp_ptr = ctypes.byref(hp)
    if case == "null_hp":
        hp_ptr = None
    elif case == "step0":
        hp.step = 0
    elif case == "neg_n":
        n = -1
    elif case == "null_ptr":
        g = None
    elif case == "overlap":
        m = FAKE + 4 * n + 40
    elif case == "misaligned":
        v = FAKE + 12 * n + 1
    elif case == "beta_one":
        hp.beta2 = 1.0
    elif case == "inf_eps":
        hp.eps = float("inf")
    got = lib.ma_adamw_step(p, g, m, v, n, hp_ptr, None)
    assert got == _lib.MA_ERR_INVALID_ARG, (case, lib.ma_last_error())


def test_empty_calls_are_no_ops(lib):
    hp = _lib._AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1,
                            decoupled=1, cautious_wd=0)
    assert lib.ma_adamw_step(None, None, None, None, 0, ctypes.byref(hp), None) == 0
    mhp = _hp()
    assert lib.ma_muon_step(None, 0, ctypes.byref(mhp), None, 0, None, None) == 0
    empty = _lib._MuonBucket(0, 64, 64, None, None, None)
    route = _lib._MuonRoute()
    assert lib.ma_muon_step(ctypes.byref(empty), 1, ctypes.byref(mhp), None, 0, None,
                            ctypes.byref(route)) == 0
    assert route.m == 0


def test_optimizer_state_bytes_match_printed(golden):
    # Printed in the handbook's "The optimizer's memory budget" section: 8 bytes of
    # state per AdamW parameter, 4 per Muon parameter (4096x1024 + 1024x4096).
    torch = pytest.importorskip("torch")
    g = golden("state_bytes.txt")
    w1 = torch.zeros(4096, 1024)
    w2 = torch.zeros(1024, 4096)
    opt = ma.MuonAdamW([{"params": [w1], "kind": "muon"}, {"params": [w2], "kind": "adamw"}])
    assert (w1.numel() + w2.numel()) / 1e6 == pytest.approx(float(g["params_millions"][0]), abs=0.05)
    assert opt.state_bytes_per_param("adamw") == float(g["adamw_state_bytes_per_param"][0])
    assert opt.state_bytes_per_param("muon") == float(g["muon_state_bytes_per_param"][0])


W1 = [(48, 768, 768), (12, 768, 3072), (12, 3072, 768)]   # one 256-tile phase
SMALL = [(2, 200, 330)]                                   # one 128-tile phase
LONG = [(2, 4096, 4096)]                                  # 256-tile phase keeping X^T


def _tune_raw(lib, shapes, reps, tiles, workspace=None, nbytes=0):
    arr = (_lib._MuonBucket * max(len(shapes), 1))()
    for i, (K, A, B) in enumerate(shapes):
        arr[i] = _lib._MuonBucket(K, A, B, 0, 0, 0)
    out = None
    if tiles is not None:
        out = (ctypes.c_int32 * max(len(tiles), 1))(*tiles)
    return lib.ma_muon_tune(arr, len(shapes), None, workspace, nbytes, None, reps, out)


def test_tune_pins_available_tiles(lib):
    """Pinning (reps = 0) is host-only: every tile a phase can run is accepted, and
    pinning zeros returns the phase to the default rule."""
    if os.environ.get("MA_NS_TILE"):
        pytest.skip("GEMM tile forced")
    try:
        for t in ([256, 256, 256], [128, 128, 128], [128, 256, 128], [0, 128, 0], [256, 128, 192]):
            assert ma.muon_tune(W1, reps=0, tiles=[t]) == [t]
        assert ma.muon_tune(SMALL, reps=0, tiles=[[128, 128, 128]]) == [[128, 128, 128]]
        assert ma.muon_tune(LONG, reps=0, tiles=[[128, 128, 256]]) == [[128, 128, 256]]
        assert ma.muon_tune(W1, reps=0, tiles=[[0, 0, 0]]) == [[0, 0, 0]]
    finally:
        ma.muon_tune_reset()


@pytest.mark.parametrize("shapes,tiles", [
    (SMALL, [256, 128, 128]),     # 256-tiles on a 128-padded phase
    (SMALL, [128, 128, 256]),
    (LONG, [256, 256, 128]),      # a combine that reads X^T has no 128-tile form
    (W1, [192, 256, 256]),        # 192-row tiles are for the combine only
    (W1, [256, 192, 256]),
    (SMALL, [128, 128, 192]),
    (LONG, [256, 256, 192]),
    ([(20, 1280, 1280)], [256, 256, 192]),   # 1280 is not a multiple of 192
    (W1, [256, 256, 64]),         # not a tile
    (W1, [256, -1, 256]),
])
def test_tune_rejects_unavailable_tiles(lib, shapes, tiles):
    if os.environ.get("MA_NS_TILE"):
        pytest.skip("GEMM tile forced")
    assert _tune_raw(lib, shapes, 0, tiles) == _lib.MA_ERR_INVALID_ARG
    assert b"not available" in lib.ma_last_error()


def test_tune_rejects_bad_arguments_before_launch(lib):
    assert _tune_raw(lib, W1, 0, None) == _lib.MA_ERR_INVALID_ARG       # nothing to pin
    assert _tune_raw(lib, W1, -1, [0, 0, 0]) == _lib.MA_ERR_INVALID_ARG
    assert _tune_raw(lib, W1, 1001, None) == _lib.MA_ERR_INVALID_ARG
    assert _tune_raw(lib, [(1, 0, 5)], 0, [0, 0, 0]) == _lib.MA_ERR_INVALID_ARG
    # timing needs the workspace: checked before any launch
    assert _tune_raw(lib, W1, 3, None) == _lib.MA_ERR_WORKSPACE
    assert _tune_raw(lib, W1, 3, None, workspace=256, nbytes=1024) == _lib.MA_ERR_WORKSPACE
    with pytest.raises(ValueError):
        ma.muon_tune(W1, reps=0, tiles=[[256, 256, 256], [256, 256, 256]])
    assert _tune_raw(lib, [], 3, None) == _lib.MA_OK                   # no phase: no-op


def test_gram_space_routing_and_workspace(lib):
    """ns_mode 1 routes buckets whose long side is at least 3.5x the Gram side (either
    orientation, any Gram side) through the Gram-space iteration, in phases of their own
    (shared by Gram-space buckets of one tile), with four more m x m buffers; squarer
    buckets keep the printed iteration."""
    mlp, sq, down = (12, 768, 3072), (48, 768, 768), (12, 3072, 768)
    assert ma.muon_phases([sq, mlp, down]) == (1, [0, 0, 0])
    assert ma.muon_phases([sq, mlp, down], ns_mode=1) == (2, [0, 1, 1])
    # Gram-space buckets of one tile share a phase whatever their fp16 scales (the
    # products apply them per matrix)
    assert ma.muon_phases([mlp, (4, 512, 2048), (12, 1024, 4096)], ns_mode=1)[0] == 1
    for (A, B), gs in [((768, 3072), 1), ((3072, 768), 1), ((1024, 2048), 0), ((1024, 3072), 0),
                       ((1024, 3584), 1), ((1024, 3583), 0), ((3584, 1024), 1),
                       ((2048, 4096), 0), ((2048, 8192), 1), ((8192, 28672), 1),
                       ((28672, 8192), 1), ((2560, 5120), 0), ((64, 128), 0), ((64, 224), 1),
                       ((64, 223), 0), ((1, 7), 1), ((2, 7), 1), ((2, 6), 0), ((512, 2048), 1),
                       ((2048, 512), 1), ((768, 768), 0)]:
        assert ma.muon_route_of(A, B, 5, ns_mode=1).ns_mode_run == gs, (A, B)
        assert ma.muon_route_of(A, B, 5, ns_mode=0).ns_mode_run == 0
        assert ma.muon_route_of(A, B, 0, ns_mode=1).ns_mode_run == 0
    m_pad = 768 if not os.environ.get("MA_NS_TILE") else None
    extra = ma.muon_workspace_bytes([mlp], ns_mode=1) - ma.muon_workspace_bytes([mlp])
    if m_pad:
        # R2, Q[0], Q[1], T, and 3 K floats of per-matrix norms and factors (256-aligned)
        assert extra == 4 * 12 * m_pad * m_pad * 2 + 256
    assert ma.muon_workspace_bytes([sq], ns_mode=1) == ma.muon_workspace_bytes([sq])
    assert ma.muon_workspace_bytes([(3, 100, 199)], ns_mode=1) == ma.muon_workspace_bytes(
        [(3, 100, 199)])
    # ma_newton_schulz's workspace serves either mode
    assert ma.newton_schulz_workspace_bytes(12, 768, 3072) == ma.muon_workspace_bytes(
        [mlp], ns_mode=1)


@pytest.mark.parametrize("case", ["null_segs", "neg_count", "neg_n", "null_ptr", "misaligned",
                                  "overlap_across", "overlap_within", "bad_hp"])
def test_adamw_step_multi_rejects_before_launch(lib, case):
    n = 1000
    segs = (_lib._AdamWSegment * 2)()
    for i in range(2):
        base = FAKE + i * 16 * n
        segs[i] = _lib._AdamWSegment(base, base + 4 * n, base + 8 * n, base + 12 * n, n)
    hp = _lib._AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1,
                            decoupled=1, cautious_wd=0)
    arr, count = segs, 2
    if case == "null_segs":
        arr = None
    elif case == "neg_count":
        count = -1
    elif case == "neg_n":
        segs[1].n = -5
    elif case == "null_ptr":
        segs[1].exp_avg = None
    elif case == "misaligned":
        segs[0].grad = FAKE + 4 * n + 2
    elif case == "overlap_across":
        segs[1].param = FAKE + 8 * n + 400          # inside segment 0's exp_avg
    elif case == "overlap_within":
        segs[0].exp_avg_sq = FAKE + 8 * n + 4        # overlaps its own exp_avg
    elif case == "bad_hp":
        hp.beta2 = 1.0
    got = lib.ma_adamw_step_multi(arr, count, ctypes.byref(hp), None)
    assert got == _lib.MA_ERR_INVALID_ARG, (case, lib.ma_last_error())
    assert lib.ma_last_error()


def test_adamw_step_multi_empty_calls_are_no_ops(lib):
    """No segments, or only empty ones: nothing to launch, MA_OK (no GPU needed)."""
    hp = _lib._AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1,
                            decoupled=1, cautious_wd=0)
    assert lib.ma_adamw_step_multi(None, 0, ctypes.byref(hp), None) == _lib.MA_OK
    segs = (_lib._AdamWSegment * 3)()
    for i in range(3):
        segs[i] = _lib._AdamWSegment(None, None, None, None, 0)
    assert lib.ma_adamw_step_multi(segs, 3, ctypes.byref(hp), None) == _lib.MA_OK
    ma.adamw_step_multi([], step=1, lr=1e-3)


def test_adamw_step_multi_overlap_sweep_matches_brute_force(lib):
    """Random layouts of 3-12 segments packed into a small address window: wherever a
    brute-force pairwise check finds a written range (param, exp_avg, exp_avg_sq) meeting
    any other range, the call is rejected before launch.  Only such layouts are tried,
    so nothing here can reach a kernel."""
    rng = np.random.default_rng(21)
    hp = _lib._AdamWHParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=1,
                            decoupled=1, cautious_wd=0)
    tried = 0
    while tried < 60:
        k = int(rng.integers(3, 13))
        segs = (_lib._AdamWSegment * k)()
        spans = []
        for i in range(k):
            n = int(rng.integers(1, 64))
            ptrs = [FAKE + 4 * int(rng.integers(0, 4000)) for _ in range(4)]
            segs[i] = _lib._AdamWSegment(*ptrs, n)
            for j, q in enumerate(ptrs):
                spans.append((q, q + 4 * n, j != 1))     # grad (index 1) is read only
        clash = any((a[2] or b[2]) and a[0] < b[1] and b[0] < a[1]
                    for x, a in enumerate(spans) for b in spans[x + 1:])
        if not clash:
            continue
        tried += 1
        assert lib.ma_adamw_step_multi(segs, k, ctypes.byref(hp), None) == _lib.MA_ERR_INVALID_ARG
        assert b"overlap" in lib.ma_last_error()


def test_stream_probe_rejects_before_launch(lib):
    P = ctypes.c_void_p
    base = 1 << 40
    n = 4096
    ins = (P * 4)(base, base + 1 * 65536, base + 2 * 65536, base + 3 * 65536)
    outs = (P * 3)(base + 4 * 65536, base + 5 * 65536, base + 6 * 65536)
    assert lib.ma_stream_probe(ins, 0, outs, 1, n, None) == _lib.MA_ERR_INVALID_ARG
    assert lib.ma_stream_probe(ins, 5, outs, 1, n, None) == _lib.MA_ERR_INVALID_ARG
    assert lib.ma_stream_probe(ins, 2, outs, 4, n, None) == _lib.MA_ERR_INVALID_ARG
    assert lib.ma_stream_probe(ins, 2, outs, 1, n + 2, None) == _lib.MA_ERR_INVALID_ARG
    assert lib.ma_stream_probe(ins, 2, outs, 1, 0, None) == _lib.MA_OK
    bad = (P * 4)(base + 4, base + 65536, 0, 0)   # misaligned
    assert lib.ma_stream_probe(bad, 2, outs, 1, n, None) == _lib.MA_ERR_INVALID_ARG
    part = (P * 3)(base + 8192, 0, 0)              # overlaps input 0 without being it
    assert lib.ma_stream_probe(ins, 2, part, 1, n, None) == _lib.MA_ERR_INVALID_ARG
    two = (P * 4)(base, base + 8192, 0, 0)         # two overlapping inputs
    assert lib.ma_stream_probe(two, 2, outs, 1, n, None) == _lib.MA_ERR_INVALID_ARG


def test_mfma_probe_rejects_before_launch(lib):
    base = 1 << 40
    assert lib.ma_mfma_probe(None, 1, 1, base, None, None) == _lib.MA_ERR_INVALID_ARG
    assert lib.ma_mfma_probe(base + 8, 1, 1, base + 65536, None, None) == _lib.MA_ERR_INVALID_ARG
    assert lib.ma_mfma_probe(base, 1, 1, None, None, None) == _lib.MA_ERR_INVALID_ARG
    assert lib.ma_mfma_probe(base, 1, 1, base + 65538, None, None) == _lib.MA_ERR_INVALID_ARG
    assert lib.ma_mfma_probe(base, 1, 1, base + 65536, base + 4, None) == _lib.MA_ERR_INVALID_ARG
    for blocks, iters in ((0, 1), (65536, 1), (1, 0), (1, (1 << 22) + 1), (-1, 5)):
        assert lib.ma_mfma_probe(base, blocks, iters, base + 65536, None, None) == \
            _lib.MA_ERR_INVALID_ARG
    assert b"outside" in lib.ma_last_error()

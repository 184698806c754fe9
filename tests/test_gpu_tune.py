"""Per-shape GEMM tiles (ma_muon_tune): every tile a phase can run accumulates each
output over the same k order, so a Muon step with any pinned or tuned choice must be
bitwise identical to the step with the default rule (whose parity against the oracle
the other GPU tests establish)."""
import itertools

import numpy as np
import pytest
import torch

import adamw_optimizer_step_muon_amd as ma
import oracle
from parity import MUON_RTOL, rel_fro

pytestmark = pytest.mark.gpu

CASES = {
    # the 12-layer GPT's buckets: one 256-tile phase whose combine reads X
    "gpt12": [(48, 768, 768), (12, 768, 3072), (12, 3072, 768)],
    # 640-wide Gram sides promoted to 256-tiles together: ragged tile edges, transposed
    "promoted": [(24, 640, 640), (12, 640, 2560), (12, 2560, 640)],
    # a Gram side above 2048: the combine reads the stored X^T (256-tiles only)
    "keeps_xt": [(2, 4096, 4096)],
    # a 1280-wide Gram side (not a multiple of 192): 256- and 128-tiles only
    "gpt20": [(20, 1280, 1280), (5, 1280, 5120), (5, 5120, 1280)],
}


def _state(shapes, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    out = []
    for K, A, B in shapes:
        p = torch.randn((K, A, B), generator=gen, device="cuda")
        g = 0.02 * torch.randn((K, A, B), generator=gen, device="cuda")
        m = 0.01 * torch.randn((K, A, B), generator=gen, device="cuda")
        out.append((p, g, m))
    return out


def _step(state, ws):
    bks = [(p.clone(), g, m.clone()) for p, g, m in state]
    ma.muon_step(bks, lr=0.02, momentum=0.95, weight_decay=0.1, workspace=ws)
    torch.cuda.synchronize()
    return bks


def _same(a, b):
    return all(torch.equal(x[0], y[0]) and torch.equal(x[2], y[2]) for x, y in zip(a, b))


def _oracle_errors(state, after):
    """The first matrix of each bucket after one step against the oracle (the state's
    momentum is nonzero, so this also covers M <- mu M + G with a previous M)."""
    errs = []
    keep = 1.0 - np.float32(0.02) * np.float32(0.1)
    for (p, g, m), (p1, _, _) in zip(state, after):
        p0 = p[0].cpu().numpy().astype(np.float64)
        ref = oracle.muon_step(p0, g[0].cpu().numpy(), m[0].cpu().numpy(), lr=float(np.float32(0.02)),
                               mu=float(np.float32(0.95)), weight_decay=float(np.float32(0.1)))
        errs.append(rel_fro(p0 * keep - p1[0].cpu().numpy(), p0 * keep - ref.param))
    return errs


@pytest.mark.parametrize("case", sorted(CASES))
def test_pinned_tiles_are_bitwise_identical(case):
    shapes = CASES[case]
    nph, _ = ma.muon_phases(shapes)
    assert nph == 1
    state = _state(shapes, 7)
    ws = torch.empty(ma.muon_workspace_bytes(shapes), dtype=torch.uint8, device="cuda")
    ma.muon_tune_reset()
    try:
        ref = _step(state, ws)
        errs = _oracle_errors(state, ref)
        print(f"{case}: default tiles, errors against the oracle {errs}", flush=True)
        assert max(errs) <= MUON_RTOL
        # the combine of Gram sides padded to 768 also has 192-row tiles
        combine = {"keeps_xt": (256,), "gpt20": (256, 128)}.get(case, (256, 128, 192))
        options = [(256, 128), (256, 128), combine]
        for tiles in itertools.product(*options):
            print(f"{case}: pinned {tiles}", flush=True)
            assert ma.muon_tune(shapes, reps=0, tiles=[list(tiles)]) == [list(tiles)]
            got = _step(state, ws)
            # bitwise the default's result, and (so) within tolerance of the oracle
            assert _same(got, ref), tiles
            assert max(_oracle_errors(state[:1], got[:1])) <= MUON_RTOL, tiles
    finally:
        ma.muon_tune_reset()


@pytest.mark.parametrize("case", ["gpt12", "keeps_xt"])
def test_tuned_tiles_keep_results(case):
    shapes = CASES[case]
    state = _state(shapes, 8)
    ws = torch.empty(ma.muon_workspace_bytes(shapes), dtype=torch.uint8, device="cuda")
    ma.muon_tune_reset()
    try:
        ref = _step(state, ws)
        tiles = ma.muon_tune(shapes, reps=2, workspace=ws)
        print(f"{case}: tuned {tiles}", flush=True)
        assert len(tiles) == 1 and all(t in (128, 256) for t in tiles[0][:2])
        assert tiles[0][2] in (128, 192, 256)
        if case == "keeps_xt":
            assert tiles[0][2] == 256
        assert _same(_step(state, ws), ref)
    finally:
        ma.muon_tune_reset()


@pytest.mark.parametrize("case", ["gpt12", "keeps_xt"])
def test_searched_configurations_keep_results(case):
    """The full search (tile, pipeline, band width, spreading): the configuration it keeps
    gives the default's result bit for bit, and so meets the oracle."""
    shapes = CASES[case]
    state = _state(shapes, 9)
    ws = torch.empty(ma.muon_workspace_bytes(shapes), dtype=torch.uint8, device="cuda")
    ma.muon_tune_reset()
    try:
        ref = _step(state, ws)
        cfg = ma.muon_tune_configs(shapes, reps=2, workspace=ws)
        print(f"{case}: searched {cfg}", flush=True)
        assert len(cfg) == 1 and all(c["tile"] in (128, 192, 256) for c in cfg[0])
        got = _step(state, ws)
        assert _same(got, ref)
        assert max(_oracle_errors(state, got)) <= MUON_RTOL
    finally:
        ma.muon_tune_reset()


@pytest.mark.parametrize("config", [{"tile": 256, "pipeline": 2}, {"band": 2}, {"band": 8},
                                    {"spread": 0}, {"xcd": 1}, {"xcd": 2}, {"xcd": 3}])
def test_pinned_configurations_are_bitwise_identical(config):
    """Each dimension pinned on its own for every product that accepts it (the 4096-wide
    phase keeps X^T, so its combine has a pipeline choice too)."""
    shapes = CASES["keeps_xt"]
    state = _state(shapes, 10)
    ws = torch.empty(ma.muon_workspace_bytes(shapes), dtype=torch.uint8, device="cuda")
    ma.muon_tune_reset()
    try:
        ref = _step(state, ws)
        ma.muon_tune_configs(shapes, reps=0, configs=[[config, config, config]])
        got = _step(state, ws)
        assert _same(got, ref), config
    finally:
        ma.muon_tune_reset()


GS_SHAPES = [(8, 2048, 8192), (8, 8192, 2048)]  # one 256-tile Gram-space phase


def _step_gs(state, ws):
    bks = [(p.clone(), g, m.clone()) for p, g, m in state]
    routes = ma.muon_step(bks, lr=0.02, momentum=0.95, weight_decay=0.1, ns_mode=1, workspace=ws)
    assert [r.ns_mode_run for r in routes] == [1, 1]
    torch.cuda.synchronize()
    return bks


@pytest.mark.parametrize("config", [{"tile": 128}, {"tile": 256, "pipeline": 2},
                                    {"band": 2}, {"band": 8}, {"spread": 0}, {"xcd": 2},
                                    {"xcd": 3}])
def test_gram_space_configurations_are_bitwise_identical(config):
    """The fp16 Gram-space launches under each pinned configuration (the fp16 kernels run
    the default pipeline, so a pinned second pipeline runs as the default) and under the
    searched one: bitwise the default's."""
    shapes = GS_SHAPES
    assert ma.muon_phases(shapes, ns_mode=1) == (1, [0, 0])
    state = _state(shapes, 11)
    ws = torch.empty(ma.muon_workspace_bytes(shapes, ns_mode=1), dtype=torch.uint8, device="cuda")
    ma.muon_tune_reset()
    try:
        ref = _step_gs(state, ws)
        # (the combine of a phase that reads X has no pipeline choice)
        comb = {"tile": 256} if "pipeline" in config else config
        ma.muon_tune_configs(shapes, reps=0, configs=[[config, config, comb]], ns_mode=1)
        assert _same(_step_gs(state, ws), ref), config
        ma.muon_tune_reset()
        cfg = ma.muon_tune_configs(shapes, reps=2, workspace=ws, ns_mode=1)
        print(f"gram-space: searched {cfg}", flush=True)
        assert _same(_step_gs(state, ws), ref)
    finally:
        ma.muon_tune_reset()


@pytest.mark.parametrize("shape", [(43, 768, 1024), (8, 2048, 2048)])
@pytest.mark.parametrize("config", [{"tile": 128}, {"tile": 256, "spread": 0},
                                    {"tile": 256, "spread": 1}])
def test_repeated_steps_are_bitwise_identical(shape, config):
    """The same step three times on the same inputs, every product on one tile shape:
    bitwise identical results.  Each wave finishes its LDS reads of an operand stage
    before the barrier after which the other waves load later stages into those slots;
    a read left behind that barrier makes the results change from run to run (where the
    reference comparisons, with their tolerance, may not notice)."""
    shapes = [shape]
    state = _state(shapes, 12)
    ws = torch.empty(ma.muon_workspace_bytes(shapes), dtype=torch.uint8, device="cuda")
    ma.muon_tune_reset()
    try:
        ma.muon_tune_configs(shapes, reps=0, configs=[[config, config, config]])
        ref = _step(state, ws)
        for rep in range(2):
            assert _same(_step(state, ws), ref), (config, rep)
    finally:
        ma.muon_tune_reset()


@pytest.mark.parametrize("config", [{"tile": 128}, {"tile": 256, "spread": 0},
                                    {"tile": 256, "spread": 1}])
def test_repeated_gram_space_steps_are_bitwise_identical(config):
    """The same repetition on the fp16 Gram-space route (ns_mode 1), whose symmetric
    products and polynomials run the same main loop on fp16 operands."""
    shapes = GS_SHAPES
    state = _state(shapes, 13)
    ws = torch.empty(ma.muon_workspace_bytes(shapes, ns_mode=1), dtype=torch.uint8, device="cuda")
    ma.muon_tune_reset()
    try:
        comb = {"tile": 256} if config["tile"] == 256 else config
        ma.muon_tune_configs(shapes, reps=0, configs=[[config, config, comb]], ns_mode=1)
        ref = _step_gs(state, ws)
        for rep in range(2):
            assert _same(_step_gs(state, ws), ref), (config, rep)
    finally:
        ma.muon_tune_reset()


@pytest.mark.parametrize("case", ["gpt12", "gpt20", "promoted"])
def test_shared_xcd_order_is_bitwise_identical(case):
    """Every product pinned to the order in which the eight XCDs share each matrix (the
    default only for matrices of at least 512 tiles), on phases whose per-matrix tile
    counts are not multiples of 8, so some XCDs run padding blocks: bitwise the default's
    result, and within tolerance of the oracle."""
    shapes = CASES[case]
    state = _state(shapes, 14)
    ws = torch.empty(ma.muon_workspace_bytes(shapes), dtype=torch.uint8, device="cuda")
    ma.muon_tune_reset()
    try:
        ref = _step(state, ws)
        shared = {"xcd": 3}
        ma.muon_tune_configs(shapes, reps=0, configs=[[shared, shared, shared]])
        got = _step(state, ws)
        assert _same(got, ref)
        assert max(_oracle_errors(state[:1], got[:1])) <= MUON_RTOL
    finally:
        ma.muon_tune_reset()

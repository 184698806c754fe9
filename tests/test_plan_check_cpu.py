"""Every launch a step would make, checked on the host (ma_muon_check_plan, no GPU).

The library replays ma_muon_step (and ma_newton_schulz) with its launchers recording
instead of launching; each Newton-Schulz GEMM block is mapped to its output tile by the
kernel's own block-to-tile function, and every operand read and result write of every
block must stay inside the buffer its argument addresses, with each output tile of a
launch computed exactly once.  Covered: the five workloads' bucket lists in both
iteration modes, every tile a phase can be pinned to, the environment tile overrides,
and a spread of ragged shapes.  A CPU mutation check (a wrong row stride, overlapping
workspace offsets, a wrong block offset in the shared XCD order) showed the check fails
on such mistakes.
"""
import itertools
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads
from conftest import ROOT

ma = pytest.importorskip("adamw_optimizer_step_muon_amd")
from adamw_optimizer_step_muon_amd import _lib  # noqa: E402

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")


def _shapes(i):
    return [(b.K, b.A, b.B) for b in workloads.workload(i).muon]


@pytest.mark.parametrize("index", range(5))
@pytest.mark.parametrize("ns_mode", [0, 1])
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_workload_step_plans(index, ns_mode, steps):
    shapes = _shapes(index)
    rep = ma.muon_check_plan(shapes, ns_mode=ns_mode, ns_steps=steps)
    nph = ma.muon_phases(shapes, ns_mode)[0]
    assert rep["launches"] >= 4 * len(shapes)
    if steps and ns_mode == 0:
        # each tile of a symmetric product is one block: 3 launches per step per phase
        assert rep["gemm_blocks"] == rep["gemm_tiles"] > 0
        assert rep["launches"] == 4 * len(shapes) + 3 * steps * nph


def _pin_options(shapes, ns_mode):
    """Every (gram, poly, combine) tile triple the library accepts for each phase."""
    nph = ma.muon_phases(shapes, ns_mode)[0]
    per_phase = []
    for ph in range(nph):
        ok = []
        for trip in itertools.product((128, 256), (128, 256), (128, 192, 256)):
            tiles = [[0, 0, 0] for _ in range(nph)]
            tiles[ph] = list(trip)
            try:
                ma.muon_tune(shapes, reps=0, tiles=tiles, ns_mode=ns_mode)
                ok.append(trip)
            except _lib.MuonAdamWError:
                pass
        per_phase.append(ok)
    ma.muon_tune_reset()
    return per_phase


@pytest.mark.parametrize("index", range(5))
@pytest.mark.parametrize("ns_mode", [0, 1])
def test_workload_plans_under_every_pinned_tile(index, ns_mode):
    shapes = _shapes(index)
    options = _pin_options(shapes, ns_mode)
    assert all(options)
    try:
        for ph, trips in enumerate(options):
            for trip in trips:
                tiles = [[0, 0, 0] for _ in options]
                tiles[ph] = list(trip)
                ma.muon_tune(shapes, reps=0, tiles=tiles, ns_mode=ns_mode)
                ma.muon_check_plan(shapes, ns_mode=ns_mode)
    finally:
        ma.muon_tune_reset()


RAGGED = [(1, 1, 1), (1, 1, 7), (2, 7, 1), (3, 300, 520), (2, 520, 300), (1, 257, 129),
          (4, 96, 96), (43, 768, 1024), (6, 4096, 2304), (6, 2304, 4096), (24, 640, 640),
          (12, 640, 2560), (12, 2560, 640), (1, 2049, 100), (5, 192, 192), (2, 129, 4100)]


@pytest.mark.parametrize("ns_mode", [0, 1])
def test_ragged_bucket_lists(ns_mode):
    ma.muon_check_plan(RAGGED, ns_mode=ns_mode)
    for s in RAGGED:
        ma.muon_check_plan([s], ns_mode=ns_mode)
        ma.muon_check_plan([s], what=1, ns_mode=ns_mode)
        ma.muon_check_plan([s], what=1, ns_mode=ns_mode, ns_steps=0)


def test_random_shapes():
    rng = np.random.default_rng(5)
    for _ in range(60):
        n = int(rng.integers(1, 6))
        shapes = [(int(rng.integers(1, 9)), int(rng.integers(1, 3000)), int(rng.integers(1, 3000)))
                  for _ in range(n)]
        for ns_mode in (0, 1):
            ma.muon_check_plan(shapes, ns_mode=ns_mode, ns_steps=int(rng.integers(0, 4)))


_SHARED_SCRIPT = """
import numpy as np
import adamw_optimizer_step_muon_amd as ma
rng = np.random.default_rng(11)
for _ in range(80):
    n = int(rng.integers(1, 5))
    shapes = [(int(rng.integers(1, 12)), int(rng.integers(1, 2600)), int(rng.integers(1, 2600)))
              for _ in range(n)]
    for mode in (0, 1):
        ma.muon_check_plan(shapes, ns_mode=mode, ns_steps=int(rng.integers(1, 3)))
print("ok")
"""


def test_random_shapes_under_the_shared_xcd_order():
    """Random bucket lists with every launch in the order where the eight XCDs share
    each matrix (MA_NS_XCD 2; by default only matrices of 512 tiles or more take it):
    tile counts per matrix that are not multiples of 8, and batches that do not fill the
    last round, each output tile still computed by exactly one block."""
    r = subprocess.run([sys.executable, "-c", _SHARED_SCRIPT], cwd=ROOT, capture_output=True,
                       text=True, env={**os.environ, "MA_NS_XCD": "2"}, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]


_ENV_SCRIPT = """
import sys, workloads
import adamw_optimizer_step_muon_amd as ma
for i in range(5):
    shapes = [(b.K, b.A, b.B) for b in workloads.workload(i).muon]
    for mode in (0, 1):
        ma.muon_check_plan(shapes, ns_mode=mode)
for s in %r:
    ma.muon_check_plan([s]); ma.muon_check_plan([s], what=1)
print("ok")
""" % (RAGGED,)


@pytest.mark.parametrize("env", [{"MA_NS_TILE": "128"}, {"MA_NS_TILE": "256"}, {"MA_NS_BIG": "1"},
                                 {"MA_NS_BAND_COMBINE": "3", "MA_NS_BAND_TRI": "0"},
                                 {"MA_NS_XCD": "0", "MA_NS_BAND_TRI": "7"},
                                 {"MA_NS_XCD": "1"}, {"MA_NS_XCD": "2", "MA_NS_BAND_COMBINE": "5"}])
def test_environment_tile_overrides(env):
    """The tuning overrides are read once per process: each runs in a child process
    (MA_NS_XCD 2 puts every launch, of any tile count, in the order where the XCDs share
    each matrix)."""
    r = subprocess.run([sys.executable, "-c", _ENV_SCRIPT], cwd=ROOT, capture_output=True,
                       text=True, env={**os.environ, **env}, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stderr[-2000:]


CONFIGS = [
    {"tile": 256, "pipeline": 2}, {"tile": 256, "pipeline": 1, "band": 2},
    {"tile": 256, "band": 8, "spread": 0}, {"tile": 128, "band": 1}, {"band": 16},
    {"spread": 1}, {"tile": 192, "band": 3, "spread": 0}, {"xcd": 2}, {"xcd": 1, "band": 2},
    {"xcd": 3}, {"xcd": 3, "band": 2, "tile": 128},
]


@pytest.mark.parametrize("index", range(5))
def test_workload_plans_under_pinned_configurations(index):
    """Every configuration dimension the tuner searches (tile, pipeline, band width,
    spreading), pinned per product wherever the phase accepts it."""
    shapes = _shapes(index)
    nph = ma.muon_phases(shapes)[0]
    tried = 0
    try:
        for ph in range(nph):
            for q in range(3):
                for c in CONFIGS:
                    cfg = [[{}, {}, {}] for _ in range(nph)]
                    cfg[ph][q] = c
                    try:
                        ma.muon_tune_configs(shapes, reps=0, configs=cfg)
                    except _lib.MuonAdamWError as e:
                        assert e.status == _lib.MA_ERR_INVALID_ARG
                        continue
                    ma.muon_check_plan(shapes)
                    tried += 1
    finally:
        ma.muon_tune_reset()
    assert tried >= 3 * nph


def test_configuration_pins_are_validated():
    shapes = [(48, 768, 768), (12, 768, 3072), (12, 3072, 768)]
    bad = [{"tile": 128, "pipeline": 2}, {"pipeline": 3}, {"band": 65}, {"spread": 2},
           {"tile": 512}, {"xcd": 4}, {"xcd": -1}]
    for c in bad:
        with pytest.raises(_lib.MuonAdamWError):
            ma.muon_tune_configs(shapes, reps=0, configs=[[c, {}, {}]])
    # the combine of this phase reads X (no X^T): no pipeline choice there
    with pytest.raises(_lib.MuonAdamWError):
        ma.muon_tune_configs(shapes, reps=0, configs=[[{}, {}, {"pipeline": 2}]])
    got = ma.muon_tune_configs(shapes, reps=0, configs=[[{"pipeline": 2}, {}, {"tile": 192}]])
    assert got[0][0]["pipeline"] == 2 and got[0][2]["tile"] == 192
    ma.muon_tune_reset()

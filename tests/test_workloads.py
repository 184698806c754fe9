"""The seeded input generators: determinism, shapes and the recipes' statistics."""
import math

import numpy as np

import workloads
from workloads import gen


def test_workload_sizes():
    wl = workloads.WORKLOADS
    assert [b.K * b.A * b.B for b in wl[0].muon] == [8192, 8192]
    assert wl[1].muon_numel == 84_934_656 and wl[1].adamw_numel == 100_682_496
    assert wl[2].muon_numel == 393_216_000 and wl[2].adamw_numel == 167_824_640
    assert wl[3].muon_numel == 1_056_964_608 and wl[3].adamw_numel == 524_388_352
    assert wl[4].muon_numel == 4_831_838_208 and wl[4].adamw_numel == 1_050_673_152
    assert wl[3].muon_hp.cautious_wd and not wl[1].muon_hp.cautious_wd


def test_streams_are_deterministic_and_independent():
    wl = workloads.workload(0)
    a = gen.np_muon_bucket_grads(wl, 0, 1)
    b = gen.np_muon_bucket_grads(wl, 0, 1)
    c = gen.np_muon_bucket_grads(wl, 0, 2)
    assert a.dtype == np.float32 and a.shape == (1, 64, 128)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    flat = gen.np_adamw_flat_grads(wl, 1)
    assert flat.shape == (4096 + 512 * 64,)
    # any tensor can be regenerated alone
    j, lo, hi = list(gen.adamw_offsets(wl))[1]
    alone = gen.np_grad(wl.seed, 1, gen.adamw_index(wl, j), (512, 64), wl.adamw_grad, gen.ADAMW_SIGMA)
    assert np.array_equal(flat[lo:hi], alone.reshape(-1))


def test_lowrank_energy_share():
    g = gen.np_grad(1, 1, 0, (384, 512), "lowrank", 1e-3).astype(np.float64)
    s = np.linalg.svd(g, compute_uv=False)
    top = (s[:8] ** 2).sum() / (s ** 2).sum()
    # 30 % low-rank plus the noise's own share of the top 8 directions
    assert 0.30 < top < 0.40


def test_rowlognormal_scales():
    g = gen.np_grad(0, 1, 0, (4000, 256), "rowlognormal", 0.02).astype(np.float64)
    row_rms = np.sqrt((g ** 2).mean(axis=1))
    log_scale = np.log(row_rms / 0.02)
    assert abs(log_scale.std() - 1.0) < 0.06


def test_conditioned_replica_condition_number():
    # checked on a 1024 x 3584 replica of the 8192 x 28672 shape
    g = gen.np_grad(4, 1, 0, (1024, 3584), "conditioned", 0.02).astype(np.float64)
    s = np.linalg.svd(g, compute_uv=False)
    assert 3.0 < math.log10(s[0] / s[-1]) < 5.0

"""The matrix-core reference loop (ma_mfma_probe) computes what its header states, so the
rate it reports is that of real MFMAs on the given operands."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
ma = pytest.importorskip("adamw_optimizer_step_muon_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _expected_wave_sum(ops: np.ndarray):
    """Sum of every accumulator element of one wave after one round, and the sum of the
    elements' magnitudes, in fp64.  Fragment f of lane l is ops[f, l, :]; for the
    32 x 32 x 16 MFMA the A fragment of lane l holds row l % 32 at k = 8 (l // 32) + 0..7 and
    the B fragment column l % 32 at the same k: D = A B summed over its entries is
    sum_k colsum(A)[k] rowsum(B)[k]."""
    total, mag = 0.0, 0.0
    for r in range(8):
        fa, fb = ops[2 * r], ops[2 * ((r + 3) % 8) + 1]
        A = np.zeros((32, 16))
        B = np.zeros((16, 32))
        for l in range(64):
            h = l // 32
            A[l % 32, 8 * h:8 * h + 8] = fa[l]
            B[8 * h:8 * h + 8, l % 32] = fb[l]
        D = A @ B
        total += D.sum()
        mag += np.abs(D).sum()
    return total, mag


@pytest.mark.parametrize("iters", [1, 3])
def test_mfma_probe_sums(iters):
    g = torch.Generator(device="cpu").manual_seed(11)
    ops32 = torch.randn(16, 64, 8, generator=g)
    ops = ops32.to(torch.bfloat16)
    blocks = 3
    out = torch.full((blocks * 512,), float("nan"), device=DEV)
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=DEV)
    ma.mfma_probe(ops.reshape(-1).to(DEV), out, iters, clocks=clocks)
    torch.cuda.synchronize()
    exp, mag = _expected_wave_sum(ops.float().numpy().astype(np.float64))
    per_wave = out.double().cpu().numpy().reshape(blocks * 8, 64).sum(axis=1)
    assert np.all(np.abs(per_wave - iters * exp) <= 1e-5 * iters * mag), (per_wave[:4], exp)
    c = clocks.cpu().numpy().reshape(blocks, 2)
    assert np.all(c > 0)


def test_mfma_probe_reports_a_clock():
    """A launch long enough to read the clock: shader-clock cycles over 100 MHz ticks lands
    in the part's clock range, and the rate stays below the 2.5 PFLOP/s rating."""
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    ops = torch.randn(16 * 64 * 8, device=DEV).to(torch.bfloat16)
    out = torch.empty(blocks * 512, device=DEV)
    clocks = torch.zeros(2 * blocks, dtype=torch.int64, device=DEV)
    iters = 20000
    ma.mfma_probe(ops, out, iters, clocks=clocks)          # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ma.mfma_probe(ops, out, iters, clocks=clocks)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    c = clocks.double().cpu().numpy().reshape(blocks, 2)
    ghz = c[:, 0].sum() / c[:, 1].sum() * 0.1
    tflops = ma.mfma_probe_flops(blocks, iters) / (ms * 1e-3) / 1e12
    print(f"mfma probe: {tflops:.0f} TFLOP/s at {ghz:.3f} GHz")
    assert 0.5 < ghz < 3.0
    assert 100 < tflops < 2600
    assert torch.isfinite(out).all()


def test_mfma_probe_rejects_bad_tensors():
    ops = torch.zeros(100, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(512, device=DEV)
    with pytest.raises(ValueError):
        ma.mfma_probe(ops, out, 1)
    ops = torch.zeros(8192, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        ma.mfma_probe(ops, torch.empty(500, device=DEV), 1)
    with pytest.raises(ValueError):
        ma.mfma_probe(ops, out, 1, clocks=torch.zeros(3, dtype=torch.int64, device=DEV))
    with pytest.raises(ma.MuonAdamWError):
        ma.mfma_probe(ops, out, 0)

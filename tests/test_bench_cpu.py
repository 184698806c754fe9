"""The benchmark's CPU-baseline leg (the fp64 oracle timed on a bounded sample)."""
import bench
import workloads


def test_cpu_baseline_samples_every_bucket_within_budget():
    out = bench.cpu_baseline(workloads.workload(0), budget_s=2.0)
    assert out["kind"] == "oracle" and out["unit"] == "ms"
    assert out["value"] > 0 and out["cores"] >= 1
    assert "1 of 1 64x128" in out["sample"] and "1 of 1 128x64" in out["sample"]
    assert "36864 of 36864 elements" in out["sample"]


def test_cpu_baseline_extrapolates_unsampled_buckets():
    # a zero budget still times one matrix (the cheapest bucket first); the other bucket
    # is scaled by the oracle's cost model
    out = bench.cpu_baseline(workloads.workload(0), budget_s=0.0)
    assert out["value"] > 0
    assert "1 of 1 64x128" in out["sample"]
    assert "0 of 1 128x64 (extrapolated by the oracle's cost model" in out["sample"]


def test_oracle_cost_orders_the_owner_subset_buckets():
    """The square 8192 x 8192 bucket is the cheapest to sample; the two rectangular
    buckets (one the other's transpose) cost the same."""
    b = workloads.workload(4).muon
    assert bench.oracle_cost(b[2]) < bench.oracle_cost(b[0]) == bench.oracle_cost(b[1])

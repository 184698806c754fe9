"""Seeded synthetic workloads shared by the tests, the oracle comparisons and
the benchmark.  Input generation only; no optimizer arithmetic lives here."""
from .configs import (QUINTIC, WORKLOADS, AdamWHP, AdamWTensor, MuonBucket, MuonHP,
                      Workload, workload)

__all__ = ["QUINTIC", "WORKLOADS", "AdamWHP", "AdamWTensor", "MuonBucket", "MuonHP",
           "Workload", "workload"]

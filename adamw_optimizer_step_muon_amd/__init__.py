"""Hybrid Muon + AdamW optimizer step for MI355X (gfx950).

The compute runs in libmuonadamw.so (hand-written HIP kernels behind the C ABI of
include/muon_adamw.h); this package is its thin Python binding plus the MuonAdamW
parameter-group wrapper.  PyTorch supplies device memory and streams only.
"""
from ._lib import (LIB_PATH, MFMA_PROBE_OPERAND_VALUES, MFMA_PROBE_THREADS, MuonAdamWError, Route, abi_version, adamw_step, adamw_step_multi, load,
                   mfma_probe, mfma_probe_flops, muon_check_plan, muon_ns_time, muon_phases, muon_route_of, muon_step,
                   muon_static_init, muon_step_static, muon_tune, muon_tune_configs,
                   muon_tune_reset,
                   muon_workspace_bytes, newton_schulz, newton_schulz_workspace_bytes,
                   stream_probe)
from .optim import MuonAdamW

__all__ = ["LIB_PATH", "MFMA_PROBE_OPERAND_VALUES", "MFMA_PROBE_THREADS", "MuonAdamWError", "Route", "abi_version", "adamw_step", "adamw_step_multi",
           "load", "mfma_probe", "mfma_probe_flops", "muon_check_plan", "muon_ns_time", "muon_phases", "muon_route_of",
           "muon_static_init", "muon_step", "muon_step_static", "muon_tune", "muon_tune_configs", "muon_tune_reset",
           "muon_workspace_bytes", "newton_schulz", "newton_schulz_workspace_bytes",
           "stream_probe", "MuonAdamW"]

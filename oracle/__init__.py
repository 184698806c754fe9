"""CPU oracle of the hybrid Muon + AdamW optimizer step (float64, numpy).

TEST INFRASTRUCTURE ONLY.  It is the yardstick the HIP library is checked
against: only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import it.  It shares no code with the HIP path (the
package ``adamw_optimizer_step_muon_amd``) and imports nothing from it.

Each function writes out the pages' definitions and cites them;
``tests/test_oracle_*.py`` pins every function to values printed on the pages,
closed forms, independent formulations and special cases.  Parity status per
function:

* newton_schulz, route, update_scale     pinned (the printed matrix iteration and
                                         the SVD form, each restated in the tests;
                                         printed spectra; invariant band)
* muon_step                              pinned (composition of pinned parts,
                                         zero-gradient decay, momentum closed form)
* muon_step with cautious_wd             special cases only; beyond them the
                                         pages print no value ("parity unpinned"
                                         for the mixed-sign case)
* adamw_step (decoupled and coupled)     pinned (printed decay experiment,
                                         first-step closed form, pure decay)
* adamw_step with cautious_wd            special cases only ("parity unpinned"
                                         for the mixed-sign case)
"""
from .adamw import AdamWResult, adamw_step
from .muon import QUINTIC, MuonResult, Route, muon_step, muon_step_bucket, newton_schulz, route, update_scale

__all__ = ["AdamWResult", "adamw_step", "QUINTIC", "MuonResult", "Route", "muon_step",
           "muon_step_bucket", "newton_schulz", "route", "update_scale"]

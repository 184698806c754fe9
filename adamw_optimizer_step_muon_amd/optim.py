"""MuonAdamW: one optimizer over "muon" and "adamw" parameter groups.

"MuonAdamW vs DistMuonAdamW: Key Differences for Single and Multi-GPU Training in
nanochat": a single optimizer takes param_groups tagged ``"kind": "muon"`` or
``"kind": "adamw"`` with per-group hyperparameters; ``step()`` after ``backward()``;
the Muon kernel works on same-shape stacks (K, ...).  "Optimizers: AdamW, Muon and
the distributed optimizer", section "Muon: orthogonalising the update": Muon for
hidden 2-D matrices, AdamW for embeddings, the output layer and vectors.

Host bookkeeping only: each group is marshalled to the C ABI (ma_muon_step over its
stacks, ma_adamw_step_multi over its tensors).  Muon parameters are 3-D (K, A, B) stacks of
same-shape matrices (a 2-D matrix counts as K = 1); stacking a model's matrices into
such buffers is the caller's layout choice.  State is fp32 and zero-initialised:
``momentum_buffer`` (4 bytes per Muon parameter), ``exp_avg`` and ``exp_avg_sq``
(8 bytes per AdamW parameter).
"""
from __future__ import annotations

from typing import Dict, List

from . import _lib

MUON_DEFAULTS = dict(lr=0.02, momentum=0.95, weight_decay=0.0, nesterov=True, ns_steps=5,
                     ns_coeffs=None, ns_eps=1e-7, cautious_wd=False, scale_mode=0, ns_mode=0)
ADAMW_DEFAULTS = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                      decoupled=True, cautious_wd=False)


class MuonAdamW:
    def __init__(self, param_groups: List[Dict]):
        import torch

        self.param_groups = []
        self.state: Dict[int, Dict] = {}
        self._workspace = None
        for g in param_groups:
            kind = g.get("kind", "muon")
            if kind not in ("muon", "adamw"):
                raise ValueError(f"unknown group kind {kind!r}")
            defaults = MUON_DEFAULTS if kind == "muon" else ADAMW_DEFAULTS
            unknown = set(g) - set(defaults) - {"params", "kind"}
            if unknown:
                raise ValueError(f"unknown {kind} hyperparameters {sorted(unknown)}")
            group = dict(defaults)
            group.update(g)
            group["kind"] = kind
            group["params"] = list(g["params"])
            group["step"] = 0
            for p in group["params"]:
                if p.dtype != torch.float32 or not p.is_contiguous():
                    raise ValueError("parameters must be contiguous float32 tensors")
                if kind == "muon":
                    if p.dim() not in (2, 3):
                        raise ValueError("Muon parameters are 2-D or (K, A, B) stacks")
                    self.state[id(p)] = {"momentum_buffer": torch.zeros_like(p)}
                else:
                    self.state[id(p)] = {"exp_avg": torch.zeros_like(p),
                                         "exp_avg_sq": torch.zeros_like(p)}
            self.param_groups.append(group)

    def state_bytes_per_param(self, kind: str) -> float:
        n = b = 0
        for g in self.param_groups:
            if g["kind"] != kind:
                continue
            for p in g["params"]:
                n += p.numel()
                b += sum(t.numel() * t.element_size() for t in self.state[id(p)].values())
        return b / n if n else 0.0

    def _muon_workspace(self, stacks, device, ns_mode):
        import torch

        need = _lib.muon_workspace_bytes([tuple(_lib._as_stack(p).shape) for p, _, _ in stacks],
                                         ns_mode)
        if need and (self._workspace is None or self._workspace.numel() < need):
            self._workspace = torch.empty(need, dtype=torch.uint8, device=device)
        return self._workspace

    def step(self) -> None:
        for g in self.param_groups:
            live = [p for p in g["params"] if p.grad is not None]
            if not live:
                continue
            g["step"] += 1
            if g["kind"] == "adamw":
                # the group's tensors in one fused pass (one launch per 48 tensors)
                b1, b2 = g["betas"]
                segs = [(p.data, p.grad, self.state[id(p)]["exp_avg"],
                         self.state[id(p)]["exp_avg_sq"]) for p in live]
                _lib.adamw_step_multi(segs, step=g["step"], lr=g["lr"], beta1=b1, beta2=b2,
                                      eps=g["eps"], weight_decay=g["weight_decay"],
                                      decoupled=g["decoupled"], cautious_wd=g["cautious_wd"])
            else:
                stacks = [(p.data, p.grad, self.state[id(p)]["momentum_buffer"]) for p in live]
                ws = self._muon_workspace(stacks, live[0].device, g["ns_mode"])
                _lib.muon_step(stacks, lr=g["lr"], momentum=g["momentum"],
                               weight_decay=g["weight_decay"], nesterov=g["nesterov"],
                               ns_steps=g["ns_steps"], ns_coeffs=g["ns_coeffs"],
                               ns_eps=g["ns_eps"], cautious_wd=g["cautious_wd"],
                               scale_mode=g["scale_mode"], ns_mode=g["ns_mode"], workspace=ws)

    def zero_grad(self, set_to_none: bool = True) -> None:
        for g in self.param_groups:
            for p in g["params"]:
                if p.grad is None:
                    continue
                if set_to_none:
                    p.grad = None
                else:
                    p.grad.zero_()

    def state_dict(self) -> Dict:
        groups, state = [], {}
        idx = 0
        for g in self.param_groups:
            ids = []
            for p in g["params"]:
                state[idx] = {k: v.clone() for k, v in self.state[id(p)].items()}
                ids.append(idx)
                idx += 1
            groups.append({k: v for k, v in g.items() if k != "params"} | {"params": ids})
        return {"state": state, "param_groups": groups}

    def load_state_dict(self, sd: Dict) -> None:
        flat = [p for g in self.param_groups for p in g["params"]]
        for (idx, st) in sd["state"].items():
            for k, v in st.items():
                self.state[id(flat[int(idx)])][k].copy_(v)
        for g, sg in zip(self.param_groups, sd["param_groups"]):
            g["step"] = sg["step"]

"""MuonAdamW: one optimizer over "muon" and "adamw" parameter groups.

"MuonAdamW vs DistMuonAdamW: Key Differences for Single and Multi-GPU Training in
nanochat": a single optimizer takes param_groups tagged ``"kind": "muon"`` or
``"kind": "adamw"`` with per-group hyperparameters; ``step()`` after ``backward()``;
the Muon kernel works on same-shape stacks (K, ...).  "Optimizers: AdamW, Muon and
the distributed optimizer", section "Muon: orthogonalising the update": Muon for
hidden 2-D matrices, AdamW for embeddings, the output layer and vectors.
"DMuon: Efficient Distributed Muon Training with Near-Adam Overhead", section 2.2
(batching): same-shape matrices are orthogonalised together.

Host bookkeeping only: each group is marshalled to the C ABI (one ma_muon_step over
all of a group's shape buckets, ma_adamw_step_multi over its AdamW tensors).

Muon parameters are bucketed by shape at construction: the K 2-D parameters of one
shape A x B become views into one contiguous (K, A, B) buffer (their values are copied
in, and ``p.data`` is re-pointed at the view, so the parameter objects the caller holds
see every update), and each parameter's momentum is a view into a (K, A, B) momentum
buffer.  A 3-D (K, A, B) parameter is a bucket of its own.  At each step the
gradients are gathered into one (K, A, B) buffer per bucket (one copy launch per
bucket; none when the gradients already are the buffer's views: the gather leaves
them so, and backward then accumulates into the buffer until ``zero_grad()`` drops
them), and a single ma_muon_step runs all buckets, so buckets that share a GEMM
configuration share its launches.  Parameters without a gradient are not stepped.
State is fp32 and zero-initialised: ``momentum_buffer`` (4 bytes per Muon parameter),
``exp_avg`` and ``exp_avg_sq`` (8 bytes per AdamW parameter).

A Muon group's ``ns_mode`` (0 by default) selects the Newton-Schulz route: 1 runs the
Gram-space iteration ("DMuon", section 2.2) on fp16 operands for the buckets whose long
side is at least 3.5x the other (MLP projections), the printed iteration elsewhere.
"""
from __future__ import annotations

from typing import Dict, List

from . import _lib

MUON_DEFAULTS = dict(lr=0.02, momentum=0.95, weight_decay=0.0, nesterov=True, ns_steps=5,
                     ns_coeffs=None, ns_eps=1e-7, cautious_wd=False, scale_mode=0, ns_mode=0)
ADAMW_DEFAULTS = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                      decoupled=True, cautious_wd=False)


class _Bucket:
    """K same-shape Muon parameters stored as one (K, A, B) buffer."""

    def __init__(self, params, stacked: bool):
        import torch

        self.params = params
        self.stacked = stacked  # one caller-provided (K, A, B) parameter
        if stacked:
            self.param = params[0].data
        else:
            self.param = torch.stack([p.data for p in params])
            for k, p in enumerate(params):
                p.data = self.param[k]
        self.grad = torch.zeros_like(self.param)
        self.momentum = torch.zeros_like(self.param)

    def momentum_view(self, k):
        return self.momentum if self.stacked else self.momentum[k]

    def live_stacks(self):
        """(param, grad, momentum) stacks for ma_muon_step: the whole bucket when every
        parameter has a gradient (gathered into the bucket's gradient buffer), one
        (1, A, B) slice per parameter that has one when only some do (a parameter
        without a gradient is not stepped; a matrix's result does not depend on the
        bucket it runs in), nothing when none does."""
        import torch

        grads = [p.grad for p in self.params]
        if all(g is None for g in grads):
            return []
        if self.stacked:
            if grads[0].data_ptr() != self.grad.data_ptr():
                self.grad.copy_(grads[0])
            return [(self.param, self.grad, self.momentum)]
        K = len(self.params)
        if any(g is None for g in grads):
            return [(self.param[k:k + 1], grads[k].reshape(1, *grads[k].shape).contiguous(),
                     self.momentum[k:k + 1]) for k in range(K) if grads[k] is not None]
        views = [self.grad[k] for k in range(K)]
        if not all(g.data_ptr() == v.data_ptr() for g, v in zip(grads, views)):
            torch.stack(grads, out=self.grad)
            # later backward passes accumulate straight into the buffer
            for p, v in zip(self.params, views):
                p.grad = v
        return [(self.param, self.grad, self.momentum)]

    @property
    def shape(self):
        return tuple(self.param.shape)


class MuonAdamW:
    def __init__(self, param_groups: List[Dict]):
        import torch

        self.param_groups = []
        self.state: Dict[int, Dict] = {}
        self._workspace = None
        self._buckets: Dict[int, List[_Bucket]] = {}
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
                if kind == "muon" and p.dim() not in (2, 3):
                    raise ValueError("Muon parameters are 2-D or (K, A, B) stacks")
            if len({id(p) for p in group["params"]}) != len(group["params"]):
                raise ValueError("a parameter appears twice in one group")
            if kind == "muon":
                buckets = self._bucket(group["params"])
                self._buckets[len(self.param_groups)] = buckets
                for b in buckets:
                    for k, p in enumerate(b.params):
                        self.state[id(p)] = {"momentum_buffer": b.momentum_view(k)}
            else:
                for p in group["params"]:
                    self.state[id(p)] = {"exp_avg": torch.zeros_like(p),
                                         "exp_avg_sq": torch.zeros_like(p)}
            self.param_groups.append(group)

    @staticmethod
    def _bucket(params) -> List[_Bucket]:
        """Same-shape 2-D parameters into (K, A, B) buckets, in order of first appearance;
        each 3-D parameter a bucket of its own."""
        order, by_shape = [], {}
        for p in params:
            if p.dim() == 3:
                order.append(("stack", id(p), [p]))
                continue
            key = tuple(p.shape)
            if key not in by_shape:
                by_shape[key] = []
                order.append(("shape", key, by_shape[key]))
            by_shape[key].append(p)
        return [_Bucket(ps, kind == "stack") for kind, _, ps in order]

    def muon_buckets(self, group_index: int = None):
        """(K, A, B) of the Muon buckets (of one group, or of every Muon group)."""
        idx = [group_index] if group_index is not None else sorted(self._buckets)
        return [b.shape for i in idx for b in self._buckets.get(i, [])]

    def state_bytes_per_param(self, kind: str) -> float:
        n = b = 0
        for g in self.param_groups:
            if g["kind"] != kind:
                continue
            for p in g["params"]:
                n += p.numel()
                b += sum(t.numel() * t.element_size() for t in self.state[id(p)].values())
        return b / n if n else 0.0

    def _muon_workspace(self, shapes, device, ns_mode):
        import torch

        need = _lib.muon_workspace_bytes(shapes, ns_mode)
        if need and (self._workspace is None or self._workspace.numel() < need):
            self._workspace = torch.empty(need, dtype=torch.uint8, device=device)
        return self._workspace

    def step(self) -> None:
        for gi, g in enumerate(self.param_groups):
            if g["kind"] == "adamw":
                live = [p for p in g["params"] if p.grad is not None]
                if not live:
                    continue
                g["step"] += 1
                # the group's tensors in one fused pass (one launch per 48 tensors)
                b1, b2 = g["betas"]
                segs = [(p.data, p.grad, self.state[id(p)]["exp_avg"],
                         self.state[id(p)]["exp_avg_sq"]) for p in live]
                _lib.adamw_step_multi(segs, step=g["step"], lr=g["lr"], beta1=b1, beta2=b2,
                                      eps=g["eps"], weight_decay=g["weight_decay"],
                                      decoupled=g["decoupled"], cautious_wd=g["cautious_wd"])
                continue
            # Muon: every bucket with gradients in one call
            stacks = [st for b in self._buckets[gi] for st in b.live_stacks()]
            if not stacks:
                continue
            g["step"] += 1
            ws = self._muon_workspace([tuple(st[0].shape) for st in stacks], stacks[0][0].device,
                                      g["ns_mode"])
            _lib.muon_step(stacks, lr=g["lr"], momentum=g["momentum"],
                           weight_decay=g["weight_decay"], nesterov=g["nesterov"],
                           ns_steps=g["ns_steps"], ns_coeffs=g["ns_coeffs"], ns_eps=g["ns_eps"],
                           cautious_wd=g["cautious_wd"], scale_mode=g["scale_mode"],
                           ns_mode=g["ns_mode"], workspace=ws)

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

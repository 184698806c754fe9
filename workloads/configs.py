"""Workload definitions for the hybrid Muon + AdamW optimizer step.

Pure data: tensor shapes, shape buckets, hyperparameters and the name of the
gradient recipe each workload draws from.  Nothing here performs any of the
optimizer's arithmetic; both the HIP path and the CPU oracle read these.

Shapes follow the transformer layouts the pages describe (hidden matrices
under Muon; embeddings, LM head and normalisation vectors under AdamW), see
"Optimizers: AdamW, Muon and the distributed optimizer", section "Muon:
orthogonalising the update" (which parameters stay on AdamW).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

# Quintic Newton-Schulz coefficients (a, b, c), the newton_schulz listing in
# "Optimizers: AdamW, Muon and the distributed optimizer", section "Muon:
# orthogonalising the update".
QUINTIC = (3.4445, -4.7750, 2.0315)


@dataclass(frozen=True)
class MuonBucket:
    """K same-shape A x B matrices stored as one contiguous (K, A, B) tensor."""

    name: str
    K: int
    A: int
    B: int

    @property
    def numel(self) -> int:
        return self.K * self.A * self.B


@dataclass(frozen=True)
class AdamWTensor:
    name: str
    shape: Tuple[int, ...]

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= s
        return n


@dataclass(frozen=True)
class MuonHP:
    lr: float = 0.02
    momentum: float = 0.95
    weight_decay: float = 0.1
    nesterov: bool = True
    ns_steps: int = 5
    coeffs: Tuple[float, float, float] = QUINTIC
    ns_eps: float = 1e-7
    cautious_wd: bool = False
    scale_mode: int = 0  # 0: 0.2*sqrt(max(A,B)); 1: sqrt(max(1, A/B))


@dataclass(frozen=True)
class AdamWHP:
    lr: float = 3e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1
    decoupled: bool = True
    cautious_wd: bool = False


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    muon: List[MuonBucket]
    adamw: List[AdamWTensor]
    steps: int
    seed: int
    # grad recipes, by name (workloads.gen implements them)
    muon_grad: str
    adamw_grad: str
    muon_hp: MuonHP = field(default_factory=MuonHP)
    adamw_hp: AdamWHP = field(default_factory=AdamWHP)
    # sigma0 of the gradient recipes: 0.02 for Muon matrices and 1e-3 for AdamW tensors
    # (the tiny workload's statement), 1e-3 for both where a workload states it
    muon_sigma: float = 0.02
    adamw_sigma: float = 1e-3

    @property
    def muon_numel(self) -> int:
        return sum(b.numel for b in self.muon)

    @property
    def adamw_numel(self) -> int:
        return sum(t.numel for t in self.adamw)

    @property
    def n_matrices(self) -> int:
        return sum(b.K for b in self.muon)


def _gpt(index, name, layers, hidden, mlp, vocab, steps, seed, muon_grad, adamw_grad,
         kv=None, cautious=False, muon_sigma=0.02):
    """Buckets for a GPT-style stack: attention Q,K,V,O and an up/down MLP."""
    kv = hidden if kv is None else kv
    buckets: List[MuonBucket] = []
    if kv == hidden:
        buckets.append(MuonBucket("attn_qkvo", 4 * layers, hidden, hidden))
    else:
        buckets.append(MuonBucket("attn_qo", 2 * layers, hidden, hidden))
        buckets.append(MuonBucket("attn_kv", 2 * layers, hidden, kv))
    buckets.append(MuonBucket("mlp_up", layers, hidden, mlp))
    buckets.append(MuonBucket("mlp_down", layers, mlp, hidden))
    adamw = [AdamWTensor("embedding", (vocab, hidden)), AdamWTensor("lm_head", (vocab, hidden))]
    # two normalisation gains per block plus the final one
    adamw += [AdamWTensor(f"norm{i}", (hidden,)) for i in range(2 * layers + 1)]
    return Workload(index, name, buckets, adamw, steps, seed, muon_grad, adamw_grad,
                    muon_hp=MuonHP(cautious_wd=cautious), muon_sigma=muon_sigma)


WORKLOADS: List[Workload] = [
    Workload(
        0, "tiny: Muon 64x128 + 128x64, AdamW 4096 + 512x64",
        [MuonBucket("w0", 1, 64, 128), MuonBucket("w1", 1, 128, 64)],
        [AdamWTensor("vec", (4096,)), AdamWTensor("embedding", (512, 64))],
        steps=3, seed=0, muon_grad="rowlognormal", adamw_grad="gauss",
    ),
    # gradients N(0, 1e-3^2) plus a rank-8 component with 30 % of the energy, for every
    # tensor (Muon matrices included)
    _gpt(1, "12-layer GPT, hidden 768, MLP 3072, vocab 65536", 12, 768, 3072, 65536,
         steps=10, seed=1, muon_grad="lowrank", adamw_grad="lowrank", muon_sigma=1e-3),
    _gpt(2, "20-layer GPT, hidden 1280, MLP 5120, vocab 65536", 20, 1280, 5120, 65536,
         steps=10, seed=2, muon_grad="rowlognormal", adamw_grad="gauss"),
    _gpt(3, "24-layer GQA model, hidden 2048, KV 512, MLP 8192, vocab 128000", 24, 2048, 8192,
         128000, steps=5, seed=3, muon_grad="rowlognormal", adamw_grad="gauss", kv=512,
         cautious=True),
    Workload(
        4, "owned subset: 8 x 8192x28672, 8 x 28672x8192, 16 x 8192x8192; AdamW 128256x8192",
        [MuonBucket("up", 8, 8192, 28672), MuonBucket("down", 8, 28672, 8192),
         MuonBucket("square", 16, 8192, 8192)],
        [AdamWTensor("embedding", (128256, 8192))],
        steps=3, seed=4, muon_grad="conditioned", adamw_grad="conditioned",
    ),
]


def workload(index: int) -> Workload:
    return WORKLOADS[index]

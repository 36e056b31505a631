"""Workload presets: adapter-stack shapes and input distributions.

Shapes follow the Llama-2 7B and 70B projection sizes the AdaFuse pages evaluate on
(Llama2-7B, results section of both summary pages); the 70B stack is the largest that
fits one 288 GB device.  Distribution parameters are standard deviations.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Projection:
    name: str
    d_out: int
    d_in: int


def llama_layer(d_model: int, d_ff: int, d_kv: int) -> tuple[Projection, ...]:
    return (
        Projection("q", d_model, d_model),
        Projection("k", d_kv, d_model),
        Projection("v", d_kv, d_model),
        Projection("o", d_model, d_model),
        Projection("gate", d_ff, d_model),
        Projection("up", d_ff, d_model),
        Projection("down", d_model, d_ff),
    )


@dataclass(frozen=True)
class StackConfig:
    """A stack of n_layers identical layers, each with the listed projections, every
    projection carrying its own bank of E LoRA adapters of rank r."""

    name: str
    n_layers: int
    projections: tuple[Projection, ...]
    d_model: int          # router input width (the hidden state h)
    E: int                # adapters per projection
    r: int                # LoRA rank
    k: int                # experts selected by the router
    scale: float          # LoRA scale s
    dtype: str            # "fp32" or "bf16" storage
    renorm: bool = True   # gates: softmax over the selected logits
    inplace: bool = True
    w_std: float = 0.02
    b_std: float = 0.01
    h_std: float = 1.0
    host_generated: bool = False   # small enough to draw with NumPy on the host
    note: str = ""
    decode_steps: int = 0           # end-to-end workload: decode tokens per request
    extra: dict = field(default_factory=dict)

    def a_std(self, d_in: int) -> float:
        return 1.0 / math.sqrt(d_in)

    def router_std(self) -> float:
        return 1.0 / math.sqrt(self.d_model)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    @property
    def kr(self) -> int:
        return self.k * self.r

    def weight_elems(self) -> int:
        return self.n_layers * sum(p.d_out * p.d_in for p in self.projections)

    def merge_bytes(self) -> int:
        """Algorithmic HBM bytes of one merge: W read + W' written + the selected
        adapters' A and B read once."""
        eb = self.elem_bytes
        w = 2 * self.weight_elems() * eb
        sel = self.n_layers * sum(self.k * self.r * (p.d_in + p.d_out) for p in self.projections) * eb
        return w + sel

    def merge_flops(self) -> int:
        return 2 * self.k * self.r * self.weight_elems()

    def adapter_bank_bytes(self) -> int:
        """Every projection's whole bank of E adapters (A and B), resident beside W."""
        return self.n_layers * sum(self.E * self.r * (p.d_in + p.d_out) for p in self.projections) * self.elem_bytes

    def decode_bytes_per_token(self) -> int:
        return self.weight_elems() * self.elem_bytes


_L7 = llama_layer(4096, 11008, 4096)
_L70 = llama_layer(8192, 28672, 1024)

TINY = StackConfig(
    name="tiny",
    n_layers=2,
    projections=(Projection("proj", 256, 256),),
    d_model=256, E=4, r=8, k=2, scale=2.0, dtype="fp32",
    host_generated=True,
    note="2 layers x one 256x256 fp32 projection, E=4, r=8, top-2, s=2",
)

LLAMA7B_E8R16K2 = StackConfig(
    name="llama7b_e8r16k2",
    n_layers=32, projections=_L7, d_model=4096,
    E=8, r=16, k=2, scale=2.0, dtype="bf16",
    note="Llama-2-7B-shaped stack (32 x q,k,v,o 4096^2; gate,up 11008x4096; down 4096x11008), "
         "bf16, E=8 adapters per projection, rank 16, top-2",
)

LLAMA7B_E16R64K4 = StackConfig(
    name="llama7b_e16r64k4",
    n_layers=32, projections=_L7, d_model=4096,
    E=16, r=64, k=4, scale=2.0, dtype="bf16",
    note="Llama-2-7B-shaped stack, bf16, E=16, rank 64, top-4 (contraction 256), "
         "gates renormalised over the top-4, logit gap >= 1e-3",
)

LLAMA70B_E8R16K2 = StackConfig(
    name="llama70b_e8r16k2",
    n_layers=80, projections=_L70, d_model=8192,
    E=8, r=16, k=2, scale=2.0, dtype="bf16", inplace=True,
    note="Llama-2-70B-shaped stack (80 x q,o 8192^2; k,v 1024x8192; gate,up 28672x8192; "
         "down 8192x28672), bf16, E=8, rank 16, top-2, merged in place then unmerged",
)

# One GPU's share of the 70B stack under 8-way tensor parallelism: the column-parallel
# projections (q, k, v, gate, up) keep 1/8 of the output rows of W and of every B with
# the full A; the row-parallel ones (o, down) keep 1/8 of the input columns of W and of
# every A with the full B.  The merge needs no exchange, so this is the whole of one
# GPU's merge.
_L70_TP8 = (
    Projection("q", 8192 // 8, 8192),
    Projection("k", 1024 // 8, 8192),
    Projection("v", 1024 // 8, 8192),
    Projection("o", 8192, 8192 // 8),
    Projection("gate", 28672 // 8, 8192),
    Projection("up", 28672 // 8, 8192),
    Projection("down", 8192, 28672 // 8),
)

LLAMA70B_TP8_E8R16K2 = StackConfig(
    name="llama70b_tp8_e8r16k2",
    n_layers=80, projections=_L70_TP8, d_model=8192,
    E=8, r=16, k=2, scale=2.0, dtype="bf16", inplace=True,
    note="one GPU's shard of the Llama-2-70B-shaped stack under 8-way tensor parallelism "
         "(80 x q 1024x8192, k,v 128x8192, o 8192x1024, gate,up 3584x8192, down 8192x3584), "
         "bf16, E=8, rank 16, top-2, in place",
)

E2E_7B = StackConfig(
    name="e2e_llama7b",
    n_layers=32, projections=_L7, d_model=4096,
    E=8, r=16, k=2, scale=2.0, dtype="bf16",
    decode_steps=128,
    note="batch-1 request on the 7B-shaped stack: pregate + merge, 128 decode steps of "
         "GEMVs through every projection, unmerge; vs a per-layer routed unmerged baseline",
)

PRESETS = {c.name: c for c in (TINY, LLAMA7B_E8R16K2, LLAMA7B_E16R64K4, LLAMA70B_E8R16K2,
                                LLAMA70B_TP8_E8R16K2, E2E_7B)}


def scaled(cfg: StackConfig, n_layers: int) -> StackConfig:
    """The same stack cut to n_layers (used for bounded samples and small parity runs)."""
    from dataclasses import replace

    return replace(cfg, name=f"{cfg.name}_L{n_layers}", n_layers=n_layers)

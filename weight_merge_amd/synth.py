"""Seeded synthetic inputs for the adapter-merge path.

This module only draws random tensors of the configured shapes and distributions.
It holds none of the method's arithmetic (no routing, no selection, no merge) so
both the GPU path and the CPU oracle can be fed from it.

Recipe (every tensor has its own seed, derived from the base seed and a key naming
its config, layer, projection and kind):
  W ~ N(0, 0.02) [d_out x d_in]; A ~ N(0, 1/sqrt(d_in)) [E x r x d_in];
  B ~ N(0, 0.01) [E x d_out x r]; h ~ N(0, 1) [d]; R ~ N(0, 1/sqrt(d)) [E x d];
  decode activations x ~ N(0, 1).  Values are drawn in fp32 and rounded (RNE) to
  the storage dtype.  Small stacks are drawn with NumPy's PCG64 on the host; large
  ones with torch's Philox generator on the device, so a 140 GB stack never crosses
  PCIe.  The router inputs are always drawn on the host.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass

import numpy as np
import torch

from .configs import StackConfig

TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def tensor_seed(base_seed: int, *key) -> int:
    """A 63-bit seed from the base seed and a key tuple (stable across processes)."""
    words = [int(base_seed) & 0xFFFFFFFF]
    for part in key:
        words.append(zlib.crc32(str(part).encode()) & 0xFFFFFFFF)
    state = np.random.SeedSequence(words).generate_state(2, dtype=np.uint32)
    return int((int(state[0]) << 31) ^ int(state[1])) & ((1 << 63) - 1)


def host_normal(seed: int, shape, std: float, dtype: str = "fp32") -> torch.Tensor:
    """N(0, std) drawn with NumPy PCG64 in fp32, returned as a CPU tensor of `dtype`."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)
    return torch.from_numpy(x).to(TORCH_DTYPE[dtype])


def device_normal(seed: int, shape, std: float, dtype: str, device) -> torch.Tensor:
    """N(0, std) drawn with torch's generator on `device` in fp32, rounded to `dtype`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(TORCH_DTYPE[dtype])


def draw(cfg: StackConfig, seed: int, key: tuple, shape, std: float, device) -> torch.Tensor:
    s = tensor_seed(seed, cfg.name.split("_L")[0], *key)
    if cfg.host_generated or device is None or str(device) == "cpu":
        t = host_normal(s, shape, std, cfg.dtype)
        return t if device is None else t.to(device)
    return device_normal(s, shape, std, cfg.dtype, device)


def router_inputs(cfg: StackConfig, seed: int):
    """(h [d], R [E x d]) on the host, in the storage dtype."""
    base = cfg.name.split("_L")[0]
    h = host_normal(tensor_seed(seed, base, "h"), (cfg.d_model,), cfg.h_std, cfg.dtype)
    R = host_normal(tensor_seed(seed, base, "router"), (cfg.E, cfg.d_model), cfg.router_std(), cfg.dtype)
    return h, R


@dataclass
class Stack:
    """Per-(layer, projection) weights and adapter banks of one stack."""

    cfg: StackConfig
    W: list      # [layer][proj] -> [d_out, d_in]
    A: list      # [layer][proj] -> [E, r, d_in]
    B: list      # [layer][proj] -> [E, d_out, r]

    def items(self):
        for l in range(self.cfg.n_layers):
            for p, proj in enumerate(self.cfg.projections):
                yield l, p, proj


def draw_layer(cfg: StackConfig, seed: int, l: int, device=None, weights: bool = True):
    """W, A and B of every projection of layer l (lists in projection order)."""
    wl, al, bl = [], [], []
    for proj in cfg.projections:
        key = (l, proj.name)
        wl.append(draw(cfg, seed, key + ("W",), (proj.d_out, proj.d_in), cfg.w_std, device)
                  if weights else None)
        al.append(draw(cfg, seed, key + ("A",), (cfg.E, cfg.r, proj.d_in), cfg.a_std(proj.d_in), device))
        bl.append(draw(cfg, seed, key + ("B",), (cfg.E, proj.d_out, cfg.r), cfg.b_std, device))
    return wl, al, bl


def make_stack(cfg: StackConfig, seed: int, device=None, weights: bool = True) -> Stack:
    """Draw W, A and B for every (layer, projection).  With weights=False only the
    adapter banks are drawn (W left as None), for callers that fill W themselves."""
    W, A, B = [], [], []
    for l in range(cfg.n_layers):
        wl, al, bl = draw_layer(cfg, seed, l, device, weights)
        W.append(wl)
        A.append(al)
        B.append(bl)
    return Stack(cfg, W, A, B)


def decode_inputs(cfg: StackConfig, seed: int, steps: int, device=None):
    """Decode activations: one x ~ N(0,1) per (step, projection type), shared across
    layers; returns {projection name: [steps, d_in]}."""
    base = cfg.name.split("_L")[0]
    out = {}
    for proj in cfg.projections:
        t = host_normal(tensor_seed(seed, base, "x", proj.name), (steps, proj.d_in), 1.0, cfg.dtype)
        out[proj.name] = t if device is None else t.to(device)
    return out


def adapter_bank(seed: int, E: int, r: int, d_out: int, d_in: int, dtype: str,
                 w_std=0.02, b_std=0.01, device=None):
    """One projection's (W, A, B) drawn on the host: for shape fuzzing and small cases."""
    W = host_normal(tensor_seed(seed, "fz", E, r, d_out, d_in, "W"), (d_out, d_in), w_std, dtype)
    A = host_normal(tensor_seed(seed, "fz", E, r, d_out, d_in, "A"), (E, r, d_in), 1.0 / np.sqrt(d_in), dtype)
    B = host_normal(tensor_seed(seed, "fz", E, r, d_out, d_in, "B"), (E, d_out, r), b_std, dtype)
    if device is not None:
        W, A, B = W.to(device), A.to(device), B.to(device)
    return W, A, B


def small_router(seed: int, E: int, d: int, dtype: str):
    """(h, R) for a router of E experts over d inputs, drawn on the host."""
    h = host_normal(tensor_seed(seed, "fz-h", E, d), (d,), 1.0, dtype)
    R = host_normal(tensor_seed(seed, "fz-R", E, d), (E, d), 1.0 / np.sqrt(d), dtype)
    return h, R

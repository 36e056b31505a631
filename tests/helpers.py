"""Shared helpers of the test suite (test infrastructure: may call the oracle)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import adafuse as O
from weight_merge_amd import synth

# Merged bf16 weights: |W'_gpu - W'_ref| <= 8e-3 |W'_ref| + 1e-4, ref the unrounded
# fp64 W + delta.  The kernel's arithmetic is RNE(W + sum_t RNE(s g b_t) a_t) with exact
# products and fp32 sums, so its error is at most 2^-8 |W'| (final rounding: half an
# ulp of bf16's 8 significant bits) plus 2^-8 sum_t |s g b_t a_t| (gate folded into B
# in bf16) plus the fp32 accumulation.
# The second term is far below 1e-4 on weight-shaped data (d_in in the thousands, so
# A ~ N(0, 1/sqrt(d_in)) is small); folded_bound() states the full bound for inputs
# where it is not.
BF16_RTOL, BF16_ATOL = 8e-3, 1e-4
# fp32 storage: one final rounding (2^-24 relative) plus fp32 accumulation over k*r
# terms; 1e-6 relative + 1e-7 absolute leaves a >10x margin and still catches a
# dropped adapter (~5e-3).
F32_RTOL, F32_ATOL = 1e-6, 1e-7
# Gates: fp32 logits differ from fp64 by <~5e-5; the gate's relative error follows.
GATE_RTOL, GATE_ATOL = 1e-4, 1e-6
MIN_GAP = 1e-3


def tol(dtype):
    return (BF16_RTOL, BF16_ATOL) if dtype == torch.bfloat16 else (F32_RTOL, F32_ATOL)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def check_close(got: torch.Tensor | np.ndarray, ref: np.ndarray, rtol: float, atol: float, what: str = ""):
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    err = np.abs(g - ref)
    bound = rtol * np.abs(ref) + atol
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; worst at {i}: "
                             f"got {g[i]!r} ref {ref[i]!r} err {err[i]:.3e} bound {bound[i]:.3e}")
    return float(np.max(err / (np.abs(ref) + atol / rtol))) if err.size else 0.0


def folded_bound(Aw, Bw, idx, gate, scale: float) -> np.ndarray:
    """Per-element error bound of the bf16 merge's arithmetic beyond the stated
    tolerance, over the selected adapters' terms sum_t |s g b_t a_t|: 2^-8 of it for
    rounding s g B to bf16 (half an ulp of 8 significant bits), plus (k r + 2) 2^-23 of
    it for the fp32 accumulation of k r products (twice the usual gamma, for margin)."""
    A64, B64 = to64(Aw), to64(Bw)
    acc = np.zeros((B64.shape[1], A64.shape[2]))
    n = 0
    for e, g in zip(np.asarray(idx).tolist(), np.asarray(gate, dtype=np.float64).tolist()):
        if 0 <= e < A64.shape[0] and g != 0.0:
            acc += np.abs(scale * g * B64[e]) @ np.abs(A64[e])
            n += A64.shape[1]
    return (2.0 ** -8 + (n + 2) * 2.0 ** -23) * acc


def folded_gate_model(W, Aw, Bw, slots, scale_sign_pairs=None):
    """The bf16 merge's arithmetic written out on the CPU (a model of the fused kernel
    for tighter checks; the oracle stays the exact fp64 method).  The fused kernel
    concatenates the selected adapters with each gate folded into the up projection
    ("AdaFuse", Japanese summary page, technical overview 2.2): here each coefficient
    c = (+-s) g is formed in fp32, c B_e is computed in fp32 and rounded to bf16, and the
    products with A_e (exact for bf16 operands) are summed in fp64.

    slots: list of (expert, gate, signed scale).  Returns the unrounded fp64 result and
    |W| + sum_t |b'_t a_t|, the scale of the kernel's fp32 accumulation error."""
    W64, A64 = to64(W), to64(Aw)
    B32 = Bw.float()
    out, mag = W64.copy(), np.abs(W64)
    for e, g, sc in slots:
        c = np.float32(sc) * np.float32(g)
        if not (0 <= e < A64.shape[0]) or c == 0:
            continue
        b = (B32[e] * torch.tensor(c, dtype=torch.float32)).to(torch.bfloat16).double().numpy()
        out = out + b @ A64[e]
        mag = mag + np.abs(b) @ np.abs(A64[e])
    return out, mag


def min_gap(z) -> float:
    s = np.sort(np.asarray(z, dtype=np.float64))
    return float(np.min(np.diff(s))) if s.size > 1 else np.inf


def gapped_router(E: int, d: int, dtype: str, seed: int):
    """(h, R, seed) from the first seed at or after `seed` whose logits (per the
    oracle) are pairwise at least 1e-3 apart, so top-k has no near-ties."""
    s = seed
    while True:
        h, R = synth.small_router(s, E, d, dtype)
        if min_gap(O.router_logits(to64(h), to64(R))) >= MIN_GAP:
            return h, R, s
        s += 1


def gapped_stack_router(cfg, seed: int):
    s = seed
    while True:
        h, R = synth.router_inputs(cfg, s)
        if min_gap(O.router_logits(to64(h), to64(R))) >= MIN_GAP:
            return h, R, s
        s += 1


def oracle_selection(h, R, k, renorm=True):
    """Selection from the oracle, as device-ready int32 / fp32 tensors (plus the fp64
    gates rounded to fp32, the exact values the kernel will read)."""
    idx, g = O.pregate(to64(h), to64(R), k, renorm)
    return torch.tensor(idx, dtype=torch.int32), torch.tensor(g, dtype=torch.float32)


def sample_rows(d_out: int, rng: np.random.Generator, n_random: int = 24, tile: int = 128) -> np.ndarray:
    """Rows covering every 16-row MFMA position of several tile bands: the first and
    last row of 8 random bands, plus random rows, plus row 0 and the last row."""
    n_bands = (d_out + tile - 1) // tile
    bands = rng.choice(n_bands, size=min(8, n_bands), replace=False)
    rows = {0, d_out - 1}
    for b in bands:
        rows.add(int(b) * tile)
        rows.add(min(d_out, (int(b) + 1) * tile) - 1)
    rows.update(int(v) for v in rng.integers(0, d_out, size=n_random))
    return np.array(sorted(rows))

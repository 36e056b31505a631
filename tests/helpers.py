"""Shared helpers of the test suite (test infrastructure: may call the oracle)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import adafuse as O
from weight_merge_amd import synth

# Merged bf16 weights: |W'_gpu - W'_ref| <= 8e-3 |W'_ref| + 1e-4, ref the unrounded
# fp64 W + delta (the stated tolerance, for every admitted input).  The kernels carry
# each coefficient s g at fp32 accuracy (a hi + lo pair of bf16 planes for B, or the
# coefficient applied to fp32 accumulators), so the error is one final bf16 rounding
# (at most 2^-8 |W'|, under half the relative term) plus ~2^-16 and fp32 accumulation
# terms of sum_t |s g b_t a_t| (see kernel_error_bound).
BF16_RTOL, BF16_ATOL = 8e-3, 1e-4
# fp32 storage (the small stacks): one final rounding (2^-24 relative) plus the fp32
# accumulation of k*r products: 1e-6 relative + 1e-7 absolute, plus (k r + 2) 2^-23
# sum_t |s g b_t a_t| for the accumulation (fp32_accumulation_bound), which only inputs
# with large A (small d_in) reach; a dropped adapter (~5e-3) still fails.
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


def term_magnitude(Aw, Bw, slots) -> np.ndarray:
    """sum over the active slots (expert, gate, signed scale) of |s g B_e| @ |A_e|: the
    magnitude of the delta's terms, which scales the kernels' accumulation error."""
    A64, B64 = to64(Aw), to64(Bw)
    acc = np.zeros((B64.shape[1], A64.shape[2]))
    for e, g, sc in slots:
        c = float(np.float32(sc) * np.float32(g))
        if 0 <= e < A64.shape[0] and c != 0.0:
            acc += np.abs(c * B64[e]) @ np.abs(A64[e])
    return acc


def fp32_accumulation_bound(Aw, Bw, slots) -> np.ndarray:
    """fp32 storage: the accumulation of k r products, (k r + 2) 2^-23 of the terms'
    magnitude (twice the usual gamma, for margin)."""
    n = sum(Aw.shape[1] for e, g, sc in slots if 0 <= e < Aw.shape[0] and g != 0)
    return (n + 2) * 2.0 ** -23 * term_magnitude(Aw, Bw, slots)


def kernel_error_bound(W, Aw, Bw, slots, ref) -> np.ndarray:
    """Tighter than the stated tolerance: what the bf16 merge's arithmetic allows.  One
    final rounding (2^-8 of the result), the split of c b into two bf16 planes (the lo
    plane's rounding: 2^-16 of each term), and fp32 sums of up to 2 k r exact products
    plus the W term (2 (2 k r + 2) 2^-24 of the magnitude, twice the usual gamma)."""
    n = sum(Aw.shape[1] for e, g, sc in slots if 0 <= e < Aw.shape[0] and g != 0)
    mag = np.abs(to64(W)) + term_magnitude(Aw, Bw, slots)
    eps = 2.0 ** -16 + 2 * (2 * n + 2) * 2.0 ** -24
    return 2.0 ** -8 * np.abs(ref) + (1 + 2.0 ** -8) * eps * mag


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


def merge_tile_rows(kr: int) -> int:
    """Rows per tile of the bf16 merge launch for contractions of kr = k r terms (32 x 256
    tiles up to 32 terms, 64 x 128 up to 64, 128 x 128 beyond)."""
    return 32 if kr <= 32 else 64 if kr <= 64 else 128


def sample_rows(d_out: int, rng: np.random.Generator, tile: int, n_random: int = 64,
                all_bands: bool = False, n_bands: int = 8) -> np.ndarray:
    """Rows of one projection to compare: the first and last row of every tile row band
    (all_bands) or of n_bands random bands, plus n_random random rows, plus row 0 and the
    last row.  `tile` is the launch's tile height, so band edges are real tile edges."""
    n_all = (d_out + tile - 1) // tile
    bands = np.arange(n_all) if all_bands else rng.choice(n_all, size=min(n_bands, n_all), replace=False)
    rows = {0, d_out - 1}
    for b in bands:
        rows.add(int(b) * tile)
        rows.add(min(d_out, (int(b) + 1) * tile) - 1)
    rows.update(int(v) for v in rng.integers(0, d_out, size=n_random))
    return np.array(sorted(rows))

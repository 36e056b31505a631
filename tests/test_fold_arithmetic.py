"""CPU checks of the two ways the bf16 merge kernels carry each coefficient c = +-s g
("AdaFuse", Japanese summary page, technical overview 2.2: the selected adapters are
concatenated and merged in one call), written out here as NumPy emulations of the
arithmetic (test code; the oracle stays the exact fp64 method):

  split fold            c B as two bf16 planes hi = bf16(c b), lo = bf16(c b - hi),
                        both multiplied by A with fp32 sums;
  scaled accumulators   unscaled bf16 B, the slots in order of increasing |c|, the fp32
                        sum multiplied by c_j / c_{j+1} between slots and by the last c
                        at the end.

Both must meet the stated tolerance |err| <= 8e-3 |ref| + 1e-4 on an input where folding
c into a single bf16 plane does not, and stay within the bound the GPU tests use."""
import numpy as np
import torch

from helpers import BF16_ATOL, BF16_RTOL, kernel_error_bound, oracle_selection, gapped_router, to64
from oracle import adafuse as O
from weight_merge_amd import synth


def bf16(x) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def emulate(W, Aw, Bw, slots, form):
    """bf16 merge of (expert, gate, signed scale) slots under one coefficient form."""
    W64, A64, B64 = to64(W), to64(Aw), to64(Bw)
    act = [(e, np.float32(sc) * np.float32(g)) for e, g, sc in slots if np.float32(sc) * np.float32(g) != 0]
    if form == "scaled":
        act.sort(key=lambda t: abs(float(t[1])))
        acc = np.zeros_like(W64)
        for j, (e, c) in enumerate(act):
            if j:
                acc = f32(acc * f32(np.float32(act[j - 1][1]) / np.float32(c)))
            acc = f32(acc + B64[e] @ A64[e])  # exact bf16 products, fp32 sum (one rounding per slot here)
        delta = f32(acc * float(act[-1][1])) if act else acc
    else:
        delta = np.zeros_like(W64)
        for e, c in act:
            x = f32(B64[e] * float(c))
            hi = bf16(x)
            b = hi if form == "single" else hi + bf16(f32(B64[e] * float(c) - hi))
            delta = f32(delta + b @ A64[e])
    return bf16(W64 + delta)


def cancelling_case():
    # d_in = 16 makes A ~ N(0, 1/4): the delta's terms reach the weights' size
    E, r, k, d_out, d_in = 3, 64, 2, 8, 16
    W, Aw, Bw = synth.adapter_bank(7, E, r, d_out, d_in, "bf16")
    h, R, _ = gapped_router(E, 64, "bf16", 3)
    idx, gate = oracle_selection(h, R, k)
    slots = [(e, g, 2.0) for e, g in zip(idx.tolist(), gate.tolist())]
    ref = O.merge(to64(W), to64(Aw), to64(Bw), idx.numpy(), gate.numpy().astype(np.float64), 2.0)
    return W, Aw, Bw, slots, ref


def ratio(got, ref):
    return float(np.max(np.abs(got - ref) / (BF16_RTOL * np.abs(ref) + BF16_ATOL)))


def test_single_plane_fold_misses_the_stated_tolerance_on_cancelling_weights():
    W, Aw, Bw, slots, ref = cancelling_case()
    assert ratio(emulate(W, Aw, Bw, slots, "single"), ref) > 1.0


def test_split_fold_and_scaled_accumulators_meet_it():
    W, Aw, Bw, slots, ref = cancelling_case()
    for form in ("split", "scaled"):
        got = emulate(W, Aw, Bw, slots, form)
        assert ratio(got, ref) < 0.6, form  # what is left is the final bf16 rounding
        assert np.all(np.abs(got - ref) <= kernel_error_bound(W, Aw, Bw, slots, ref)), form


def test_forms_agree_with_the_oracle_on_switches_and_many_slots():
    E, r, d_out, d_in = 16, 64, 24, 40
    W, Aw, Bw = synth.adapter_bank(11, E, r, d_out, d_in, "bf16")
    slots = [(3, 0.4, -2.0), (9, 0.6, -2.0), (1, 0.05, 2.0), (14, 0.15, 2.0), (9, 0.3, 2.0), (2, 0.5, 2.0)]
    ref = to64(W).copy()
    for e, g, sc in slots:
        ref += float(np.float32(sc) * np.float32(g)) * to64(Bw)[e] @ to64(Aw)[e]
    for form in ("split", "scaled"):
        got = emulate(W, Aw, Bw, slots, form)
        assert np.all(np.abs(got - ref) <= BF16_RTOL * np.abs(ref) + BF16_ATOL), form
        assert np.all(np.abs(got - ref) <= kernel_error_bound(W, Aw, Bw, slots, ref)), form


def test_scaled_accumulators_survive_extreme_gate_ratios():
    # gates 1 and 1e-39 (an fp32 subnormal): in increasing order the ratio is tiny, never
    # huge, so nothing overflows and the tiny slot simply vanishes below the tolerance
    W, Aw, Bw = synth.adapter_bank(13, 4, 64, 16, 32, "bf16")
    slots = [(0, 1.0, 2.0), (2, 1e-39, 2.0)]
    got = emulate(W, Aw, Bw, slots, "scaled")
    ref = to64(W) + 2.0 * to64(Bw)[0] @ to64(Aw)[0]
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - ref) <= BF16_RTOL * np.abs(ref) + BF16_ATOL)


def test_unit_coefficient_split_has_an_empty_lo_plane():
    # c = 1: c b is already bf16, so lo is zero and the split fold is the exact merge
    Bw = synth.adapter_bank(3, 4, 8, 24, 40, "bf16")[2]
    b = to64(Bw)
    hi = bf16(f32(b * 1.0))
    assert np.array_equal(hi, b)
    assert np.all(bf16(f32(b - hi)) == 0)
